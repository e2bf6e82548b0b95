// Index Branch projections: the G index query heads (one per GQA group) and
// the one shared index key head are linear maps of the hidden states
// [yhxrc, 二: one scoring head per group plus one shared key head; yifor,
// 工程實踐啟示: two added projection matrices]:
//   q_idx[t, g, :] = W_qi[g] x[t],   k_idx[row(t), :] = W_ki x[t]
// computed as one GEMM of x [n, d_model] against the stacked weights
// [64 (G+1), d_model], so x is read once for both. The key head is written
// straight into its cache row (row(t) = t, or ctx_lens[t]-1 of sequence t in
// decode). fp32 accumulation; outputs rounded to bf16 (nearest even).
//
// Many tokens with d_model a multiple of 256 (k_index_project_ws, below):
// four loader waves keep the next double steps of x and the weights in
// flight in registers and feed a two-slot LDS ring; four compute waves hold
// 128 tokens x NC/4 of the columns each. Otherwise (k_index_project):
// workgroup of 128 tokens x NC 64-column units (all G+1 units when G+1 <= 5,
// else two parts), 8 waves as 2 (tokens) x 4 (columns); each wave holds
// 4 x NC accumulator tiles of 16 x 16 (NC = 1 for few tokens: more
// workgroups, each with one 64-column unit). d_model is consumed in 32-wide slices
// staged in a ring of four LDS buffers (three slices in flight while one is
// computed) by direct-to-LDS loads with an XOR swizzle
// of the 16-byte chunks, so the MFMA operand reads are conflict-free. The
// MFMA computes (W x^T) tiles: each lane ends with 4 consecutive output
// columns of one token, stored as 8 bytes. Small batches (decode) split
// d_model across workgroups; the fp32 partials are then summed in a fixed
// order by a second kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

namespace {

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kPRows = 128;  // tokens per workgroup
constexpr int kPK = 32;      // d_model slice per stage (one MFMA k-step)
constexpr int kRing = 4;     // LDS stages: three loads in flight behind the one computed
constexpr int kXBytes = kPRows * kPK * 2;

// Number of 64-slot load rounds of a wave for NROWS rows of 4 chunks.
template <int NROWS>
__device__ __forceinline__ int wave_loads(int wave) {
  int n = 0;
#pragma unroll
  for (int it = 0; it < (NROWS * 4 + 511) / 512; ++it) n += (it * 512 + wave * 64 < NROWS * 4) ? 1 : 0;
  return n;
}

// Stages 32-element slices of NROWS rows into LDS rows of 64 bytes; LDS chunk
// p of row r holds global chunk p ^ ((r >> 1) & 3) (rows 0, 2, 4, 6 of a
// 16-row operand read then fall in distinct banks). row_ptr(r) gives row r's
// first element at the slice.
template <int NROWS, typename RowPtr>
__device__ __forceinline__ void stage_rows(lds_char* dst, RowPtr row_ptr, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int it = 0; it < (NROWS * 4 + 511) / 512; ++it) {
    const int s0 = it * 512 + wave * 64;
    if (s0 < NROWS * 4) {
      const int slot = s0 + lane;
      const int r = slot >> 2, p = slot & 3;
      lds_dma16(row_ptr(r) + ((p ^ ((r >> 1) & 3)) << 3), dst + s0 * 16);
    }
  }
}

// f(integral_constant<int, I>) for I = B .. E-1, in order.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// MFMA operand of row r (LDS), k-chunk j (8 elements at 8j of the slice).
__device__ __forceinline__ bf16x8 lds_chunk(const lds_char* base, int r, int j) {
  const u32x4 v = *(const lds_u32x4*)(base + r * 64 + ((j ^ ((r >> 1) & 3)) << 4));
  return as_bf16x8(v);
}

}  // namespace

template <int NC>
__global__ __launch_bounds__(512, 1) void k_index_project(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_qi, const uint16_t* __restrict__ w_ki,
    int64_t n, int d_model, int G, int stages_per_split, uint16_t* __restrict__ q_idx,
    uint16_t* __restrict__ k_idx, const int32_t* __restrict__ ctx_lens, int64_t max_ctx,
    float* __restrict__ part) {
  constexpr int kWRows = NC * 64;
  constexpr int kStage = kXBytes + kWRows * 64;
  __shared__ __attribute__((aligned(1024))) char lds_raw[kRing * kStage];
  lds_char* lds = (lds_char*)lds_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, qd = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)blockIdx.x * kPRows;
  const int col0 = (int)blockIdx.y * kWRows;  // first stacked weight row of this part
  const int ncols = 64 * (G + 1);
  const int nk = d_model / kPK;
  const int st0 = (int)blockIdx.z * stages_per_split;
  const int st1 = min(nk, st0 + stages_per_split);

  // rows past the tokens or past the stacked weights repeat a valid row; their
  // results are never stored
  auto x_row = [&](int r) { return x + min<int64_t>(m0 + r, n - 1) * d_model; };
  auto w_row = [&](int r) {
    const int gc = min(col0 + r, ncols - 1);
    return gc < 64 * G ? w_qi + (int64_t)gc * d_model : w_ki + (int64_t)(gc - 64 * G) * d_model;
  };
  auto load_stage = [&](int st) {
    lds_char* dst = lds + ((st - st0) % kRing) * kStage;
    const int k0 = st * kPK;
    stage_rows<kPRows>(dst, [&](int r) { return x_row(r) + k0; }, tid);
    stage_rows<kWRows>(dst + kXBytes, [&](int r) { return w_row(r) + k0; }, tid);
  };
  const int per_stage = wave_loads<kPRows>(wave) + wave_loads<kWRows>(wave);  // this wave's loads per stage

  f32x4 acc[4][NC];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) acc[rt][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int st = st0; st < min(st1, st0 + kRing - 1); ++st) load_stage(st);
  for (int st = st0; st < st1; ++st) {
    // stage st has landed once at most the later stages' loads are pending
    wait_vmcnt_upto(min(kRing - 2, st1 - 1 - st) * per_stage);
    __syncthreads();  // every wave's part of stage st is in LDS; stage st-1's buffer is free
    if (st + kRing - 1 < st1) load_stage(st + kRing - 1);
    const lds_char* xs = lds + ((st - st0) % kRing) * kStage;
    const lds_char* ws = xs + kXBytes;
    bf16x8 xb[4], wa[NC];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) xb[rt] = lds_chunk(xs, wm * 64 + rt * 16 + c, qd);
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) wa[ct] = lds_chunk(ws, wn * NC * 16 + ct * 16 + c, qd);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) acc[rt][ct] = mfma16x16x32(wa[ct], xb[rt], acc[rt][ct]);
  }

  // lane (c, qd) of tile (rt, ct) holds token m0 + wm*64 + rt*16 + c, stacked
  // columns col0 + wn*NC*16 + ct*16 + 4qd .. +3
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int64_t t = m0 + wm * 64 + rt * 16 + c;
    if (t >= n) continue;
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      const int gc = col0 + wn * NC * 16 + ct * 16 + 4 * qd;
      if (gc >= ncols) continue;
      const f32x4 v = acc[rt][ct];
      if (part) {
        *reinterpret_cast<f32x4*>(part + ((int64_t)blockIdx.z * n + t) * ncols + gc) = v;
        continue;
      }
      const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      uint16_t* dst;
      if (gc < 64 * G) {
        dst = q_idx + t * (int64_t)(64 * G) + gc;
      } else {
        const int64_t row = ctx_lens ? t * max_ctx + ctx_lens[t] - 1 : t;
        dst = k_idx + row * 64 + (gc - 64 * G);
      }
      *reinterpret_cast<u32x2*>(dst) = o;
    }
  }
}

// Many tokens, d_model a multiple of 64 kWsDepth: 128 tokens x NCT 64-column
// units per workgroup, eight waves in two roles. Waves 4-7 load: each keeps
// its quarter of the next kWsDepth double steps (64 of d_model each: x 128
// rows and the weights 64 NCT rows of 128 bytes, every row read as one
// 128-byte piece) in flight in registers and, one double step ahead of the
// computation, writes a double step into a two-slot LDS ring. Waves 0-3
// compute: wave w holds all 128 tokens against column tiles [w NCT, (w+1) NCT)
// of 16 (8 NCT accumulator tiles) and reads its operands from the ring. One
// barrier per double step separates the slot being read from the slot being
// written. All loads are ordinary register loads, so the compiler's waits are
// exact: each loader wave consumes its loads in the order it issued them,
// with kWsDepth - 1 double steps still in flight (about 170 KiB per CU). In a
// slot, row r's 16-byte chunk p sits at chunk p ^ f(r), f(r) = (r & 7) ^
// ((r >> 3) & 1): the operand reads (16 consecutive rows, one chunk each) and
// the row writes are then free of bank conflicts for 32 and for 64 banks.
constexpr int kWsDepth = 4;
constexpr int kWsStep = 64;                  // d_model per double step
constexpr int kWsXBytes = kPRows * kWsStep * 2;
constexpr int kWsX = kPRows * 8 / 256;       // 16-byte x chunks per loader lane and double step

__device__ __forceinline__ int ws_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int NCT>
__global__ __launch_bounds__(512, 1) void k_index_project_ws(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_qi, const uint16_t* __restrict__ w_ki,
    int64_t n, int d_model, int G, uint16_t* __restrict__ q_idx, uint16_t* __restrict__ k_idx,
    const int32_t* __restrict__ ctx_lens, int64_t max_ctx) {
  constexpr int kWRows = NCT * 64;           // weight rows per workgroup
  constexpr int kWsW = kWRows * 8 / 256;     // 16-byte weight chunks per loader lane and double step
  constexpr int kSlot = kWsXBytes + kWRows * kWsStep * 2;
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kSlot];
  lds_char* lds = (lds_char*)lds_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t m0 = (int64_t)blockIdx.x * kPRows;
  const int col0 = (int)blockIdx.y * kWRows;
  const int ncols = 64 * (G + 1);
  const int nk = d_model / kWsStep;

  if (wave >= 4) {
    // loader: chunk q = 256 i + lt (lt = tid - 256) of a part is row
    // 32 i + lt / 8, chunk lt % 8 (8 elements at 8 (lt % 8) of the double
    // step). Weight part i lies in unit (col0 + 32 i) / 64 (col0 is a
    // multiple of 64), rows 32 (i % 2) + lt / 8 of it; units past the last
    // repeat it (never stored).
    const int lt = tid - 256, lr = lt >> 3, lp = lt & 7;
    const uint32_t dst0 = (uint32_t)(lr * 128 + ((lp ^ ws_swz(lr)) << 4));
    const char* xbase = (const char*)(x + m0 * d_model);
    uint32_t xo[kWsX];
#pragma unroll
    for (int i = 0; i < kWsX; ++i)
      xo[i] = (uint32_t)(((min<int64_t>(m0 + 32 * i + lr, n - 1) - m0) * d_model + 8 * lp) * 2);
    const char* wb[kWsW];
#pragma unroll
    for (int i = 0; i < kWsW; ++i) {
      const int u = min(col0 / 64 + i / 2, G);
      wb[i] = (const char*)((u < G ? w_qi + (int64_t)u * 64 * d_model : w_ki) + (int64_t)(32 * (i & 1)) * d_model);
    }
    const uint32_t wo = (uint32_t)((lr * d_model + 8 * lp) * 2);
    u32x4 ring[kWsDepth][kWsX + kWsW];
    // double step s (clamped to the last: steps past the end load valid data
    // that is never read)
    auto load_step = [&](int s, u32x4 (&dst)[kWsX + kWsW]) {
      const uint32_t kb = (uint32_t)(min(s, nk - 1) * kWsStep * 2);
#pragma unroll
      for (int i = 0; i < kWsX; ++i) dst[i] = ld16(xbase + xo[i] + kb);
#pragma unroll
      for (int i = 0; i < kWsW; ++i) dst[kWsX + i] = ld16(wb[i] + wo + kb);
    };
    // row 32 i + lr has the swizzle of lr (32 i changes neither r & 7 nor
    // (r >> 3) & 1)
    auto write_step = [&](int s, const u32x4 (&src)[kWsX + kWsW]) {
      lds_char* slot = lds + (s & 1) * kSlot + dst0;
#pragma unroll
      for (int i = 0; i < kWsX; ++i) *(lds_u32x4*)(slot + 4096 * i) = src[i];
#pragma unroll
      for (int i = 0; i < kWsW; ++i) *(lds_u32x4*)(slot + kWsXBytes + 4096 * i) = src[kWsX + i];
    };
    static_for<0, kWsDepth>([&](auto is) {
      constexpr int s = decltype(is)::value;
      load_step(s, ring[s]);
    });
    write_step(0, ring[0]);
    load_step(kWsDepth, ring[0]);
    wait_lgkmcnt0();
    __syncthreads();  // double step 0 is in slot 0
    // iteration g (the computation of double step g runs meanwhile): double
    // step g+1 into slot (g+1) & 1, then its registers take g+1+kWsDepth
    for (int g0 = 0; g0 < nk; g0 += kWsDepth) {
      static_for<0, kWsDepth>([&](auto ij) {
        constexpr int j = decltype(ij)::value, rs = (j + 1) % kWsDepth;
        const int g = g0 + j;
        write_step(g + 1, ring[rs]);
        load_step(g + 1 + kWsDepth, ring[rs]);
        wait_lgkmcnt0();
        __syncthreads();  // double step g+1 is in its slot; g's slot is free
      });
    }
    return;
  }

  // compute: lane (c, qd) reads row 16t + c (x) or 16 (w NCT + ct) + c
  // (weights), logical chunk 4h + qd for half h of the double step
  const int c = lane & 15, qd = lane >> 4, sw = ws_swz(c);
  f32x4 acc[8][NCT];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[t][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
  auto frag = [&](const lds_char* base, int row, int h) {
    const u32x4 v = *(const lds_u32x4*)(base + row * 128 + (((4 * h + qd) ^ sw) << 4));
    return as_bf16x8(v);
  };
  __syncthreads();  // double step 0 is in slot 0
  for (int g = 0; g < nk; ++g) {
    const lds_char* xs = lds + (g & 1) * kSlot;
    const lds_char* wsl = xs + kWsXBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 wa[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) wa[ct] = frag(wsl, 16 * (wave * NCT + ct) + c, h);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 xb = frag(xs, 16 * t + c, h);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[t][ct] = mfma16x16x32(wa[ct], xb, acc[t][ct]);
      }
    }
    __syncthreads();  // this slot is read; the next double step is in the other
  }

  // lane (c, qd) of tile (t, ct): token m0 + 16t + c, stacked columns
  // col0 + 16 (wave NCT + ct) + 4qd .. +3
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int64_t tok = m0 + 16 * t + c;
    if (tok >= n) continue;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int tc0 = col0 + 16 * (wave * NCT + ct);
      if (tc0 >= ncols) continue;
      const int gc = tc0 + 4 * qd;
      const f32x4 v = acc[t][ct];
      const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      uint16_t* dst;
      if (gc < 64 * G) {
        dst = q_idx + tok * (int64_t)(64 * G) + gc;
      } else {
        const int64_t row = ctx_lens ? tok * max_ctx + ctx_lens[tok] - 1 : tok;
        dst = k_idx + row * 64 + (gc - 64 * G);
      }
      *reinterpret_cast<u32x2*>(dst) = o;
    }
  }
}

// Sum of the d_model splits' partials in split order, rounded to bf16.
__global__ __launch_bounds__(256) void k_index_project_reduce(const float* __restrict__ part, int64_t n, int G,
                                                              int splits, uint16_t* __restrict__ q_idx,
                                                              uint16_t* __restrict__ k_idx,
                                                              const int32_t* __restrict__ ctx_lens, int64_t max_ctx) {
  const int ncols = 64 * (G + 1);
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one 4-column group
  if (e >= n * (ncols / 4)) return;
  const int64_t t = e / (ncols / 4);
  const int gc = (int)(e % (ncols / 4)) * 4;
  const float* src = part + t * ncols + gc;
  const int64_t zstride = n * ncols;
  f32x4 s = *reinterpret_cast<const f32x4*>(src);
  // eight partials in flight at a time, added in split order
  for (int z0 = 1; z0 < splits; z0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (z0 + u < splits) v[u] = *reinterpret_cast<const f32x4*>(src + (int64_t)(z0 + u) * zstride);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (z0 + u < splits) {
        s[0] += v[u][0];
        s[1] += v[u][1];
        s[2] += v[u][2];
        s[3] += v[u][3];
      }
  }
  const u32x2 o = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  uint16_t* dst;
  if (gc < 64 * G) {
    dst = q_idx + t * (int64_t)(64 * G) + gc;
  } else {
    const int64_t row = ctx_lens ? t * max_ctx + ctx_lens[t] - 1 : t;
    dst = k_idx + row * 64 + (gc - 64 * G);
  }
  *reinterpret_cast<u32x2*>(dst) = o;
}

ProjectPlan plan_index_project(int64_t n, int d_model, int G) {
  ProjectPlan pl;
  const int units = G + 1;
  pl.m_tiles = (n + kPRows - 1) / kPRows;
  if (pl.m_tiles * ((units + 4) / 5) >= 64) {
    // many tokens: each workgroup takes all (or half) of the columns, so x is
    // read once (or twice)
    pl.parts = units <= 5 ? 1 : 2;
    pl.nc = (units + pl.parts - 1) / pl.parts;
    // whole multiples of kWsDepth steps: the warp-specialised kernel
    pl.ws = d_model % (kWsStep * kWsDepth) == 0;
  } else {
    // few tokens (decode): one 64-column unit per workgroup, d_model split
    pl.parts = units;
    pl.nc = 1;
  }
  const int nk = d_model / kPK;
  const int64_t base = pl.m_tiles * pl.parts;
  // about two workgroups per CU; each split at least four slices deep, and the
  // fp32 partials (splits x n x columns) kept below half the weights' bytes
  int64_t splits = 1;
  if (base < 256 && !pl.ws)
    splits = std::max<int64_t>(1, std::min<int64_t>({(512 + base - 1) / base, nk / 4, d_model / (4 * n)}));
  pl.stages_per_split = (int)((nk + splits - 1) / splits);
  pl.splits = (nk + pl.stages_per_split - 1) / pl.stages_per_split;
  pl.part_floats = pl.splits > 1 ? (size_t)pl.splits * n * 64 * units : 0;
  return pl;
}

template <int NC>
static void launch_nc(const LaunchProject& a, const ProjectPlan& pl, hipStream_t st) {
  float* part = pl.splits > 1 ? a.part : nullptr;
  hipLaunchKernelGGL(k_index_project<NC>, dim3((unsigned)pl.m_tiles, pl.parts, pl.splits), dim3(512), 0, st, a.x,
                     a.w_qi, a.w_ki, a.n, a.d_model, a.G, pl.stages_per_split, a.q_idx, a.k_idx, a.ctx_lens,
                     a.max_ctx, part);
}

template <int NCT>
static void launch_ws(const LaunchProject& a, const ProjectPlan& pl, hipStream_t st) {
  hipLaunchKernelGGL(k_index_project_ws<NCT>, dim3((unsigned)pl.m_tiles, pl.parts), dim3(512), 0, st, a.x, a.w_qi,
                     a.w_ki, a.n, a.d_model, a.G, a.q_idx, a.k_idx, a.ctx_lens, a.max_ctx);
}

void launch_index_project(const LaunchProject& a, hipStream_t st) {
  const ProjectPlan pl = plan_index_project(a.n, a.d_model, a.G);
  if (pl.ws) {
    switch (pl.nc) {
      case 1: launch_ws<1>(a, pl, st); break;
      case 2: launch_ws<2>(a, pl, st); break;
      case 3: launch_ws<3>(a, pl, st); break;
      case 4: launch_ws<4>(a, pl, st); break;
      case 5: launch_ws<5>(a, pl, st); break;
      default: break;
    }
    return;
  }
  switch (pl.nc) {
    case 1: launch_nc<1>(a, pl, st); break;
    case 2: launch_nc<2>(a, pl, st); break;
    case 3: launch_nc<3>(a, pl, st); break;
    case 4: launch_nc<4>(a, pl, st); break;
    case 5: launch_nc<5>(a, pl, st); break;
    default: return;
  }
  if (pl.splits > 1) {
    const int64_t groups = a.n * 16 * (a.G + 1);
    hipLaunchKernelGGL(k_index_project_reduce, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st, a.part,
                       a.n, a.G, pl.splits, a.q_idx, a.k_idx, a.ctx_lens, a.max_ctx);
  }
}

}  // namespace msa
