// Index Branch scoring with block max-pooling on gfx950 MFMA.
//
// For a query row i of group g and an older key block b, the pooled score is
//   S[i, g, b] = max over the B_k keys j of block b of q_idx[i, g, :] . k_idx[j, :]
// (raw dot products, no scale and no exponential: ranking raw scores selects the
// same blocks as ranking their softmax [pnsm, section 7; yhxrc, 二], and block
// scores are max-pooled [yifor, 設計核心]). The local block is always selected,
// so it is never scored: with query tiles aligned to B_k the causal mask is the
// loop bound b < b_loc and no per-token mask is needed.
//
// Contraction on MFMA: S^T tile (16 keys x 16 rows) = K (16 x 32 dims) * Q^T
// (32 dims x 16 rows), two steps over d_idx = 64. Each lane then holds four keys
// of one row, so the pooling max is three in-lane maxima per tile plus two
// cross-lane lane-swap steps per block.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// One workgroup (4 waves) per (query block qb, chunk of key blocks); it
// covers the 128*G index rows (i, g) of the query block, 32*G per wave. Each
// 16 KiB key block is loaded once per workgroup straight into LDS
// (global_load_lds, double-buffered) and read as MFMA operands by all waves.
// LDS layout: 128 rows of 128 B; 16-byte chunk x of row r sits at chunk
// position x ^ ((r >> 1) & 7), which keeps the operand reads conflict-free.
// Key blocks per workgroup (NSTG 128-key stages at B_k = 128, one stage
// otherwise): short workgroups spread the causal triangle's uneven work over
// the chip when there are few query blocks (at 32K, chunks of 4 and 8 blocks
// measured 1.05x and 1.3x slower than 2); long sequences have work for
// millions of workgroups, and longer chunks load each workgroup's 64 KiB of
// index queries once for more key blocks.
//
// Workgroups form a 1-D grid over the causal triangle only: query block q
// holds st(q) = q (+1 when B_k < 128: its own stage) stages, cut into
// ceil(st(q) / NS) chunks, and workgroup w finds its (q, chunk) from the
// closed-form count of the chunks before q.
__host__ __device__ __forceinline__ int64_t chunks_before(int64_t x, int ns) {
  // sum over q < x of ceil(q / ns)
  const int64_t a = x / ns, r = x % ns;
  int64_t s = ns * a * (a - 1) / 2 + a * (ns - 1);
  if (r > 0) s += a + (r - 1) * (a + 1);
  return s;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Stages key rows 0..127 of a 128-key stage; rows >= nvalid repeat row
// nvalid-1 (they only feed blocks no query row reads).
__device__ __forceinline__ void stage_kidx(lds_char* dst, const uint16_t* src_rows, int wave, int nvalid) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int s0 = (it * 4 + wave) * 64;
    const int slot = s0 + lane;
    const int r = slot >> 3, p = slot & 7;
    const int x = p ^ ((r >> 1) & 7);
    lds_dma16(src_rows + min(r, nvalid - 1) * kIndexDim + x * 8, dst + s0 * 16);
  }
}

// SUB = 128 / B_k blocks per 128-key stage (1, 2 or 4): each stage yields SUB
// pooled scores per row, from its key tiles s*8/SUB .. (s+1)*8/SUB - 1. With
// SUB > 1 a query block's own stage also holds blocks older than some of its
// rows, so it is scored too; every row writes only its blocks b < b_loc.
template <int G, int SUB, int NSTG>
__global__ __launch_bounds__(256, 2) void k_index_prefill(const uint16_t* __restrict__ q_idx,
                                                          const uint16_t* __restrict__ k_idx,
                                                          float* __restrict__ sblk, int64_t row0,
                                                          int64_t row_end, int qb_begin, int qb_end, int nb) {
  constexpr int RT = 2 * G;        // 16-row tiles per wave
  constexpr int NS = SUB == 1 ? NSTG : 1;  // 128-key stages per chunk
  constexpr int KC = NS * SUB;             // blocks per chunk
  constexpr int TPB = 8 / SUB;     // key tiles per block
  constexpr int BKS = kBlock / SUB;
  constexpr int ADD = SUB > 1 ? 1 : 0;     // st(q) = q + ADD
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * 16384];
  lds_char* lds = (lds_char*)lds_raw;
  // (query block, chunk) of this workgroup: the largest qb with
  // chunks_before(qb + ADD) - chunks_before(qb_begin + ADD) <= w
  const int64_t w = (int64_t)blockIdx.x;
  const int64_t base = chunks_before(qb_begin + ADD, NS);
  int lo = qb_begin, hi = qb_end - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunks_before(mid + ADD, NS) - base <= w) lo = mid; else hi = mid - 1;
  }
  const int qb = __builtin_amdgcn_readfirstlane(lo);
  const int chunk = (int)__builtin_amdgcn_readfirstlane((int)(w - (chunks_before(qb + ADD, NS) - base)));
  const int last = SUB > 1 ? qb : qb - 1;  // last stage holding a block older than some row
  const int kb0 = chunk * NS;
  if (kb0 > last) return;
  const int kb1 = min(kb0 + NS, last + 1);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, qd = lane >> 4;
  auto stage_rows = [&](int kb) { return (int)min<int64_t>(kBlock, row_end - (int64_t)kb * kBlock); };

  stage_kidx(lds, k_idx + (int64_t)kb0 * kBlock * kIndexDim, wave, stage_rows(kb0));

  // flat index row (i*G + g) of this wave's first row; the window's rows are
  // [row0, row_end) (a query block can start before or end after them)
  const int64_t flat0 = (int64_t)qb * kBlock * G + (int64_t)wave * 32 * G;
  const int64_t flat_lo = row0 * G, flat_end = row_end * G;
  bf16x8 qop[RT][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t row = flat0 + rt * 16 + c;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row >= flat_lo && row < flat_end) v = ld16(q_idx + (row - flat_lo) * kIndexDim + 32 * s + 8 * qd);
      qop[rt][s] = as_bf16x8(v);
    }
  }

  // pooled scores of the chunk: lane group qd keeps the rows of tiles rt = qd
  // (mod 4), KC blocks each, and writes them as one run per row
  float res[(RT + 3) / 4][KC];
#pragma unroll
  for (int j = 0; j < (RT + 3) / 4; ++j)
#pragma unroll
    for (int x = 0; x < KC; ++x) res[j][x] = -__builtin_inff();

  // fully unrolled over the chunk's stages, so every pooled maximum lands in
  // a fixed register (the block position is a constant)
#pragma unroll
  for (int x = 0; x < NS; ++x) {
    const int kb = kb0 + x;
    if (kb >= kb1) break;
    wait_vmcnt0();
    __syncthreads();  // stage kb staged; the other buffer is free
    if (kb + 1 < kb1)
      stage_kidx(lds + ((x + 1) & 1) * 16384, k_idx + (int64_t)(kb + 1) * kBlock * kIndexDim, wave,
                 stage_rows(kb + 1));
    const lds_char* st = lds + (x & 1) * 16384;
    // issue priority up through the stage's MFMAs and down for the pooling
    // and the writes: the other workgroups' waves on the SIMD, at other
    // points of their own stages, fill the slots left meanwhile (1M: index
    // scoring 2 % faster; 32K unchanged)
    __builtin_amdgcn_s_setprio(1);
    float mx[SUB][RT];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int sb = t / TPB;
      const int r = 16 * t + c;
      const int sw = (c >> 1) & 7;
      const u32x4 v0 = *(const lds_u32x4*)(st + r * 128 + ((qd ^ sw) << 4));
      const u32x4 v1 = *(const lds_u32x4*)(st + r * 128 + (((4 + qd) ^ sw) << 4));
      const bf16x8 a0 = as_bf16x8(v0), a1 = as_bf16x8(v1);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma16x16x32(a0, qop[rt][0], acc);
        acc = mfma16x16x32(a1, qop[rt][1], acc);
        float m = t % TPB == 0 ? fmaxf(acc[0], acc[1]) : fmaxf(fmaxf(mx[sb][rt], acc[0]), acc[1]);
        mx[sb][rt] = fmaxf(fmaxf(m, acc[2]), acc[3]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) mx[sb][rt] = max_lane_groups(mx[sb][rt]);
    // all four lane groups now hold the block maxima; group qd keeps tiles rt = qd mod 4
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
      for (int j = 0; j < (RT + 3) / 4; ++j) {
        float v = mx[sb][4 * j];
#pragma unroll
        for (int u = 1; u < 4; ++u)
          if (4 * j + u < RT) v = qd == u ? mx[sb][4 * j + u] : v;
        res[j][x * SUB + sb] = v;
      }
  }
  const int nkb = (kb1 - kb0) * SUB;  // blocks of the chunk
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t row = flat0 + rt * 16 + c;
    if ((rt & 3) != qd || row < flat_lo || row >= flat_end) continue;
    // blocks the row reads: b < b_loc
    const int nout = SUB == 1 ? nkb : max(0, min(nkb, (int)((row / G) / BKS) - kb0 * SUB));
    float* dst = sblk + (row - flat_lo) * nb + kb0 * SUB;
    const float* rv = res[rt >> 2];
    if (nout == KC && (reinterpret_cast<uintptr_t>(dst) & (4 * KC - 1)) == 0) {
      if constexpr (KC == 2) {
        *reinterpret_cast<f32x2*>(dst) = (f32x2){rv[0], rv[1]};
      } else {
#pragma unroll
        for (int v4 = 0; v4 < KC / 4; ++v4)
          *reinterpret_cast<f32x4*>(dst + 4 * v4) = (f32x4){rv[4 * v4], rv[4 * v4 + 1], rv[4 * v4 + 2], rv[4 * v4 + 3]};
      }
    } else {
#pragma unroll
      for (int xx = 0; xx < KC; ++xx)
        if (xx < nout) dst[xx] = rv[xx];
    }
  }
}

// Decode: one row per (sequence, group); one workgroup per (sequence, chunk of
// kDecKB key blocks), each wave scoring whole key blocks. The shared index key
// cache is streamed once (the two half-row loads of a key row hit the same L2
// line); lanes c < G of the MFMA column dimension carry the G index query heads.
constexpr int kDecKB = 8;

template <int G, int SUB>
__global__ __launch_bounds__(256) void k_index_decode(const uint16_t* __restrict__ q_idx,
                                                      const uint16_t* __restrict__ k_idx,
                                                      const int32_t* __restrict__ ctx_lens,
                                                      float* __restrict__ sblk, int64_t max_ctx,
                                                      int nb, int topk) {
  constexpr int TPB = 8 / SUB;  // key tiles per block
  constexpr int BKS = kBlock / SUB;
  const int sq = (int)blockIdx.y;
  const int L = ctx_lens[sq];
  const int b_loc = (L - 1) / BKS;
  if (b_loc < topk) return;  // every older block is selected; no scores needed
  const int kb0 = (int)blockIdx.x * kDecKB;
  const int nst = (b_loc + SUB - 1) / SUB;  // 128-key stages holding an older block
  if (kb0 >= nst) return;
  const int kb1 = min(kb0 + kDecKB, nst);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, qd = lane >> 4;

  bf16x8 qop[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < G) v = ld16(q_idx + ((int64_t)sq * G + c) * kIndexDim + 32 * s + 8 * qd);
    qop[s] = as_bf16x8(v);
  }
  const uint16_t* kbase = k_idx + (int64_t)sq * max_ctx * kIndexDim;

  // two stages per iteration: all 32 loads are issued before the first MFMA
  for (int kb = kb0 + wave; kb < kb1; kb += 8) {
    const int kb2 = kb + 4;
    const bool two = kb2 < kb1;
    u32x4 a[2][8][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int blk = h ? (two ? kb2 : kb) : kb;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        // rows past the context feed only blocks >= b_loc (SUB > 1)
        const int64_t key = min<int64_t>((int64_t)blk * kBlock + 16 * t + c, L - 1);
        const uint16_t* krow = kbase + key * kIndexDim + 8 * qd;
        a[h][t][0] = ld16(krow);
        a[h][t][1] = ld16(krow + 32);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float mx[SUB];
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb) mx[sb] = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma16x16x32(as_bf16x8(a[h][t][0]), qop[0], acc);
        acc = mfma16x16x32(as_bf16x8(a[h][t][1]), qop[1], acc);
        mx[t / TPB] = fmaxf(mx[t / TPB], fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
      }
      const int blk = h ? kb2 : kb;
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb) {
        const float m = max_lane_groups(mx[sb]);
        const int b = blk * SUB + sb;
        if (qd == 0 && c < G && (h == 0 || two) && b < b_loc) sblk[((int64_t)sq * G + c) * nb + b] = m;
      }
    }
  }
}

template <int G, int SUB, int NSTG>
static void launch_prefill_ns(const LaunchIndexPrefill& a, hipStream_t st) {
  constexpr int NS = SUB == 1 ? NSTG : 1;
  constexpr int ADD = SUB > 1 ? 1 : 0;
  const int64_t wgs = chunks_before(a.qb_end + ADD, NS) - chunks_before(a.qb_begin + ADD, NS);
  if (wgs <= 0) return;
  hipLaunchKernelGGL((k_index_prefill<G, SUB, NSTG>), dim3((unsigned)wgs), dim3(256), 0, st, a.q_idx, a.k_idx,
                     a.sblk, a.row0, a.row_end, a.qb_begin, a.qb_end, a.nb);
}

// Chunk length: two stages for small calls (up to kFewChunks workgroups of
// two), else 8, or 16 beyond 8 * kManyChunks (32K prefill: 2, 4, 8 stages
// measured 0.238, 0.223, 0.213 ms).
constexpr int64_t kFewChunks = 1 << 12;
constexpr int64_t kManyChunks = 1 << 16;

template <int G, int SUB>
static void launch_prefill_g(const LaunchIndexPrefill& a, hipStream_t st) {
  if (a.qb_end <= a.qb_begin) return;
  if constexpr (SUB > 1) {
    launch_prefill_ns<G, SUB, 1>(a, st);
  } else {
    const int64_t w2 = chunks_before(a.qb_end, 2) - chunks_before(a.qb_begin, 2);
    if (w2 <= kFewChunks)
      launch_prefill_ns<G, SUB, 2>(a, st);
    else if (w2 <= 8 * kManyChunks)
      launch_prefill_ns<G, SUB, 8>(a, st);
    else
      launch_prefill_ns<G, SUB, 16>(a, st);
  }
}

template <int SUB>
static void launch_prefill_sub(const LaunchIndexPrefill& a, hipStream_t st) {
  switch (a.G) {
    case 1: launch_prefill_g<1, SUB>(a, st); break;
    case 2: launch_prefill_g<2, SUB>(a, st); break;
    case 3: launch_prefill_g<3, SUB>(a, st); break;
    case 4: launch_prefill_g<4, SUB>(a, st); break;
    case 5: launch_prefill_g<5, SUB>(a, st); break;
    case 6: launch_prefill_g<6, SUB>(a, st); break;
    case 7: launch_prefill_g<7, SUB>(a, st); break;
    case 8: launch_prefill_g<8, SUB>(a, st); break;
    default: break;
  }
}

void launch_index_prefill(const LaunchIndexPrefill& a, hipStream_t st) {
  switch (a.bk) {
    case 128: launch_prefill_sub<1>(a, st); break;
    case 64: launch_prefill_sub<2>(a, st); break;
    case 32: launch_prefill_sub<4>(a, st); break;
    default: break;
  }
}

template <int G, int SUB>
static void launch_decode_g(const LaunchIndexDecode& a, hipStream_t st) {
  const int stages = (int)((a.max_ctx + kBlock - 1) / kBlock);
  const int chunks = (stages + kDecKB - 1) / kDecKB;
  dim3 grid(chunks, a.batch);
  hipLaunchKernelGGL((k_index_decode<G, SUB>), grid, dim3(256), 0, st, a.q_idx, a.k_idx, a.ctx_lens, a.sblk,
                     a.max_ctx, a.nb, a.topk);
}

template <int SUB>
static void launch_decode_sub(const LaunchIndexDecode& a, hipStream_t st) {
  switch (a.G) {
    case 1: launch_decode_g<1, SUB>(a, st); break;
    case 2: launch_decode_g<2, SUB>(a, st); break;
    case 3: launch_decode_g<3, SUB>(a, st); break;
    case 4: launch_decode_g<4, SUB>(a, st); break;
    case 5: launch_decode_g<5, SUB>(a, st); break;
    case 6: launch_decode_g<6, SUB>(a, st); break;
    case 7: launch_decode_g<7, SUB>(a, st); break;
    case 8: launch_decode_g<8, SUB>(a, st); break;
    default: break;
  }
}

void launch_index_decode(const LaunchIndexDecode& a, hipStream_t st) {
  switch (a.bk) {
    case 128: launch_decode_sub<1>(a, st); break;
    case 64: launch_decode_sub<2>(a, st); break;
    case 32: launch_decode_sub<4>(a, st); break;
    default: break;
  }
}

}  // namespace msa
