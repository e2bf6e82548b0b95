// Main Branch: exact softmax attention restricted to the selected KV blocks,
// organised KV-outer ("outer gather Q") [pnsm, section 7; yhxrc, 二;
// yololab, "KV Outer Gather Q是什麼？"].
//
// Prefill: a persistent grid drains the tile queue built by the reverse index.
// A tile is (group g, KV block b, up to tile_q queries that selected b). The
// workgroup stages K_b row-major and V_b transposed in LDS once, then each wave
// gathers the 16 query heads of one query at a time (4 KiB, contiguous in the
// [N, Hq, d] layout) and computes, on MFMA,
//   S^T (128 keys x 16 heads) = K_b (128 x 128) . Q^T        (32 MFMA 16x16x32)
//   P^T = exp2(S^T * scale*log2e - m),  l = sum P, per head
//   O^T (128 d x 16 heads)   = V_b^T (128 x 128 keys) . P^T  (32 MFMA)
// The S^T orientation puts one head's scores in one lane column, so the softmax
// reductions are in-lane plus two cross-lane steps, and the P^T accumulator
// fragments feed the second contraction directly as its B operand (the key
// order inside a 32-key step is permuted identically in V^T's A operand).
// Output: one softmax partial per (query, head, selected slot): o/l rounded to
// bf16 and lse2 = m + log2(l); merged later by the combine pass (two-phase
// combine without atomics [pnsm, section 7]). Causal masking is needed only when
// b is the query's own block.
//
// Decode: one wave per (sequence, group, selected slot) with the same
// contraction on a single query.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int KS = 136;  // LDS row stride (bf16) of K_b  [128 keys][128 d]
constexpr int VS = 136;  // LDS row stride (bf16) of V_b^T [128 d][128 keys]

// Stage V rows (128 keys x 128 d, row stride rstride elements) transposed into
// Vt. `nthr` threads cooperate; thread `tid` handles key quads kq = tid%16 (+16
// per pass) and d-chunks dc = (tid/16) (+ nthr/16 per pass).
template <int NTHR>
__device__ __forceinline__ void stage_vt(uint16_t* Vt, const uint16_t* vrow0, int64_t rstride, int nvalid,
                                         int tid) {
  constexpr int DC_STEP = NTHR / 16;
#pragma unroll
  for (int pk = 0; pk < 2; ++pk) {
    const int kq = (tid & 15) + 16 * pk;
#pragma unroll
    for (int dc0 = 0; dc0 < 16; dc0 += DC_STEP) {
      const int dc = dc0 + (tid >> 4);
      u32x4 rows[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 4 * kq + rr;
        rows[rr] = (u32x4){0u, 0u, 0u, 0u};
        if (key < nvalid) rows[rr] = ld16(vrow0 + (int64_t)key * rstride + dc * 8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1, sh = (e & 1) * 16;
        const uint32_t b0 = (rows[0][w] >> sh) & 0xffffu, b1 = (rows[1][w] >> sh) & 0xffffu;
        const uint32_t b2 = (rows[2][w] >> sh) & 0xffffu, b3 = (rows[3][w] >> sh) & 0xffffu;
        u32x2 pk2 = {b0 | (b1 << 16), b2 | (b3 << 16)};
        *reinterpret_cast<u32x2*>(&Vt[(dc * 8 + e) * VS + 4 * kq]) = pk2;
      }
    }
  }
}

// Attention of one query's 16 heads against the staged block.
//   qop: Q^T B-operands (4 steps over d); kread(t, s): K A-operand for key tile t,
//   d-step s. Returns the normalised O^T fragments and lse2 for head (lane & 15).
template <int QN>
struct QueryGroup {
  bf16x8 qop[QN][4];
  f32x4 acc[QN][8];
  float m[QN], l[QN];
};

template <int QN>
__device__ __forceinline__ void attend_group(QueryGroup<QN>& qg, const uint16_t* Ks, const uint16_t* Vt,
                                             const int* diag_lim, float scale_log2) {
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
  // An opaque zero offset keeps the K/V fragment reads inside the query loop
  // (otherwise they are hoisted across queries into ~256 extra registers).
  int lds_off = 0;
  asm volatile("" : "+v"(lds_off));
  // S^T = K . Q^T
#pragma unroll
  for (int n = 0; n < QN; ++n)
#pragma unroll
    for (int t = 0; t < 8; ++t) qg.acc[n][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 a =
          as_bf16x8(*reinterpret_cast<const u32x4*>(&Ks[lds_off + (16 * t + c) * KS + 32 * s + 8 * qd]));
#pragma unroll
      for (int n = 0; n < QN; ++n) qg.acc[n][t] = mfma16x16x32(a, qg.qop[n][s], qg.acc[n][t]);
    }
  }
  // softmax over keys (per head = per lane column)
  bf16x8 pop[QN][4];
#pragma unroll
  for (int n = 0; n < QN; ++n) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = qg.acc[n][t][r] * scale_log2;
        if (16 * t + 4 * qd + r > diag_lim[n]) x = -__builtin_inff();
        qg.acc[n][t][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(qg.acc[n][t][r] - mx);
        qg.acc[n][t][r] = p;
        sum += p;
      }
    sum += shfl_xor_f(sum, 16);
    sum += shfl_xor_f(sum, 32);
    qg.m[n] = mx;
    qg.l[n] = sum;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 w;
      w[0] = pack_bf16x2(qg.acc[n][2 * s][0], qg.acc[n][2 * s][1]);
      w[1] = pack_bf16x2(qg.acc[n][2 * s][2], qg.acc[n][2 * s][3]);
      w[2] = pack_bf16x2(qg.acc[n][2 * s + 1][0], qg.acc[n][2 * s + 1][1]);
      w[3] = pack_bf16x2(qg.acc[n][2 * s + 1][2], qg.acc[n][2 * s + 1][3]);
      pop[n][s] = as_bf16x8(w);
    }
  }
  // O^T = V^T . P^T
#pragma unroll
  for (int n = 0; n < QN; ++n)
#pragma unroll
    for (int t = 0; t < 8; ++t) qg.acc[n][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint16_t* vp = &Vt[lds_off + (16 * dt + c) * VS + 32 * s + 4 * qd];
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 16);
      const bf16x8 a = as_bf16x8((u32x4){lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
      for (int n = 0; n < QN; ++n) qg.acc[n][dt] = mfma16x16x32(a, pop[n][s], qg.acc[n][dt]);
    }
  }
}

__device__ __forceinline__ void store_partial(const f32x4 (&acc)[8], float m, float l, uint16_t* part_o,
                                              float* part_lse, int64_t slot) {
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
  const float inv = 1.0f / l;
  uint16_t* dst = part_o + (slot * kHpg + c) * kHeadDim + 4 * qd;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    u32x2 w = {pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv), pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv)};
    *reinterpret_cast<u32x2*>(dst + 16 * dt) = w;
  }
  if (qd == 0) part_lse[slot * kHpg + c] = m + __builtin_amdgcn_logf(l);
}

constexpr int kAttnQN = 2;

__global__ __launch_bounds__(256, 2) void k_attn_prefill(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ entries, const int32_t* __restrict__ tiles, int32_t* __restrict__ tile_info,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse, int64_t n_tokens, int64_t row0, int G,
    int nbw, int topk, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBlock * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kHeadDim * VS];
  __shared__ int s_tile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, qd = lane >> 4;
  const int T = tile_info[0];
  const int Hq = G * kHpg;

  for (;;) {
    if (tid == 0) s_tile = atomicAdd(&tile_info[1], 1);
    __syncthreads();
    const int t = s_tile;
    if (t >= T) break;
    const int l = tiles[4 * t + 0];
    const int begin = tiles[4 * t + 1];
    const int len = tiles[4 * t + 2];
    const int g = l / nbw, b = l % nbw;
    const int64_t key0 = (int64_t)b * kBlock;
    const int nvalid = (int)min<int64_t>(kBlock, n_tokens - key0);

    // stage K_b (row-major) and V_b^T
    const uint16_t* kb = k + (key0 * G + g) * kHeadDim;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = p * 16 + (tid >> 4), cc = tid & 15;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (r < nvalid) val = ld16(kb + (int64_t)r * G * kHeadDim + cc * 8);
      *reinterpret_cast<u32x4*>(&Ks[r * KS + cc * 8]) = val;
    }
    stage_vt<256>(Vt, v + (key0 * G + g) * kHeadDim, (int64_t)G * kHeadDim, nvalid, tid);
    __syncthreads();

    for (int e0 = wave * kAttnQN; e0 < len; e0 += 4 * kAttnQN) {
      QueryGroup<kAttnQN> qg;
      int ent[kAttnQN], lim[kAttnQN];
#pragma unroll
      for (int n = 0; n < kAttnQN; ++n) {
        const int idx = min(e0 + n, len - 1);
        ent[n] = entries[begin + idx];
        const int64_t i = row0 + (ent[n] >> 4);
        lim[n] = ((i >> 7) == b) ? (int)(i - key0) : kBlock;  // causal limit inside the own block
        const uint16_t* qrow = q + ((i * Hq) + g * kHpg + c) * kHeadDim + 8 * qd;
#pragma unroll
        for (int s = 0; s < 4; ++s) qg.qop[n][s] = as_bf16x8(ld16(qrow + 32 * s));
      }
      attend_group<kAttnQN>(qg, Ks, Vt, lim, scale_log2);
#pragma unroll
      for (int n = 0; n < kAttnQN; ++n) {
        if (e0 + n < len) {
          const int64_t slot = ((int64_t)(ent[n] >> 4) * G + g) * topk + (ent[n] & 15);
          store_partial(qg.acc[n], qg.m[n], qg.l[n], part_o, part_lse, slot);
        }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(64) void k_attn_decode(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v,
                                                    const int32_t* __restrict__ ctx_lens,
                                                    const int32_t* __restrict__ sel,
                                                    uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
                                                    int64_t max_ctx, int G, int topk, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBlock * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kHeadDim * VS];
  const int item = blockIdx.x;
  const int sq = item / (G * topk), g = (item / topk) % G;
  const int b = sel[item];
  if (b < 0) return;
  const int tid = threadIdx.x, c = tid & 15, qd = tid >> 4;
  const int64_t i = ctx_lens[sq] - 1;
  const int64_t key0 = (int64_t)b * kBlock;
  const int nvalid = (int)min<int64_t>(kBlock, max_ctx - key0);
  const int Hq = G * kHpg;
  const uint16_t* kb = k + ((int64_t)sq * max_ctx * G + key0 * G + g) * kHeadDim;
  for (int p = 0; p < 32; ++p) {
    const int r = p * 4 + (tid >> 4), cc = tid & 15;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (r < nvalid) val = ld16(kb + (int64_t)r * G * kHeadDim + cc * 8);
    *reinterpret_cast<u32x4*>(&Ks[r * KS + cc * 8]) = val;
  }
  stage_vt<64>(Vt, v + ((int64_t)sq * max_ctx * G + key0 * G + g) * kHeadDim, (int64_t)G * kHeadDim, nvalid,
               tid);
  __syncthreads();
  QueryGroup<1> qg;
  const uint16_t* qrow = q + ((int64_t)sq * Hq + g * kHpg + c) * kHeadDim + 8 * qd;
#pragma unroll
  for (int s = 0; s < 4; ++s) qg.qop[0][s] = as_bf16x8(ld16(qrow + 32 * s));
  int lim[1] = {((i >> 7) == b) ? (int)(i - key0) : kBlock};
  attend_group<1>(qg, Ks, Vt, lim, scale_log2);
  store_partial(qg.acc[0], qg.m[0], qg.l[0], part_o, part_lse, item);
}

void launch_attn_prefill(const LaunchAttnPrefill& a, hipStream_t st) {
  hipLaunchKernelGGL(k_attn_prefill, dim3(a.grid), dim3(256), 0, st, a.q, a.k, a.v, a.entries, a.tiles,
                     a.tile_info, a.part_o, a.part_lse, a.n_tokens, a.row0, a.G, a.nbw, a.topk, a.scale_log2);
}

void launch_attn_decode(const LaunchAttnDecode& a, hipStream_t st) {
  const int items = a.batch * a.G * a.topk;
  if (items <= 0) return;
  hipLaunchKernelGGL(k_attn_decode, dim3(items), dim3(64), 0, st, a.q, a.k, a.v, a.ctx_lens, a.sel, a.part_o,
                     a.part_lse, a.max_ctx, a.G, a.topk, a.scale_log2);
}

}  // namespace msa
