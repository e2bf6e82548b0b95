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

// Stage K_b row-major into Ks (128 keys x 128 d, padded rows). `rstride` is the
// element distance between consecutive keys; keys >= nvalid are zero-filled.
template <int NTHR>
__device__ __forceinline__ void stage_k(uint16_t* Ks, const uint16_t* krow0, int64_t rstride, int nvalid, int tid) {
#pragma unroll
  for (int p = 0; p < 2048 / NTHR; ++p) {
    const int it = p * NTHR + tid;
    const int r = it >> 4, cc = it & 15;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (r < nvalid) val = ld16(krow0 + (int64_t)r * rstride + cc * 8);
    *reinterpret_cast<u32x4*>(&Ks[r * KS + cc * 8]) = val;
  }
}

// Stage V_b transposed into Vt [d][key]. Work item `it` (0..511) covers key
// quad kq (4 keys) x d-chunk dc (8 dims): kq = it%16 + 16*(it/256), dc =
// (it/16)%16. Within a wave kq varies fastest, which keeps both the global
// reads and the transposed 8-byte LDS writes free of bank conflicts.
template <int NTHR>
__device__ __forceinline__ void stage_vt(uint16_t* Vt, const uint16_t* vrow0, int64_t rstride, int nvalid,
                                         int tid) {
#pragma unroll
  for (int p = 0; p < 512 / NTHR; ++p) {
    const int it = p * NTHR + tid;
    const int kq = (it & 15) | ((it >> 8) << 4);
    const int dc = (it >> 4) & 15;
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

// Per-wave state of QN queries (16 heads each) against staged blocks.
//   qop: Q^T B-operands (4 steps over d); s: S^T / P^T fragments of the current
//   block; o: O^T accumulators (head = lane & 15, d = 16*dt + 4*(lane/16) + r);
//   m, l: running max (log2 domain) and denominator per head.
template <int QN>
struct QueryGroup {
  bf16x8 qop[QN][4];
  f32x4 s[QN][8];
  f32x4 o[QN][8];
  float m[QN], l[QN];
};

template <int QN>
__device__ __forceinline__ void load_q(QueryGroup<QN>& qg, int n, const uint16_t* qrow) {
#pragma unroll
  for (int st = 0; st < 4; ++st) qg.qop[n][st] = as_bf16x8(ld16(qrow + 32 * st));
}

// S^T = K_b . Q^T for the QN queries (4 steps over d per 16-key tile).
template <int QN>
__device__ __forceinline__ void scores(QueryGroup<QN>& qg, const uint16_t* Ks) {
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
  // An opaque zero offset keeps the K fragment reads inside the query loop
  // (otherwise they are hoisted across queries into ~128 extra registers).
  int lds_off = 0;
  asm volatile("" : "+v"(lds_off));
#pragma unroll
  for (int n = 0; n < QN; ++n)
#pragma unroll
    for (int t = 0; t < 8; ++t) qg.s[n][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8 a =
          as_bf16x8(*reinterpret_cast<const u32x4*>(&Ks[lds_off + (16 * t + c) * KS + 32 * st + 8 * qd]));
#pragma unroll
      for (int n = 0; n < QN; ++n) qg.s[n][t] = mfma16x16x32(a, qg.qop[n][st], qg.s[n][t]);
    }
  }
}

// Online-softmax update of (m, l, O) with the block's scores, then
// O^T += V_b^T . P^T. Keys with index > lim[n] inside the block are masked
// (causal limit in the query's own block; lim >= 127 means no mask). The
// logit scale is folded into the exponent: p = 2^(s*c - m*c), m tracked on raw
// scores. FIRST: the state is fresh (no rescaling of O and l needed).
template <int QN, bool FIRST>
__device__ __forceinline__ void softmax_pv(QueryGroup<QN>& qg, const uint16_t* Vt, const int* lim,
                                           float scale_log2) {
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
  int lds_off = 0;
  asm volatile("" : "+v"(lds_off));
  bf16x8 pop[QN][4];
#pragma unroll
  for (int n = 0; n < QN; ++n) {
    if (lim[n] < kBlock - 1) {  // wave-uniform: only the query's own block
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * t + 4 * qd + r > lim[n]) qg.s[n][t][r] = -__builtin_inff();
    }
    float mx = FIRST ? -__builtin_inff() : qg.m[n];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      mx = fmaxf(fmaxf(mx, fmaxf(qg.s[n][t][0], qg.s[n][t][1])), fmaxf(qg.s[n][t][2], qg.s[n][t][3]));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float mc = mx * scale_log2;
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(qg.s[n][t][r], scale_log2, -mc));
        qg.s[n][t][r] = pv;
        sum += pv;
      }
    sum += shfl_xor_f(sum, 16);
    sum += shfl_xor_f(sum, 32);
    if (FIRST) {
      qg.l[n] = sum;
    } else {
      const float alpha = __builtin_amdgcn_exp2f((qg.m[n] - mx) * scale_log2);
      qg.l[n] = qg.l[n] * alpha + sum;
#pragma unroll
      for (int t = 0; t < 8; ++t) qg.o[n][t] *= alpha;
    }
    qg.m[n] = mx;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      u32x4 w;
      w[0] = pack_bf16x2(qg.s[n][2 * st][0], qg.s[n][2 * st][1]);
      w[1] = pack_bf16x2(qg.s[n][2 * st][2], qg.s[n][2 * st][3]);
      w[2] = pack_bf16x2(qg.s[n][2 * st + 1][0], qg.s[n][2 * st + 1][1]);
      w[3] = pack_bf16x2(qg.s[n][2 * st + 1][2], qg.s[n][2 * st + 1][3]);
      pop[n][st] = as_bf16x8(w);
    }
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint16_t* vp = &Vt[lds_off + (16 * dt + c) * VS + 32 * st + 4 * qd];
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 16);
      const bf16x8 a = as_bf16x8((u32x4){lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
      for (int n = 0; n < QN; ++n) {
        if (FIRST && st == 0)
          qg.o[n][dt] = mfma16x16x32(a, pop[n][st], (f32x4){0.f, 0.f, 0.f, 0.f});
        else
          qg.o[n][dt] = mfma16x16x32(a, pop[n][st], qg.o[n][dt]);
      }
    }
  }
}

// Normalised O (bf16, [16 heads][128 d] at dst) and lse2 = m*c + log2(l) of
// one query (c = scale*log2 e).
__device__ __forceinline__ void store_normalised(const f32x4 (&o)[8], float m, float l, float scale_log2,
                                                 uint16_t* dst16x128, float* lse16) {
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
  const float inv = 1.0f / l;
  uint16_t* dst = dst16x128 + c * kHeadDim + 4 * qd;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    u32x2 w = {pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv), pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
    *reinterpret_cast<u32x2*>(dst + 16 * dt) = w;
  }
  if (qd == 0) lse16[c] = m * scale_log2 + __builtin_amdgcn_logf(l);
}

constexpr int kAttnQN = 2;

// Sparse (KV-outer) part: persistent workgroups drain the tile queue. Each wave
// takes QN queries of the tile at a time; the next group's Q is loaded into the
// Q registers as soon as the current scores are formed, so its latency overlaps
// the softmax and the P.V contraction.
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

    QueryGroup<kAttnQN> qg;
    int ent[kAttnQN];
    int e0 = wave * kAttnQN;
    if (e0 < len) {
#pragma unroll
      for (int n = 0; n < kAttnQN; ++n) {
        ent[n] = entries[begin + min(e0 + n, len - 1)];
        const int64_t i = row0 + (ent[n] >> 4);
        load_q(qg, n, q + ((i * Hq) + g * kHpg + c) * kHeadDim + 8 * qd);
      }
    }
    stage_k<256>(Ks, k + (key0 * G + g) * kHeadDim, (int64_t)G * kHeadDim, nvalid, tid);
    stage_vt<256>(Vt, v + (key0 * G + g) * kHeadDim, (int64_t)G * kHeadDim, nvalid, tid);
    __syncthreads();

    for (; e0 < len; e0 += 4 * kAttnQN) {
      scores(qg, Ks);
      int lim[kAttnQN], cur[kAttnQN];
#pragma unroll
      for (int n = 0; n < kAttnQN; ++n) {
        cur[n] = ent[n];
        const int64_t i = row0 + (cur[n] >> 4);
        lim[n] = ((i >> 7) == b) ? (int)(i - key0) : kBlock;  // causal limit inside the own block
      }
      const int e1 = e0 + 4 * kAttnQN;
      if (e1 < len) {  // prefetch the next group's Q into the (now free) Q registers
#pragma unroll
        for (int n = 0; n < kAttnQN; ++n) {
          ent[n] = entries[begin + min(e1 + n, len - 1)];
          const int64_t i = row0 + (ent[n] >> 4);
          load_q(qg, n, q + ((i * Hq) + g * kHpg + c) * kHeadDim + 8 * qd);
        }
      }
      softmax_pv<kAttnQN, true>(qg, Vt, lim, scale_log2);
#pragma unroll
      for (int n = 0; n < kAttnQN; ++n) {
        if (e0 + n < len) {
          const int64_t slot = ((int64_t)(cur[n] >> 4) * G + g) * topk + (cur[n] & 15);
          store_normalised(qg.o[n], qg.m[n], qg.l[n], scale_log2, part_o + slot * kHpg * kHeadDim,
                           part_lse + slot * kHpg);
        }
      }
    }
    __syncthreads();
  }
}

// Dense part: blocks selected by every query of a 16-query unit are computed
// query-stationary (FlashAttention-style online softmax over the unit's shared
// blocks, K/V staged once per block for all 16 queries). One workgroup of 8
// waves per (unit, group), two queries per wave. A unit whose every selected
// block is shared writes the final output directly; otherwise its single
// partial is merged with the KV-outer partials by the combine pass.
__global__ __launch_bounds__(512, 1) void k_attn_dense(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ dense_cnt, const int32_t* __restrict__ dense_list, uint16_t* __restrict__ dense_o,
    float* __restrict__ dense_lse, uint16_t* __restrict__ out, float* __restrict__ lse_out, int64_t n_tokens,
    int64_t row0, int nrows, int nunits, int G, int topk, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBlock * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kHeadDim * VS];
  const int unit = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, qd = lane >> 4;
  const int Hq = G * kHpg;
  const int nd = dense_cnt[g * nunits + unit];
  const int32_t* list = dense_list + ((int64_t)g * nunits + unit) * topk;
  const int i_rel0 = unit * 16 + wave * kAttnQN;
  const int b_loc = (int)((row0 + unit * 16) / kBlock);
  const bool final_out = nd == min(topk, b_loc + 1);

  QueryGroup<kAttnQN> qg;
  int lim[kAttnQN];
#pragma unroll
  for (int n = 0; n < kAttnQN; ++n) {
    const int64_t i = row0 + min(i_rel0 + n, nrows - 1);
    load_q(qg, n, q + ((i * Hq) + g * kHpg + c) * kHeadDim + 8 * qd);
    qg.m[n] = -__builtin_inff();  // running state: the first block rescales by 2^-inf = 0
    qg.l[n] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) qg.o[n][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  for (int d = 0; d < nd; ++d) {
    const int b = list[d];
    const int64_t key0 = (int64_t)b * kBlock;
    const int nvalid = (int)min<int64_t>(kBlock, n_tokens - key0);
    stage_k<512>(Ks, k + (key0 * G + g) * kHeadDim, (int64_t)G * kHeadDim, nvalid, tid);
    stage_vt<512>(Vt, v + (key0 * G + g) * kHeadDim, (int64_t)G * kHeadDim, nvalid, tid);
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kAttnQN; ++n) {
      const int64_t i = row0 + min(i_rel0 + n, nrows - 1);
      lim[n] = (b == b_loc) ? (int)(i - key0) : kBlock;
    }
    scores(qg, Ks);
    softmax_pv<kAttnQN, false>(qg, Vt, lim, scale_log2);
    __syncthreads();
  }
#pragma unroll
  for (int n = 0; n < kAttnQN; ++n) {
    const int i_rel = i_rel0 + n;
    if (i_rel >= nrows) continue;
    if (final_out) {
      const float inv = 1.0f / qg.l[n];
      uint16_t* dst = out + ((int64_t)i_rel * Hq + g * kHpg + c) * kHeadDim + 4 * qd;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        u32x2 w = {pack_bf16x2(qg.o[n][dt][0] * inv, qg.o[n][dt][1] * inv),
                   pack_bf16x2(qg.o[n][dt][2] * inv, qg.o[n][dt][3] * inv)};
        *reinterpret_cast<u32x2*>(dst + 16 * dt) = w;
      }
      if (lse_out && qd == 0)
        lse_out[(int64_t)i_rel * Hq + g * kHpg + c] =
            (qg.m[n] * scale_log2 + __builtin_amdgcn_logf(qg.l[n])) * 0.69314718055994530942f;
    } else {
      const int64_t row = (int64_t)i_rel * G + g;
      store_normalised(qg.o[n], qg.m[n], qg.l[n], scale_log2, dense_o + row * kHpg * kHeadDim,
                       dense_lse + row * kHpg);
    }
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
  const int64_t base = ((int64_t)sq * max_ctx * G + key0 * G + g) * kHeadDim;
  QueryGroup<1> qg;
  load_q(qg, 0, q + ((int64_t)sq * Hq + g * kHpg + c) * kHeadDim + 8 * qd);
  stage_k<64>(Ks, k + base, (int64_t)G * kHeadDim, nvalid, tid);
  stage_vt<64>(Vt, v + base, (int64_t)G * kHeadDim, nvalid, tid);
  __syncthreads();
  int lim[1] = {((i >> 7) == b) ? (int)(i - key0) : kBlock};
  scores(qg, Ks);
  softmax_pv<1, true>(qg, Vt, lim, scale_log2);
  store_normalised(qg.o[0], qg.m[0], qg.l[0], scale_log2, part_o + (int64_t)item * kHpg * kHeadDim,
                   part_lse + (int64_t)item * kHpg);
}

void launch_attn_prefill(const LaunchAttnPrefill& a, hipStream_t st) {
  hipLaunchKernelGGL(k_attn_prefill, dim3(a.grid), dim3(256), 0, st, a.q, a.k, a.v, a.entries, a.tiles,
                     a.tile_info, a.part_o, a.part_lse, a.n_tokens, a.row0, a.G, a.nbw, a.topk, a.scale_log2);
}

void launch_attn_dense(const LaunchAttnDense& a, hipStream_t st) {
  if (a.nunits <= 0) return;
  hipLaunchKernelGGL(k_attn_dense, dim3(a.nunits, a.G), dim3(512), 0, st, a.q, a.k, a.v, a.dense_cnt, a.dense_list,
                     a.dense_o, a.dense_lse, a.out, a.lse_out, a.n_tokens, a.row0, a.nrows, a.nunits, a.G, a.topk,
                     a.scale_log2);
}

void launch_attn_decode(const LaunchAttnDecode& a, hipStream_t st) {
  const int items = a.batch * a.G * a.topk;
  if (items <= 0) return;
  hipLaunchKernelGGL(k_attn_decode, dim3(items), dim3(64), 0, st, a.q, a.k, a.v, a.ctx_lens, a.sel, a.part_o,
                     a.part_lse, a.max_ctx, a.G, a.topk, a.scale_log2);
}

}  // namespace msa
