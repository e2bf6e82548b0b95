// Second phase of the two-phase combine [pnsm, section 7]: merge the <= k
// softmax partials of every (query, head) without atomics.
//
// Slot u of row rr and group g carries o_u (normalised, bf16) and
// lse2_u = m_u + log2(l_u). With M = max_u lse2_u and w_u = 2^(lse2_u - M):
//   out = sum_u w_u o_u / sum_u w_u,    lse = (M + log2 sum_u w_u) * ln 2.
// The number of valid slots is min(k, b_loc + 1), the size of the selection.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// One workgroup per (row rr, group g); thread t: head t/16, dims 8*(t%16)..+7.
// Prefill rows may carry one extra partial from the dense pass covering the
// blocks shared by the row's whole 16-row unit; their slots are then skipped
// (both lists are ascending, so one merge walk finds them). Rows whose every
// selected block was shared were written by the dense pass and are skipped.
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ part_o,
                                                 const float* __restrict__ part_lse, uint16_t* __restrict__ out,
                                                 float* __restrict__ lse_out, int G, int topk, int64_t row0,
                                                 const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ sel,
                                                 int64_t sel_gstride, const int32_t* __restrict__ dense_cnt,
                                                 const int32_t* __restrict__ dense_list,
                                                 const uint16_t* __restrict__ dense_o,
                                                 const float* __restrict__ dense_lse, int nunits) {
  const int64_t rg = blockIdx.x;
  const int64_t rr = rg / G;
  const int g = (int)(rg % G);
  const int t = threadIdx.x, lane = t & 63, h = t >> 4, d0 = (t & 15) * 8;
  const int b_loc = ctx_lens ? (ctx_lens[rr] - 1) / kBlock : (int)((row0 + rr) / kBlock);
  const int nsel = min(topk, b_loc + 1);
  const int64_t slot0 = rg * topk;

  // slots whose block was covered by the dense pass: lane u < nsel tests its
  // block against the unit's shared list; one ballot gives the wave the mask
  uint64_t skip = 0ull;
  int nd = 0;
  if (dense_cnt) {
    const int unit = (int)(rr >> 4);
    nd = dense_cnt[g * nunits + unit];
    if (nd == nsel) return;  // written in full by the dense pass
    const int32_t* dl = dense_list + ((int64_t)g * nunits + unit) * topk;
    bool covered = false;
    if (lane < nsel) {
      const int b = sel[(int64_t)g * sel_gstride + rr * topk + lane];
      for (int j = 0; j < nd; ++j) covered |= (dl[j] == b);
    }
    skip = __ballot(covered);
  }
  const uint64_t use = ((nsel >= 64) ? ~0ull : ((1ull << nsel) - 1ull)) & ~skip;

  float lse_u[kMaxTopk];
  float M = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < kMaxTopk; ++u) {
    lse_u[u] = -__builtin_inff();
    if ((use >> u) & 1ull) lse_u[u] = __builtin_nontemporal_load(part_lse + (slot0 + u) * kHpg + h);
    M = fmaxf(M, lse_u[u]);
  }
  float dl2 = -__builtin_inff();
  if (nd > 0) {
    dl2 = __builtin_nontemporal_load(dense_lse + rg * kHpg + h);
    M = fmaxf(M, dl2);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (nd > 0) {
    const float w = __builtin_amdgcn_exp2f(dl2 - M);
    wsum += w;
    const u32x4 o = ld16_nt(dense_o + (rg * kHpg + h) * kHeadDim + d0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += w * bf2f(o[e] & 0xffffu);
      acc[2 * e + 1] += w * bf2f(o[e] >> 16);
    }
  }
#pragma unroll
  for (int u = 0; u < kMaxTopk; ++u) {
    if (!((use >> u) & 1ull)) continue;
    const float w = __builtin_amdgcn_exp2f(lse_u[u] - M);
    wsum += w;
    const u32x4 o = ld16_nt(part_o + ((slot0 + u) * kHpg + h) * kHeadDim + d0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += w * bf2f(o[e] & 0xffffu);
      acc[2 * e + 1] += w * bf2f(o[e] >> 16);
    }
  }
  const float inv = 1.0f / wsum;
  const int Hq = G * kHpg;
  u32x4 res;
#pragma unroll
  for (int e = 0; e < 4; ++e) res[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *reinterpret_cast<u32x4*>(out + (rr * Hq + g * kHpg + h) * kHeadDim + d0) = res;
  if (lse_out && (t & 15) == 0)
    lse_out[rr * Hq + g * kHpg + h] = (M + __builtin_amdgcn_logf(wsum)) * 0.69314718055994530942f;
}

void launch_combine(const LaunchCombine& a, hipStream_t st) {
  const int64_t n = a.nrows * a.G;
  if (n <= 0) return;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)n), dim3(256), 0, st, a.part_o, a.part_lse, a.out, a.lse_out, a.G,
                     a.topk, a.row0, a.ctx_lens, a.sel, a.sel_gstride, a.dense_cnt, a.dense_list, a.dense_o,
                     a.dense_lse, a.nunits);
}

}  // namespace msa
