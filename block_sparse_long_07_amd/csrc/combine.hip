// Second phase of the two-phase combine [pnsm, section 7] for decode: merge
// the <= k softmax partials of every (sequence, head) without atomics. (Prefill
// merges its partials at the end of the dense attention pass.)
//
// Slot u of row rr and group g carries o_u (normalised, bf16) and
// lse2_u = m_u + log2(l_u). With M = max_u lse2_u and w_u = 2^(lse2_u - M):
//   out = sum_u w_u o_u / sum_u w_u,    lse = (M + log2 sum_u w_u) * ln 2.
// The number of valid slots is min(k, b_loc + 1), the size of the selection.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// Decode: one workgroup per (sequence, group); thread t: head h = t/16, dims
// d0 = 8*(t%16) .. +7. Partials are stored in fragment order: element (head h,
// dim 16dt + 4qd + r) at dt*256 + (16qd + h)*4 + r of the slot, so the eight
// dims of a thread are two 8-byte pieces (qd and qd + 1 of tile dt).
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ part_o,
                                                 const float* __restrict__ part_lse, uint16_t* __restrict__ out,
                                                 float* __restrict__ lse_out, int G, int topk,
                                                 const int32_t* __restrict__ ctx_lens, int bk_shift) {
  const int64_t rg = blockIdx.x;
  const int64_t rr = rg / G;
  const int g = (int)(rg % G);
  const int t = threadIdx.x, h = t >> 4, d0 = (t & 15) * 8;
  const int dt = d0 >> 4, qd = (d0 & 15) >> 2;
  const int b_loc = (ctx_lens[rr] - 1) >> bk_shift;
  const int nsel = min(topk, b_loc + 1);
  const int64_t slot0 = rg * topk;

  float lse_u[kMaxTopk];
  float M = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < kMaxTopk; ++u) {
    lse_u[u] = -__builtin_inff();
    if (u < nsel) lse_u[u] = __builtin_nontemporal_load(part_lse + (slot0 + u) * kHpg + h);
    M = fmaxf(M, lse_u[u]);
  }
  // every slot's loads are issued before any is used, so their latencies
  // overlap; the sum then runs in slot order
  u32x2 pa[kMaxTopk], pb[kMaxTopk];
#pragma unroll
  for (int u = 0; u < kMaxTopk; ++u) {
    pa[u] = pb[u] = (u32x2){0u, 0u};
    if (u < nsel) {
      const uint16_t* src = part_o + (slot0 + u) * (kHpg * kHeadDim) + dt * 256 + (16 * qd + h) * 4;
      pa[u] = *reinterpret_cast<const u32x2*>(src);
      pb[u] = *reinterpret_cast<const u32x2*>(src + 64);  // qd + 1
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
#pragma unroll
  for (int u = 0; u < kMaxTopk; ++u) {
    if (u < nsel) {
      const float w = __builtin_amdgcn_exp2f(lse_u[u] - M);
      wsum += w;
      const uint32_t o[4] = {pa[u][0], pa[u][1], pb[u][0], pb[u][1]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += w * bf2f(o[e] & 0xffffu);
        acc[2 * e + 1] += w * bf2f(o[e] >> 16);
      }
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
                     a.topk, a.ctx_lens, a.bk_shift);
}

}  // namespace msa
