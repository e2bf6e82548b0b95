// Index Branch KL alignment: the training signal of the block selector
// [pnsm, section 4; yhxrc, 二]. For a query row i and group g with support
// T = {j <= i : floor(j / B_k) in Sel[g, i]}:
//   teacher  P_main(j) = mean over the group's 16 query heads h of
//                        exp(scale * q[i,h] . k[j,g] - lse[i,h])
//   student  P_idx(j)  = softmax over T of s_j = q_idx[i,g] . k_idx[j]
//   loss     KL(P_main || P_idx)
// and the gradients of the summed loss with respect to q_idx and k_idx only
// (the main branch is detached): with gs_j = P_idx(j) - P_main(j),
//   dq_idx[i,g] = sum_T gs_j k_idx[j],   dk_idx[j] += gs_j q_idx[i,g].
// lse is the forward pass's (natural-log) output, so the teacher is the
// forward's own attention distribution.
//
// Work is organised like the KV-outer main branch: the reverse index of the
// selections lists, per (group, block), the queries that selected it (every
// pair, no dense split), cut into chunks of up to kKlChunk queries. One
// workgroup per chunk stages the block's K and k_idx in LDS once and takes
// the queries 16 at a time (8 waves x 2). Pass 1 writes, per (query, slot),
// the max and the sum of exp of the index scores over the block; a combine
// gives each (row, group) its log-normaliser. Pass 2 recomputes the scores,
// the teacher (S = Q K^T on MFMA; each lane holds four heads of one key) and
// gs, writes per (query, slot) the loss term and the dq_idx contribution, and
// accumulates dk_idx for the block's keys over the whole chunk (gs staged in
// LDS, one key row per lane), added to the output once per chunk.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kKlWaves = 8;
constexpr int kKStride = 272;    // LDS bytes per staged K row (256 + 16: spreads the banks)
constexpr int kIStride = 144;    // LDS bytes per staged k_idx row (128 + 16)
constexpr int kKlLds = kBlock * kKStride + kBlock * kIStride + 16 * kBlock * 4 + 16 * kIndexDim * 2;

__device__ __forceinline__ float sum_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// sum / max over the 16 lanes of a lane group (lanes differing in bits 0-3)
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

__device__ __forceinline__ void unpack8(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// PASS 1: per-slot (max, sum exp) of the index scores over the block.
// PASS 2: loss term, dq_idx contribution and the chunk's dk_idx.
template <int PASS>
__global__ __launch_bounds__(512, 2) void k_kl_pass(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ q_idx,
    const uint16_t* __restrict__ k_idx, const float* __restrict__ lse, const float* __restrict__ lse_idx,
    const int32_t* __restrict__ entries, const int32_t* __restrict__ chunks, const int32_t* __restrict__ chunk_info,
    float* __restrict__ part_m, float* __restrict__ part_l, float* __restrict__ loss_part,
    float* __restrict__ dq_part, float* __restrict__ dk_idx, int64_t n_tokens, int64_t row0, int G, int topk,
    float scale_log2) {
  __shared__ __attribute__((aligned(16))) char lds_raw[kKlLds];
  char* kst = lds_raw;
  char* ist = kst + kBlock * kKStride;
  float* gbuf = reinterpret_cast<float*>(ist + kBlock * kIStride);          // [16 queries][128 keys]
  uint16_t* qibuf = reinterpret_cast<uint16_t*>(gbuf + 16 * kBlock);         // [16 queries][64]
  const int t_id = blockIdx.x;
  if (t_id >= chunk_info[0]) return;
  const int g = chunks[4 * t_id], begin = chunks[4 * t_id + 1], len = chunks[4 * t_id + 2], b = chunks[4 * t_id + 3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, qd = lane >> 4;
  const int Hq = G * kHpg;
  const int64_t key0 = (int64_t)b * kBlock;
  const int nvalid = (int)min<int64_t>(kBlock, n_tokens - key0);  // keys of the block that exist

  // stage the block: K rows (pass 2) and k_idx rows, zero past the sequence
  if (PASS == 2) {
    for (int x = tid; x < kBlock * 16; x += 512) {
      const int r = x >> 4, ch = x & 15;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < nvalid) v = ld16(k + ((key0 + r) * G + g) * kHeadDim + ch * 8);
      *reinterpret_cast<u32x4*>(kst + r * kKStride + ch * 16) = v;
    }
  }
  for (int x = tid; x < kBlock * 8; x += 512) {
    const int r = x >> 3, ch = x & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < nvalid) v = ld16(k_idx + (key0 + r) * kIndexDim + ch * 8);
    *reinterpret_cast<u32x4*>(ist + r * kIStride + ch * 16) = v;
  }
  __syncthreads();

  float dk_acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) dk_acc[e] = 0.f;

  for (int s0 = 0; s0 < len; s0 += 16) {
    const int nsub = min(16, len - s0);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int tq = 2 * wave + n;  // query of the sub-tile
      if (tq >= nsub) continue;  // wave-uniform
      const int ent = entries[begin + s0 + tq];
      const int i_rel = ent >> 4, u = ent & 15;
      const int64_t i = row0 + i_rel;
      const int64_t slot = ((int64_t)i_rel * G + g) * topk + u;
      const int lim = (int)min<int64_t>(kBlock - 1, i - key0);  // keys <= lim are in T
      // the lane's 16 dims of q_idx[i, g]
      float qi[16];
      {
        const uint16_t* src = q_idx + ((int64_t)i_rel * G + g) * kIndexDim + 16 * qd;
        const u32x4 w0 = ld16(src), w1 = ld16(src + 8);
        unpack8(w0, qi);
        unpack8(w1, qi + 8);
        if (PASS == 2 && c == 0) {
          *reinterpret_cast<u32x4*>(qibuf + tq * kIndexDim + 16 * qd) = w0;
          *reinterpret_cast<u32x4*>(qibuf + tq * kIndexDim + 16 * qd + 8) = w1;
        }
      }
      if (PASS == 1) {
        float m = -__builtin_inff(), l = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int kk = 16 * t + c;
          float kv[16];
          unpack8(*reinterpret_cast<const u32x4*>(ist + kk * kIStride + 32 * qd), kv);
          unpack8(*reinterpret_cast<const u32x4*>(ist + kk * kIStride + 32 * qd + 16), kv + 8);
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) s = __builtin_fmaf(qi[e], kv[e], s);
          s = sum_lane_groups(s);
          if (kk <= lim) {
            const float mn = fmaxf(m, s);
            l = l * __expf(m - mn) + __expf(s - mn);
            m = mn;
          }
        }
        // merge (m, l) over the 16 keys of the lane group
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float m2 = __shfl_xor(m, o, kWave), l2 = __shfl_xor(l, o, kWave);
          const float mn = fmaxf(m, m2);
          l = (l == 0.f ? 0.f : l * __expf(m - mn)) + (l2 == 0.f ? 0.f : l2 * __expf(m2 - mn));
          m = mn;
        }
        if (lane == 0) {
          part_m[slot] = m;
          part_l[slot] = l;
        }
      } else {
        bf16x8 qop[4];
        const uint16_t* qrow = q + ((int64_t)i_rel * Hq + g * kHpg + c) * kHeadDim + 8 * qd;
#pragma unroll
        for (int st = 0; st < 4; ++st) qop[st] = as_bf16x8(ld16(qrow + 32 * st));
        // log2 e * lse of the lane's four heads 4qd .. 4qd+3
        const f32x4 lh = *reinterpret_cast<const f32x4*>(lse + (int64_t)i_rel * Hq + g * kHpg + 4 * qd);
        const float l2e = 1.4426950408889634f;
        const float lz = lse_idx[(int64_t)i_rel * G + g];
        float loss = 0.f;
        float dq[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) dq[e] = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int kk = 16 * t + c;
          // teacher: S[4qd + r][key kk] = q_h . k_kk over 4 d-steps
          f32x4 sm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const bf16x8 kb = as_bf16x8(*reinterpret_cast<const u32x4*>(kst + kk * kKStride + (32 * st + 8 * qd) * 2));
            sm = mfma16x16x32(qop[st], kb, sm);
          }
          float p = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) p += __builtin_amdgcn_exp2f(sm[r] * scale_log2 - lh[r] * l2e);
          const bool in_t = kk <= lim;
          p = sum_lane_groups(p);
          const float pm = in_t ? p * (1.0f / kHpg) : 0.f;
          // student
          float kv[16];
          unpack8(*reinterpret_cast<const u32x4*>(ist + kk * kIStride + 32 * qd), kv);
          unpack8(*reinterpret_cast<const u32x4*>(ist + kk * kIStride + 32 * qd + 16), kv + 8);
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) s = __builtin_fmaf(qi[e], kv[e], s);
          s = sum_lane_groups(s);
          const float lp = s - lz;  // log P_idx
          const float gs = in_t ? __expf(lp) - pm : 0.f;
          if (in_t && pm > 0.f) loss += pm * (__logf(pm) - lp);
#pragma unroll
          for (int e = 0; e < 16; ++e) dq[e] = __builtin_fmaf(gs, kv[e], dq[e]);
          if (qd == 0) gbuf[tq * kBlock + kk] = gs;
        }
        loss = sum16(loss);
        if (lane == 0) loss_part[slot] = loss;
#pragma unroll
        for (int e = 0; e < 16; ++e) dq[e] = sum16(dq[e]);
        if (c == 0) {
          float* dst = dq_part + slot * kIndexDim + 16 * qd;
#pragma unroll
          for (int e = 0; e < 16; e += 4)
            *reinterpret_cast<f32x4*>(dst + e) = (f32x4){dq[e], dq[e + 1], dq[e + 2], dq[e + 3]};
        }
      }
    }
    if (PASS == 2) {
      __syncthreads();  // gs and q_idx of the sub-tile staged
      // wave w: keys 16w + c; the lane's 16 dims 16qd ..
      const int kk = 16 * wave + c;
      for (int n = 0; n < nsub; ++n) {
        const float gv = gbuf[n * kBlock + kk];
        float qv[16];
        unpack8(*reinterpret_cast<const u32x4*>(qibuf + n * kIndexDim + 16 * qd), qv);
        unpack8(*reinterpret_cast<const u32x4*>(qibuf + n * kIndexDim + 16 * qd + 8), qv + 8);
#pragma unroll
        for (int e = 0; e < 16; ++e) dk_acc[e] = __builtin_fmaf(gv, qv[e], dk_acc[e]);
      }
      __syncthreads();  // before the next sub-tile overwrites the buffers
    }
  }
  if (PASS == 2) {
    const int kk = 16 * wave + c;
    if (kk < nvalid) {
      float* dst = dk_idx + (key0 + kk) * kIndexDim + 16 * qd;
#pragma unroll
      for (int e = 0; e < 16; ++e) atomicAdd(dst + e, dk_acc[e]);
    }
  }
}

// log-normaliser of each (row, group) over its support from the slot partials
__global__ __launch_bounds__(256) void k_kl_lse(const float* __restrict__ part_m, const float* __restrict__ part_l,
                                                float* __restrict__ lse_idx, int nrows, int64_t row0, int G,
                                                int topk) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= (int64_t)nrows * G) return;
  const int64_t i = row0 + x / G;
  const int nsel = (int)min<int64_t>(topk, i / kBlock + 1);
  float m = -__builtin_inff();
  for (int u = 0; u < nsel; ++u) m = fmaxf(m, part_m[x * topk + u]);
  float l = 0.f;
  for (int u = 0; u < nsel; ++u) l += part_l[x * topk + u] * __expf(part_m[x * topk + u] - m);
  lse_idx[x] = m + __logf(l);
}

// loss and dq_idx of each (row, group): sums of the slot terms; one wave each
__global__ __launch_bounds__(256) void k_kl_out(const float* __restrict__ loss_part, const float* __restrict__ dq_part,
                                                float* __restrict__ loss, float* __restrict__ dq_idx, int nrows,
                                                int64_t row0, int64_t n_tokens, int G, int topk) {
  const int64_t x = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (x >= (int64_t)nrows * G) return;
  const int lane = threadIdx.x & 63;
  const int64_t i_rel = x / G, i = row0 + i_rel;
  const int g = (int)(x % G);
  const int nsel = (int)min<int64_t>(topk, i / kBlock + 1);
  float d = 0.f, l = 0.f;
  for (int u = 0; u < nsel; ++u) {
    d += dq_part[(x * topk + u) * kIndexDim + lane];
    l += loss_part[x * topk + u];
  }
  dq_idx[x * kIndexDim + lane] = d;
  if (lane == 0) loss[(int64_t)g * n_tokens + i] = l;
}

__global__ __launch_bounds__(256) void k_zero_f32(float* __restrict__ p, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x)
    p[x] = 0.f;
}

void launch_kl_window(const LaunchKl& a, hipStream_t st) {
  if (a.nrows <= 0) return;
  hipLaunchKernelGGL(k_kl_pass<1>, dim3(a.chunk_cap), dim3(512), 0, st, a.q, a.k, a.q_idx, a.k_idx, a.lse,
                     a.lse_idx, a.entries, a.chunks, a.chunk_info, a.part_m, a.part_l, a.loss_part, a.dq_part,
                     a.dk_idx, a.n_tokens, a.row0, a.G, a.topk, a.scale_log2);
  const int64_t rows = (int64_t)a.nrows * a.G;
  hipLaunchKernelGGL(k_kl_lse, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, a.part_m, a.part_l,
                     a.lse_idx, a.nrows, a.row0, a.G, a.topk);
  hipLaunchKernelGGL(k_kl_pass<2>, dim3(a.chunk_cap), dim3(512), 0, st, a.q, a.k, a.q_idx, a.k_idx, a.lse,
                     a.lse_idx, a.entries, a.chunks, a.chunk_info, a.part_m, a.part_l, a.loss_part, a.dq_part,
                     a.dk_idx, a.n_tokens, a.row0, a.G, a.topk, a.scale_log2);
  hipLaunchKernelGGL(k_kl_out, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a.loss_part, a.dq_part,
                     a.loss, a.dq_idx, a.nrows, a.row0, a.n_tokens, a.G, a.topk);
}

void launch_zero_f32(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
}

}  // namespace msa
