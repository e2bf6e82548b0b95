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
// pair, no dense split), cut into chunks of up to 512 queries. One workgroup
// per chunk stages the block's K and k_idx (also transposed) in LDS once and
// takes the queries 16 at a time. Pass 1 writes, per (query, slot), the max
// and the sum of exp of the index scores over the block; a combine gives each
// (row, group) its log-normaliser. Pass 2 computes the teacher of each query
// over the block's keys (S = Q K^T on MFMA, two queries per wave, into LDS),
// then each wave takes 16 keys for all 16 queries: the index scores in both
// orientations on MFMA, gs in both layouts, and dk_idx^T = q_idx^T G and
// dq_idx^T = k_idx^T G^T as MFMAs with gs split into two bf16 parts (about 16
// significant bits). dq_idx and the loss are summed over the block's key
// tiles in a fixed order and written per (query, slot); dk_idx is accumulated
// over the whole chunk and written as the chunk's partial, which a last pass
// adds, per key block and in a fixed order, to the output (no atomics: the
// result does not depend on scheduling).
#include <type_traits>

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// staged K: row r at r * 256 bytes, its 16-byte piece p at position p ^ (r & 15)
// (the teacher's operand reads then hit 64 distinct banks per lane group)
constexpr int kIStride = 144;    // LDS bytes per staged k_idx row (128 + 16)
constexpr int kTStride = 272;    // LDS bytes per row of the transposed k_idx (128 keys + 8 pad)
constexpr int kSub = 16;         // queries per sub-tile of pass 1
constexpr int kSub2 = 16;        // queries per sub-tile of pass 2 (MFMA column blocks of 16)
constexpr int kPStride = kSub2 + 4;  // floats per teacher row (spreads the banks)
constexpr int kQStride = 72;     // bf16 per q_idx row (64 + 8)
constexpr int kRStride = kSub2 + 1;  // floats per row of the dq reduction buffer

typedef short kl_i16x4 __attribute__((ext_vector_type(4)));

// Scheduling pattern of one pipelined region: NM MFMAs, NV VALU and ND LDS
// reads spread evenly between them; nothing moves across the region's end.
template <int NM, int NV, int ND, int I = 0>
__device__ __forceinline__ void kl_sched_region() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    constexpr int vi = (NV * (I + 1)) / NM - (NV * I) / NM;
    constexpr int di = (ND * (I + 1)) / NM - (ND * I) / NM;
    if constexpr (vi > 0) __builtin_amdgcn_sched_group_barrier(0x002, vi, 0);  // VALU
    if constexpr (di > 0) __builtin_amdgcn_sched_group_barrier(0x100, di, 0);  // LDS read
    kl_sched_region<NM, NV, ND, I + 1>();
  } else {
    __builtin_amdgcn_sched_barrier(0);
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

// MFMA 16x16x16 bf16: lane (i, q) holds A[i][4q + j] and B[4q + j][i], j < 4;
// the result has the 16x16x32 product's layout.
__device__ __forceinline__ f32x4 kl_mfma16(kl_i16x4 a, kl_i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float sum_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// (max, sum of exp) pairs merged over the four lane groups (lanes l ^ 16, l ^ 32)
__device__ __forceinline__ void merge_lane_groups(float& m, float& l) {
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) {
    const float m2 = __shfl_xor(m, o, kWave), l2 = __shfl_xor(l, o, kWave);
    const float mn = fmaxf(m, m2);
    l = (l == 0.f ? 0.f : l * __expf(m - mn)) + (l2 == 0.f ? 0.f : l2 * __expf(m2 - mn));
    m = mn;
  }
}

// g = hi + lo, both bf16 (about 16 significant bits), packed as MFMA operands
__device__ __forceinline__ void split_bf16(const float (&g)[4], kl_i16x4& hi, kl_i16x4& lo) {
  uint32_t h[2], l[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    h[j] = pack_bf16x2(g[2 * j], g[2 * j + 1]);
    l[j] = pack_bf16x2(g[2 * j] - bf2f(h[j] & 0xffffu), g[2 * j + 1] - bf2f(h[j] >> 16));
  }
  hi = __builtin_bit_cast(kl_i16x4, (u32x2){h[0], h[1]});
  lo = __builtin_bit_cast(kl_i16x4, (u32x2){l[0], l[1]});
}

// The sub-tile's per-query data, loaded one sub-tile ahead: thread x < 16 the
// entry and (pass 2) log-normaliser of query x; thread x < 128 the 16-byte
// piece x & 7 of query x >> 3's q_idx row.
struct SubMeta {
  int ent;
  float lz;
  u32x4 qv;
};

template <bool LZ, int NQ>
__device__ __forceinline__ void load_meta(SubMeta& m, const int32_t* entries, const uint16_t* q_idx,
                                          const float* lse_idx, int at, int nsub, int G, int g) {
  const int tid = threadIdx.x;
  m.ent = -1;
  m.lz = 0.f;
  m.qv = (u32x4){0u, 0u, 0u, 0u};
  if (tid < NQ && tid < nsub) {
    m.ent = entries[at + tid];
    if (LZ) m.lz = lse_idx[(int64_t)(m.ent >> 4) * G + g];
  }
  if (tid < NQ * 8) {
    const int n = tid >> 3;
    if (n < nsub) {
      const int ent = entries[at + n];
      m.qv = ld16(q_idx + ((int64_t)(ent >> 4) * G + g) * kIndexDim + (tid & 7) * 8);
    }
  }
}

// publishes a SubMeta into LDS: slot, support limit and log-normaliser of each
// query (limit -1: no query), q_idx rows and their transpose
template <int NQ, class L>
__device__ __forceinline__ void store_meta(L& S, const SubMeta& m, int64_t row0, int64_t key0, int G, int g,
                                           int topk) {
  const int tid = threadIdx.x;
  if (tid < NQ) {
    int sl = 0, lm = -1;
    if (m.ent >= 0) {
      const int i_rel = m.ent >> 4;
      sl = (i_rel * G + g) * topk + (m.ent & 15);
      lm = (int)min<int64_t>(kBlock - 1, row0 + i_rel - key0);
    }
    S.slot[tid] = sl;
    S.lim[tid] = lm;
    S.lz[tid] = m.lz;
  }
  if (tid < NQ * 8) {
    const int n = tid >> 3, ch = tid & 7;
    *reinterpret_cast<u32x4*>(&S.qib[n][ch * 8]) = m.qv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      S.qibT[ch * 8 + 2 * j][n] = (uint16_t)(m.qv[j] & 0xffffu);
      S.qibT[ch * 8 + 2 * j + 1][n] = (uint16_t)(m.qv[j] >> 16);
    }
  }
}

// index scores of the wave's 16 keys (kw ..) for queries 16j .. 16j+15 of the
// sub-tile: sa[r] = S_idx[query 16j + 4qd + r][key kw + c],
// sb[r] = S_idx[query 16j + c][key kw + 4qd + r]
template <class L>
__device__ __forceinline__ void index_scores_tile(const L& S, int kw, int j, f32x4& sa, f32x4& sb) {
  const int lane = threadIdx.x & 63, c = lane & 15, qd = lane >> 4;
  sa = (f32x4){0.f, 0.f, 0.f, 0.f};
  sb = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(&S.qib[16 * j + c][32 * st + 8 * qd]));
    const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(S.ist + (kw + c) * kIStride + (32 * st + 8 * qd) * 2));
    sa = mfma16x16x32(qa, ka, sa);
    sb = mfma16x16x32(ka, qa, sb);
  }
}

template <class L>
__device__ __forceinline__ void stage_kidx(L& S, const uint16_t* k_idx, int64_t key0, int nvalid, bool transpose) {
  for (int x = threadIdx.x; x < kBlock * 8; x += blockDim.x) {
    const int r = x >> 3, ch = x & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < nvalid) v = ld16(k_idx + (key0 + r) * kIndexDim + ch * 8);
    *reinterpret_cast<u32x4*>(S.ist + r * kIStride + ch * 16) = v;
    if (transpose) {
      uint16_t* col = reinterpret_cast<uint16_t*>(S.istT) + r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        col[(8 * ch + 2 * j) * (kTStride / 2)] = (uint16_t)(v[j] & 0xffffu);
        col[(8 * ch + 2 * j + 1) * (kTStride / 2)] = (uint16_t)(v[j] >> 16);
      }
    }
  }
}

struct KlLds1 {
  char ist[kBlock * kIStride];            // k_idx rows
  uint16_t qib[kSub][kQStride];           // q_idx rows of the sub-tile
  uint16_t qibT[kIndexDim][kSub];         // (unused here)
  float mlb[8][kSub][2];                  // per-wave (max, sum exp)
  float lz[kSub];
  int lim[kSub];                          // keys <= lim are in the query's support
  int slot[kSub];
  char istT[1];                           // (unused here)
};

struct KlLds2 {
  char kst[kBlock * 256];                 // K rows of the block (swizzled, see above)
  char ist[kBlock * kIStride];            // k_idx rows
  char istT[kIndexDim * kTStride];        // k_idx transposed: [dim][key]
  float pbuf[kBlock][kPStride];           // teacher P_main[key][query]
  uint16_t qib[kSub2][kQStride];
  uint16_t qibT[kIndexDim][kSub2];
  float red[4][kIndexDim][kRStride];      // dq partials [dim][query] of two key tiles each
  float lossb[8][kSub2];
  float lz[kSub2];                        // log-normaliser of each query
  int lim[kSub2];
  int slot[kSub2];
};

// Pass 1: per-slot (max, sum exp) of the index scores over the block. Wave w
// takes keys 16w .. 16w+15 of every query of the sub-tile.
__global__ __launch_bounds__(512) void k_kl_norm(const uint16_t* __restrict__ q_idx,
                                                 const uint16_t* __restrict__ k_idx,
                                                 const int32_t* __restrict__ entries,
                                                 const int32_t* __restrict__ chunks,
                                                 const int32_t* __restrict__ chunk_info, float* __restrict__ part_m,
                                                 float* __restrict__ part_l, int64_t n_tokens, int64_t row0, int G,
                                                 int topk) {
  __shared__ __attribute__((aligned(16))) KlLds1 S;
  const int t_id = blockIdx.x;
  if (t_id >= chunk_info[0]) return;
  const int g = chunks[4 * t_id], begin = chunks[4 * t_id + 1], len = chunks[4 * t_id + 2], b = chunks[4 * t_id + 3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, qd = lane >> 4;
  const int64_t key0 = (int64_t)b * kBlock;
  const int nvalid = (int)min<int64_t>(kBlock, n_tokens - key0);
  const int kw = 16 * wave;
  stage_kidx(S, k_idx, key0, nvalid, false);
  SubMeta cur, nxt;
  load_meta<false, kSub>(cur, entries, q_idx, nullptr, begin, min(kSub, len), G, g);
  for (int s0 = 0; s0 < len; s0 += kSub) {
    const int nsub = min(kSub, len - s0);
    store_meta<kSub>(S, cur, row0, key0, G, g, topk);
    if (s0 + kSub < len)
      load_meta<false, kSub>(nxt, entries, q_idx, nullptr, begin + s0 + kSub, min(kSub, len - s0 - kSub), G, g);
    lds_barrier();  // block staged; the sub-tile's queries in LDS
    f32x4 sa, sb;
    index_scores_tile(S, kw, 0, sa, sb);
    const int lm = S.lim[c];
    float m = -__builtin_inff(), l = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (kw + 4 * qd + r <= lm) m = fmaxf(m, sb[r]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (kw + 4 * qd + r <= lm) l += __expf(sb[r] - m);
    merge_lane_groups(m, l);
    if (qd == 0) {
      S.mlb[wave][c][0] = m;
      S.mlb[wave][c][1] = l;
    }
    lds_barrier();
    if (tid < nsub) {
      float mm = -__builtin_inff(), ll = 0.f;
      for (int w = 0; w < 8; ++w) {
        const float m2 = S.mlb[w][tid][0], l2 = S.mlb[w][tid][1];
        const float mn = fmaxf(mm, m2);
        ll = (ll == 0.f ? 0.f : ll * __expf(mm - mn)) + (l2 == 0.f ? 0.f : l2 * __expf(m2 - mn));
        mm = mn;
      }
      part_m[S.slot[tid]] = mm;
      part_l[S.slot[tid]] = ll;
    }
    lds_barrier();  // before the next sub-tile overwrites the buffers
    cur = nxt;
  }
}

// Pass 2: loss term and dq_idx contribution per slot, and the chunk's dk_idx.
// Per sub-tile of kSub2 queries: wave w computes the teacher of its kSub2/8
// queries for all 128 keys into pbuf (key tiles software-pipelined); then wave
// w takes keys 16w .. 16w+15 for all the sub-tile's queries (column blocks of
// 16): S_idx on MFMA in both orientations, gs in both layouts, and
// dk^T = q_idx^T G, dq^T = k_idx^T G^T as 16x16x16 MFMAs.
__global__ __launch_bounds__(512, 1) void k_kl_grad(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ q_idx,
    const uint16_t* __restrict__ k_idx, const float* __restrict__ lse, const float* __restrict__ lse_idx,
    const int32_t* __restrict__ entries, const int32_t* __restrict__ chunks, const int32_t* __restrict__ chunk_info,
    float* __restrict__ loss_part, float* __restrict__ dq_part, float* __restrict__ dk_part, int64_t n_tokens,
    int64_t row0, int G, int topk, float scale_log2) {
  __shared__ __attribute__((aligned(16))) KlLds2 S;
  const int t_id = blockIdx.x;
  if (t_id >= chunk_info[0]) return;
  const int g = chunks[4 * t_id], begin = chunks[4 * t_id + 1], len = chunks[4 * t_id + 2], b = chunks[4 * t_id + 3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, qd = lane >> 4;
  const int Hq = G * kHpg;
  const int64_t key0 = (int64_t)b * kBlock;
  const int nvalid = (int)min<int64_t>(kBlock, n_tokens - key0);
  const int kw = 16 * wave;

  for (int x = tid; x < kBlock * 16; x += 512) {
    const int r = x >> 4, ch = x & 15;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < nvalid) v = ld16(k + ((key0 + r) * G + g) * kHeadDim + ch * 8);
    *reinterpret_cast<u32x4*>(S.kst + r * 256 + ((ch ^ (r & 15)) << 4)) = v;
  }
  stage_kidx(S, k_idx, key0, nvalid, true);

  // the teacher's inputs of the wave's queries TQ*w ..
  constexpr int TQ = kSub2 / 8;
  struct TeachIn {
    int ent[TQ];
    bf16x8 qop[TQ][4];
    f32x4 lh[TQ];
  };
  auto load_teach = [&](TeachIn& t, int at, int nsub) {
#pragma unroll
    for (int h = 0; h < TQ; ++h) {
      const int tq = TQ * wave + h;
      t.ent[h] = -1;
      if (tq < nsub) {
        const int ent = entries[at + tq];
        t.ent[h] = ent;
        const int i_rel = ent >> 4;
        const uint16_t* qrow = q + ((int64_t)i_rel * Hq + g * kHpg + c) * kHeadDim + 8 * qd;
#pragma unroll
        for (int st = 0; st < 4; ++st) t.qop[h][st] = as_bf16x8(ld16(qrow + 32 * st));
        t.lh[h] = *reinterpret_cast<const f32x4*>(lse + (int64_t)i_rel * Hq + g * kHpg + 4 * qd);
      }
    }
  };
  SubMeta cur, nxt;
  TeachIn tc, tn;
  load_meta<true, kSub2>(cur, entries, q_idx, lse_idx, begin, min(kSub2, len), G, g);
  load_teach(tc, begin, min(kSub2, len));

  f32x4 dk_acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) dk_acc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int s0 = 0; s0 < len; s0 += kSub2) {
    const int nsub = min(kSub2, len - s0);
    store_meta<kSub2>(S, cur, row0, key0, G, g, topk);
    // the next sub-tile's inputs stream in while this one is computed
    if (s0 + kSub2 < len) {
      load_meta<true, kSub2>(nxt, entries, q_idx, lse_idx, begin + s0 + kSub2, min(kSub2, len - s0 - kSub2), G, g);
      load_teach(tn, begin + s0 + kSub2, min(kSub2, len - s0 - kSub2));
    }
    if (s0 == 0) lds_barrier();  // K staged
    // teacher of the wave's queries: S = Q K^T per key tile (lane: key c, heads
    // 4qd .. 4qd+3; each K operand serves all of them), P_main = mean over the
    // 16 heads of exp(z - lse)
    {
      const float l2e = 1.4426950408889634f;
      int lm[TQ];
      f32x4 lh[TQ];
      int nq = 0;  // valid queries of the wave (a prefix; wave-uniform)
#pragma unroll
      for (int h = 0; h < TQ; ++h) {
        lm[h] = tc.ent[h] < 0 ? -1 : (int)min<int64_t>(kBlock - 1, row0 + (tc.ent[h] >> 4) - key0);
        lh[h] = tc.lh[h] * l2e;
        nq += tc.ent[h] >= 0;
      }
      // key tiles software-pipelined: the MFMAs of tile t+1 are issued between
      // the exponentials of tile t (their K operands read one tile ahead)
      f32x4 sm[2][TQ];
      bf16x8 kb[2][4];
      auto read_k = [&](bf16x8 (&dst)[4], int t) {
        const int kk = 16 * t + c;
#pragma unroll
        for (int st = 0; st < 4; ++st)
          dst[st] = as_bf16x8(*reinterpret_cast<const u32x4*>(S.kst + kk * 256 + (((4 * st + qd) ^ c) << 4)));
      };
      auto qk = [&](f32x4 (&dst)[TQ], const bf16x8 (&kop)[4]) {
#pragma unroll
        for (int h = 0; h < TQ; ++h) dst[h] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int h = 0; h < TQ; ++h)
            if (h < nq) dst[h] = mfma16x16x32(tc.qop[h][st], kop[st], dst[h]);
      };
      read_k(kb[0], 0);
      qk(sm[0], kb[0]);
      read_k(kb[1], 1);
      static_for<0, 8>([&](auto it) {
        constexpr int t = decltype(it)::value;
        if constexpr (t + 2 < 8) read_k(kb[t & 1], t + 2);
        if constexpr (t + 1 < 8) qk(sm[(t + 1) & 1], kb[(t + 1) & 1]);
        const int kk = 16 * t + c;
#pragma unroll
        for (int h = 0; h < TQ; ++h) {
          float p = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            p += __builtin_amdgcn_exp2f(__builtin_fmaf(sm[t & 1][h][r], scale_log2, -lh[h][r]));
          p = sum_lane_groups(p);
          if (qd == 0) S.pbuf[kk][TQ * wave + h] = kk <= lm[h] ? p * (1.0f / kHpg) : 0.f;
        }
        constexpr int nm = t + 1 < 8 ? 4 * TQ : 0, nd = t + 2 < 8 ? 4 : 0;
        kl_sched_region<nm, TQ * 14, nd>();
      });
    }
    lds_barrier();  // the sub-tile's queries and teacher ready

    // index part: wave w, keys kw .. kw+15, queries in column blocks of 16
    constexpr int NJ = kSub2 / 16;
    float loss[NJ];
    f32x4 dq[NJ][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      f32x4 sa, sb;
      index_scores_tile(S, kw, j, sa, sb);
      // gs in layout a (lane: key kw + c, queries 16j + 4qd + r) and b (lane:
      // query 16j + c, keys kw + 4qd + r); the loss terms in layout b
      float ga[4], gb[4];
      float ls = 0.f;
      {
        const f32x4 pm4 = *reinterpret_cast<const f32x4*>(&S.pbuf[kw + c][16 * j + 4 * qd]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = 16 * j + 4 * qd + r;
          ga[r] = kw + c <= S.lim[n] ? __expf(sa[r] - S.lz[n]) - pm4[r] : 0.f;
        }
        const int n = 16 * j + c;
        const int lm = S.lim[n];
        const float lzc = S.lz[n];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = kw + 4 * qd + r;
          const float pm = S.pbuf[kk][n];
          const float lp = sb[r] - lzc;
          const bool in_t = kk <= lm;
          gb[r] = in_t ? __expf(lp) - pm : 0.f;
          if (in_t && pm > 0.f) ls += pm * (__logf(pm) - lp);
        }
      }
      loss[j] = sum_lane_groups(ls);
      kl_i16x4 gah, gal, gbh, gbl;
      split_bf16(ga, gah, gal);
      split_bf16(gb, gbh, gbl);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        // dk^T[16dt + i][key] += sum_n q_idx[n][16dt + i] G[n][key]
        const kl_i16x4 qa = *reinterpret_cast<const kl_i16x4*>(&S.qibT[16 * dt + c][16 * j + 4 * qd]);
        dk_acc[dt] = kl_mfma16(qa, gah, dk_acc[dt]);
        dk_acc[dt] = kl_mfma16(qa, gal, dk_acc[dt]);
        // dq^T[16dt + i][query] = sum over the wave's keys of k_idx[key][16dt + i] G^T[key][query]
        const kl_i16x4 ka = *reinterpret_cast<const kl_i16x4*>(S.istT + (16 * dt + c) * kTStride + (kw + 4 * qd) * 2);
        dq[j][dt] = kl_mfma16(ka, gbh, (f32x4){0.f, 0.f, 0.f, 0.f});
        dq[j][dt] = kl_mfma16(ka, gbl, dq[j][dt]);
      }
    }
    if (qd == 0) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) S.lossb[wave][16 * j + c] = loss[j];
    }
    // dq over the 8 key tiles in a fixed order: waves 0-3 store, waves 4-7 add
    // theirs (tile w + (w - 4)), then one thread per (query, dim) sums the four
    if (wave < 4) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) S.red[wave][16 * dt + 4 * qd + r][16 * j + c] = dq[j][dt][r];
    }
    lds_barrier();
    if (wave >= 4) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) S.red[wave - 4][16 * dt + 4 * qd + r][16 * j + c] += dq[j][dt][r];
    }
    lds_barrier();
    for (int x = tid; x < kSub2 * kIndexDim; x += 512) {
      const int n = x >> 6, d = x & 63;
      if (n < nsub)
        dq_part[(int64_t)S.slot[n] * kIndexDim + d] = (S.red[0][d][n] + S.red[1][d][n]) + (S.red[2][d][n] + S.red[3][d][n]);
    }
    if (tid < nsub) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) v += S.lossb[w][tid];
      loss_part[S.slot[tid]] = v;
    }
    lds_barrier();  // before the next sub-tile overwrites the buffers
    cur = nxt;
    tc = tn;
  }
  // the chunk's dk_idx rows [128 keys][64]: lane (key kw + c, qd) holds dims
  // 16dt + 4qd .. +3
  float* dst = dk_part + (int64_t)t_id * kBlock * kIndexDim + (kw + c) * kIndexDim + 4 * qd;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = dk_acc[dt];
}

// dk_idx of key block b (eight workgroups per block, an eighth of its rows each): the chunk partials of every
// group's list for b, added in (group, chunk) order to the rows' running sums
__global__ __launch_bounds__(256) void k_kl_dk(const float* __restrict__ dk_part, const int32_t* __restrict__ tile_start,
                                               float* __restrict__ dk_idx, int64_t n_tokens, int nbw, int G) {
  const int b = blockIdx.x;
  const int64_t key0 = (int64_t)b * kBlock;
  const int nvalid = (int)min<int64_t>(kBlock, n_tokens - key0);
  constexpr int kPer = kBlock * kIndexDim / 4 / 8;  // f32x4 of the workgroup's eighth
  for (int x = blockIdx.y * kPer + threadIdx.x; x < (blockIdx.y + 1) * kPer; x += blockDim.x) {
    const int kk = (x * 4) / kIndexDim;
    if (kk >= nvalid) continue;
    f32x4 acc = *reinterpret_cast<const f32x4*>(dk_idx + key0 * kIndexDim + x * 4);
    for (int g = 0; g < G; ++g) {
      const int t0 = tile_start[g * nbw + b], t1 = tile_start[g * nbw + b + 1];
      // eight chunk partials in flight at a time, added in chunk order
      for (int t = t0; t < t1; t += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = t + u < t1 ? *reinterpret_cast<const f32x4*>(dk_part + (int64_t)(t + u) * kBlock * kIndexDim + x * 4)
                            : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (t + u < t1) acc = acc + v[u];
      }
    }
    *reinterpret_cast<f32x4*>(dk_idx + key0 * kIndexDim + x * 4) = acc;
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
  // every slot's loads are issued before the sums, which run in slot order
  float dv[kMaxTopk], lv[kMaxTopk];
#pragma unroll
  for (int u = 0; u < kMaxTopk; ++u) {
    dv[u] = u < nsel ? dq_part[(x * topk + u) * kIndexDim + lane] : 0.f;
    lv[u] = u < nsel ? loss_part[x * topk + u] : 0.f;
  }
  float d = 0.f, l = 0.f;
#pragma unroll
  for (int u = 0; u < kMaxTopk; ++u) {
    if (u < nsel) {
      d += dv[u];
      l += lv[u];
    }
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
  hipLaunchKernelGGL(k_kl_norm, dim3(a.chunk_cap), dim3(512), 0, st, a.q_idx, a.k_idx, a.entries, a.chunks,
                     a.chunk_info, a.part_m, a.part_l, a.n_tokens, a.row0, a.G, a.topk);
  const int64_t rows = (int64_t)a.nrows * a.G;
  hipLaunchKernelGGL(k_kl_lse, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, a.part_m, a.part_l,
                     a.lse_idx, a.nrows, a.row0, a.G, a.topk);
  hipLaunchKernelGGL(k_kl_grad, dim3(a.chunk_cap), dim3(512), 0, st, a.q, a.k, a.q_idx, a.k_idx, a.lse, a.lse_idx,
                     a.entries, a.chunks, a.chunk_info, a.loss_part, a.dq_part, a.dk_part, a.n_tokens, a.row0, a.G,
                     a.topk, a.scale_log2);
  hipLaunchKernelGGL(k_kl_dk, dim3(a.nbw, 8), dim3(256), 0, st, a.dk_part, a.tile_start, a.dk_idx, a.n_tokens, a.nbw,
                     a.G);
  hipLaunchKernelGGL(k_kl_out, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a.loss_part, a.dq_part,
                     a.loss, a.dq_idx, a.nrows, a.row0, a.n_tokens, a.G, a.topk);
}

void launch_zero_f32(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
}

}  // namespace msa
