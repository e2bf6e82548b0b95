// Wave-level arg-max and top-k building blocks of the block selection
// (exp-free: the order of the raw pooled scores decides [pnsm, section 7]),
// shared by the selection kernels and the decode attention kernel, which
// ranks its own row. Order: score descending, block index ascending.
#pragma once

#include "msa_device.h"

namespace msa {

// One step of a symmetric arg-max butterfly inside 16-lane rows: lane i meets
// lane xor 1 (step 0), xor 2 (1), 7-i within its 8-lane half (2), 15-i (3),
// all DPP moves; after the four steps every lane of the row holds the row's
// best (score desc, index asc).
template <int STEP>
__device__ __forceinline__ void argmax_step(float& bv, int& bi) {
  constexpr int ctrl = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(bv), __float_as_int(bv), ctrl, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(bi, bi, ctrl, 0xF, 0xF, false);
  // bitwise, not short-circuit: the compares combine as lane masks with no
  // branches (a short-circuit form compiles to exec-mask branches per step)
  const bool take = (ov > bv) | ((ov == bv) & (oi < bi));
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}
__device__ __forceinline__ void argmax_row16(float& bv, int& bi) {
  argmax_step<0>(bv, bi);
  argmax_step<1>(bv, bi);
  argmax_step<2>(bv, bi);
  argmax_step<3>(bv, bi);
}
// across the four rows of a wave: v_permlane16_swap / v_permlane32_swap hand
// each lane its partner's pair (lane xor 16, then xor 32)
__device__ __forceinline__ void argmax_rows(float& bv, int& bi) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const auto sv = h ? __builtin_amdgcn_permlane32_swap(__float_as_uint(bv), __float_as_uint(bv), false, false)
                      : __builtin_amdgcn_permlane16_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
    const auto si = h ? __builtin_amdgcn_permlane32_swap((unsigned)bi, (unsigned)bi, false, false)
                      : __builtin_amdgcn_permlane16_swap((unsigned)bi, (unsigned)bi, false, false);
    const float v0 = __uint_as_float(sv[0]), v1 = __uint_as_float(sv[1]);
    const int i0 = (int)si[0], i1 = (int)si[1];
    const bool take1 = (v1 > v0) | ((v1 == v0) & (i1 < i0));
    bv = take1 ? v1 : v0;
    bi = take1 ? i1 : i0;
  }
}

// The second smallest of x over the 16 lanes of each 16-lane row, in every
// lane of the row: the butterfly of argmax_row16 over (smallest, second
// smallest) pairs (two disjoint sets' pairs merge into the union's).
template <int STEP>
__device__ __forceinline__ void min2_step(float& m1, float& m2) {
  constexpr int ctrl = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
  const float o1 = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(m1), __float_as_int(m1), ctrl, 0xF, 0xF, false));
  const float o2 = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(m2), __float_as_int(m2), ctrl, 0xF, 0xF, false));
  const float lo = fminf(m1, o1), hi = fmaxf(m1, o1);
  m2 = fminf(hi, fminf(m2, o2));
  m1 = lo;
}
__device__ __forceinline__ float second_min_row16(float x) {
  float m1 = x, m2 = __builtin_inff();
  min2_step<0>(m1, m2);
  min2_step<1>(m1, m2);
  min2_step<2>(m1, m2);
  min2_step<3>(m1, m2);
  return m2;
}

// (score, index) a precedes b: higher score, or equal score and lower index
__device__ __forceinline__ bool before(float av, int ai, float bv, int bi) {
  return (av > bv) | ((av == bv) & (ai < bi));
}

// Sorted list of a lane's best L candidates (score desc, index asc). `cv`,
// `ci` enters if it precedes the last entry; everything from its place on
// shifts down one slot (so among equal scores the lower indices stay first).
template <int L>
__device__ __forceinline__ void list_insert(float (&v)[L], int (&id)[L], float cv, int ci) {
  if (!before(cv, ci, v[L - 1], id[L - 1])) return;
  bool shift = false;
#pragma unroll
  for (int t = 0; t < L; ++t) {
    shift |= before(cv, ci, v[t], id[t]);
    const float nv = shift ? cv : v[t];
    const int ni = shift ? ci : id[t];
    cv = shift ? v[t] : cv;
    ci = shift ? id[t] : ci;
    v[t] = nv;
    id[t] = ni;
  }
}
// The same for candidates that arrive in ascending index order: a strictly
// greater score enters (placed after every equal one), which keeps the lower
// indices among equal scores with one compare per slot.
template <int L>
__device__ __forceinline__ void list_insert_asc(float (&v)[L], int (&id)[L], float cv, int ci) {
  if (!(cv > v[L - 1])) return;
  bool shift = false;
#pragma unroll
  for (int t = 0; t < L; ++t) {
    shift |= cv > v[t];
    const float nv = shift ? cv : v[t];
    const int ni = shift ? ci : id[t];
    cv = shift ? v[t] : cv;
    ci = shift ? id[t] : ci;
    v[t] = nv;
    id[t] = ni;
  }
}
// the lane holding the winner `bi` pops its head
template <int L>
__device__ __forceinline__ void list_pop_if(float (&v)[L], int (&id)[L], int bi) {
  if (id[0] == bi) {
#pragma unroll
    for (int t = 0; t + 1 < L; ++t) {
      v[t] = v[t + 1];
      id[t] = id[t + 1];
    }
    v[L - 1] = -__builtin_inff();
    id[L - 1] = 0x7fffffff;
  }
}
template <int L>
__device__ __forceinline__ void list_clear(float (&v)[L], int (&id)[L]) {
#pragma unroll
  for (int t = 0; t < L; ++t) {
    v[t] = -__builtin_inff();
    id[t] = 0x7fffffff;
  }
}

// The best km1 (<= kMaxTopk - 1) of the candidates row[0 .. b_loc-1] by the NW
// waves of the calling workgroup (every thread of the workgroup calls; it has
// exactly NW waves). Lane l of wave w ranks the candidates w*64 + l + 64*NW*j
// into a register list of its best kMaxTopk-1; km1 rounds of a wave-wide
// arg-max pop each wave's best km1 into LDS (sv, si: NW * (kMaxTopk-1)
// entries); wave 0 then ranks the NW*km1 survivors the same way (the row's
// best km1 are among them: each wave kept its subset's best) and pops the
// row's best km1, writing their block ids to out[0 .. km1-1] (LDS) in
// ascending order. One workgroup barrier (LDS only) inside; out is complete for wave 0
// on return (other waves read it after a barrier of their own). after_loads()
// runs in every wave once the candidates are read.
template <int NW, class F = void (*)()>
__device__ __forceinline__ void select_row_rt(const float* __restrict__ row, int b_loc, int km1, float* sv,
                                              int* si, int* out, F after_loads = [] {}) {
  constexpr int L = kMaxTopk - 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float v[L];
  int id[L];
  list_clear(v, id);
  constexpr int kBatch = 8;
  constexpr int kStride = 64 * NW;
  for (int b0 = wave * 64 + lane; b0 < b_loc; b0 += kStride * kBatch) {
    float cand[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) cand[u] = b0 + kStride * u < b_loc ? row[b0 + kStride * u] : 0.f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (b0 + kStride * u < b_loc) list_insert_asc(v, id, cand[u], b0 + kStride * u);
  }
  after_loads();
  for (int rd = 0; rd < km1; ++rd) {
    float bv = v[0];
    int bi = id[0];
    argmax_row16(bv, bi);
    argmax_rows(bv, bi);
    if (lane == 0) {
      sv[wave * L + rd] = bv;
      si[wave * L + rd] = bi;
    }
    list_pop_if(v, id, bi);
  }
  lds_barrier();
  if (wave != 0) return;
  // the survivors (wave w's rd-th best at w*L + rd, rd < km1) into wave 0's
  // lane lists, then km1 rounds over the list heads
  list_clear(v, id);
  for (int j = lane; j < NW * L; j += 64)
    if (j % L < km1) list_insert(v, id, sv[j], si[j]);
  int pick = 0;  // lane r < km1: the r-th pick
  for (int r = 0; r < km1; ++r) {
    float bv = v[0];
    int bi = id[0];
    argmax_row16(bv, bi);
    argmax_rows(bv, bi);
    if (lane == r) pick = bi;
    list_pop_if(v, id, bi);
  }
  // ascending: lane r < km1 ranks its pick among all picks
  int rank = 0;
  for (int j = 0; j < km1; ++j) rank += __builtin_amdgcn_readlane(pick, j) < pick;
  if (lane < km1) out[rank] = pick;
}

// Exact top km1 of the candidates row[0 .. b_loc-1] (score descending, index
// ascending) by a threshold search over the workgroup's NW waves, C
// candidates per lane (b_loc <= 64*NW*C): candidate b = (j*NW + w)*64 + l
// sits in slot j of lane l of wave w, as the order-preserving image of its
// score (-0 folded onto +0; 0 for no candidate, below every score). T, the
// km1-th largest image, is found bit by bit from the top (the largest t with
// at least km1 images >= t), each count a sum of ballot popcounts over the
// slots and, across waves, through LDS (cnt: 2*NW ints). Every image above T
// is taken; if more than km1 images reach T, the ties at T go by index: X,
// the (km1 - #above)-th tie in index order, is found the same way over the
// index bits. The picks are gathered in LDS (tmp: kMaxTopk ints, ctr: one
// int) and wave 0 writes them to out[0 .. km1-1] in ascending order. Every
// thread of the workgroup calls (NW is 1 or the workgroup's wave count; with
// NW = 1 the search has no barrier); out is complete for wave 0 on return.
// after_loads() runs in every wave once the candidates are read (for the
// caller's own memory traffic, which then overlaps the ranking).
template <int NW, int C, class F = void (*)()>
__device__ __forceinline__ void select_row_thr(const float* __restrict__ row, int b_loc, int km1, int* cnt,
                                               int* tmp, int* ctr, int* out, F after_loads = [] {}) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave >= NW) {  // (NW = 1: wave 0 ranks alone, the others wait)
    after_loads();
    lds_barrier();
    return;
  }
  uint32_t key[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int b = (j * NW + wave) * 64 + lane;
    key[j] = b < b_loc ? ord_f32(row[b] + 0.0f) : 0u;
  }
  after_loads();
  if (threadIdx.x == 0) *ctr = 0;
  int it = 0;
  // number of candidates over the workgroup whose slot passes `pred`
  auto total = [&](auto pred) -> int {
    int c = 0;
#pragma unroll
    for (int j = 0; j < C; ++j) c += __builtin_popcountll(__ballot(pred(j)));
    if constexpr (NW == 1) return c;
    int* slot = cnt + (it++ & 1) * NW;
    if (lane == 0) slot[wave] = c;
    lds_barrier();  // (the other half of cnt is free: every wave has read it before this barrier)
    int sum = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += slot[w];
    return sum;
  };
  uint32_t T = 0;
  int n_ge = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t t = T | (1u << bit);
    const int n = total([&](int j) { return key[j] >= t; });
    if (n >= km1) {
      T = t;
      n_ge = n;
    }
  }
  // ties at T: the first (km1 - #above) by index
  int X = 0x7fffffff;
  if (n_ge > km1) {
    const int n_gt = total([&](int j) { return key[j] > T; });
    const int need = km1 - n_gt;
    X = 0;  // the largest X with fewer than `need` ties below index X
    for (int bit = 20; bit >= 0; --bit) {
      const int x = X | (1 << bit);
      const int n = total([&](int j) { return key[j] == T && (j * NW + wave) * 64 + lane < x; });
      if (n < need) X = x;
    }
  }
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int b = (j * NW + wave) * 64 + lane;
    if (key[j] > T || (key[j] == T && b <= X)) tmp[atomicAdd(ctr, 1)] = b;
  }
  lds_barrier();
  if (wave != 0) return;
  // ascending: lane r < km1 ranks pick r among the picks
  if (lane < km1) {
    const int x = tmp[lane];
    int rank = 0;
    for (int j = 0; j < km1; ++j) rank += tmp[j] < x;
    out[rank] = x;
  }
}

}  // namespace msa
