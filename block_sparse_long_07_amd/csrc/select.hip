// Exp-free top-k block selection with the forced local block [pnsm, section 7;
// yhxrc, 二].
//
// Each index row (query i or decode sequence, group g) keeps the local block
// b_loc plus the k-1 best older blocks by pooled raw score, ties to the lower
// block index. Softmax preserves the order of the scores, so no max/exp/sum is
// evaluated; the specialised small-k register top-k follows the pages' kernel
// choice of a per-thread register list for small k [pnsm, section 7].
//
// Many rows (prefill): 16 lanes per row, 4 rows per wave. Lane s of a row
// ranks the candidates b = s, s+16, ... < b_loc in ascending order and keeps
// its best k-1 (score, index) pairs in registers, sorted by (score descending,
// index ascending): a candidate enters only if it is strictly greater than
// the current (k-1)-th score and is placed after every equal score, so among
// equal scores the lowest indices are kept. The 16 lane lists of a row are
// then merged by k-1 rounds of a row-wide arg-max over the list heads (a DPP
// butterfly inside the 16-lane row; ties to the lower index), the winning lane
// popping its head. The chosen indices are sorted ascending and written with
// b_loc last and -1 padding.
#include <utility>

#include "msa_device.h"
#include "msa_launch.h"
#include "topk_row.h"

namespace msa {

constexpr int64_t kWaveRowsMax = 16384;

template <int KM1>
__global__ __launch_bounds__(256) void k_select(const float* __restrict__ sblk, int nb,
                                                int32_t* __restrict__ sel, int64_t sel_gstride,
                                                int64_t sel_rstride, int64_t nrows, int G, int64_t row0,
                                                const int32_t* __restrict__ ctx_lens, int bk_shift) {
  const int s = threadIdx.x & 15;
  const int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const bool valid = r < nrows * G;
  const int64_t rr = valid ? r / G : 0;
  const int g = valid ? (int)(r % G) : 0;
  int b_loc = 0;
  if (valid) b_loc = ctx_lens ? (ctx_lens[rr] - 1) >> bk_shift : (int)((row0 + rr) >> bk_shift);
  // candidates this row must rank (0 when every older block is taken anyway)
  const int need = (KM1 > 0 && valid && b_loc > KM1) ? b_loc : 0;

  float v[KM1 > 0 ? KM1 : 1];
  int id[KM1 > 0 ? KM1 : 1];
#pragma unroll
  for (int t = 0; t < KM1; ++t) {
    v[t] = -__builtin_inff();
    id[t] = 0x7fffffff;
  }
  if constexpr (KM1 > 0) {
    const float* row = sblk + r * (int64_t)nb;
    // Insert before the first strictly smaller score; from there on every
    // element shifts down one place (the displaced ones keep their order, so
    // equal scores stay in ascending index order).
    auto insert = [&](float cv, int ci) {
      bool shift = false;
#pragma unroll
      for (int t = 0; t < KM1; ++t) {
        shift |= cv > v[t];
        const float nv = shift ? cv : v[t];
        const int ni = shift ? ci : id[t];
        cv = shift ? v[t] : cv;
        ci = shift ? id[t] : ci;
        v[t] = nv;
        id[t] = ni;
      }
    };
    // Long rows (k = 16, at least kFloorMin candidates in some row of the
    // wave) also keep floor: a lower bound of the row's 15th best score so
    // far, the second smallest of the 16 lanes' best scores (15 lanes each
    // hold a score >= it, so no score strictly below it can be among the
    // row's 15 best; equal scores still go through the lane's own rule). Most
    // of their candidates then fail one compare instead of costing the wave a
    // list insertion, which bounds this loop (without insertions it streams
    // at the HBM rate); on shorter rows the exchange costs more than it
    // saves. That loop runs while any lane of the wave has candidates left,
    // so that every lane takes part in every exchange (a lane reading a
    // disabled lane gets its own value back).
    constexpr int kFloorMin = 2048;
    if (KM1 == 15 && __any(need >= kFloorMin)) {
      float floor_v = -__builtin_inff();
      for (int b0 = s; __any(b0 < need); b0 += 64) {
        float cvs[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) cvs[q] = (b0 + 16 * q < need) ? row[b0 + 16 * q] : -__builtin_inff();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool ins = (cvs[q] > v[KM1 - 1]) & (cvs[q] >= floor_v);
          if (__any(ins) && ins) insert(cvs[q], b0 + 16 * q);  // (skipped by the wave when no lane needs it)
        }
        floor_v = second_min_row16(v[0]);
      }
    } else {
      for (int b0 = s; b0 < need; b0 += 64) {
        // four candidates per lane per step: the loads are issued together
        float cvs[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) cvs[q] = (b0 + 16 * q < need) ? row[b0 + 16 * q] : -__builtin_inff();
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (cvs[q] > v[KM1 - 1]) insert(cvs[q], b0 + 16 * q);
      }
    }
  }
  if (!valid) return;  // whole 16-lane rows leave together
  if (b_loc <= KM1) {  // every block 0..b_loc is selected
    if (s <= KM1) sel[(int64_t)g * sel_gstride + rr * sel_rstride + s] = (s <= b_loc) ? s : -1;
    return;
  }
  if constexpr (KM1 == 0) {  // k = 1: the local block alone
    if (s == 0) sel[(int64_t)g * sel_gstride + rr * sel_rstride] = b_loc;
  } else {
    int chosen[KM1];
#pragma unroll
    for (int rd = 0; rd < KM1; ++rd) {
      // arg-max of the heads over the row
      float bv = v[0];
      int bi = id[0];
      argmax_row16(bv, bi);
      chosen[rd] = bi;
      if (id[0] == bi) {  // the winning lane pops its head
#pragma unroll
        for (int t = 0; t + 1 < KM1; ++t) {
          v[t] = v[t + 1];
          id[t] = id[t + 1];
        }
        v[KM1 - 1] = -__builtin_inff();
        id[KM1 - 1] = 0x7fffffff;
      }
    }
    // ascending block ids (bubble network over the k-1 chosen indices)
#pragma unroll
    for (int a = 0; a < KM1; ++a) {
#pragma unroll
      for (int t = 0; t + 1 < KM1 - a; ++t) {
        const int lo = min(chosen[t], chosen[t + 1]);
        const int hi = max(chosen[t], chosen[t + 1]);
        chosen[t] = lo;
        chosen[t + 1] = hi;
      }
    }
    // lane s writes slot s (slot k-1 is b_loc)
    int mine = b_loc;
#pragma unroll
    for (int u = 0; u < KM1; ++u) mine = (s == u) ? chosen[u] : mine;
    if (s <= KM1) sel[(int64_t)g * sel_gstride + rr * sel_rstride + s] = mine;
  }
}

// Few rows with many candidates (decode): one wave per row. Lane l ranks the
// candidates b = l, l+64, ... (ascending, so the same register insertion keeps
// its k-1 best with ties to the lower index); the 64 lane lists are then merged
// by k-1 rounds of a wave-wide arg-max over the list heads (a DPP butterfly
// within 16-lane rows, then v_permlane16/32 swaps across rows), each round
// popping the winner's head.
template <int KM1>
__global__ __launch_bounds__(64) void k_select_wave(const float* __restrict__ sblk, int nb,
                                                    int32_t* __restrict__ sel, int64_t sel_gstride,
                                                    int64_t sel_rstride, int G, int64_t row0,
                                                    const int32_t* __restrict__ ctx_lens, int bk_shift) {
  const int lane = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int64_t rr = r / G;
  const int g = (int)(r % G);
  const int b_loc = ctx_lens ? (ctx_lens[rr] - 1) >> bk_shift : (int)((row0 + rr) >> bk_shift);
  int32_t* out = sel + (int64_t)g * sel_gstride + rr * sel_rstride;
  if (b_loc <= KM1) {
    if (lane <= KM1) out[lane] = (lane <= b_loc) ? lane : -1;
    return;
  }
  if constexpr (KM1 == 0) {
    if (lane == 0) out[0] = b_loc;
  } else {
    float v[KM1];
    int id[KM1];
#pragma unroll
    for (int t = 0; t < KM1; ++t) {
      v[t] = -__builtin_inff();
      id[t] = 0x7fffffff;
    }
    const float* row = sblk + r * (int64_t)nb;
    // 16 candidates per lane are loaded before any is ranked, so their
    // latencies overlap; they are then inserted in ascending order
    constexpr int kBatch = 16;
    for (int b0 = lane; b0 < b_loc; b0 += 64 * kBatch) {
      float cand[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) cand[u] = b0 + 64 * u < b_loc ? row[b0 + 64 * u] : -__builtin_inff();
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        float cv = cand[u];
        if (b0 + 64 * u < b_loc && cv > v[KM1 - 1]) {
          int ci = b0 + 64 * u;
          bool shift = false;
#pragma unroll
          for (int t = 0; t < KM1; ++t) {
            shift |= cv > v[t];
            const float nv = shift ? cv : v[t];
            const int ni = shift ? ci : id[t];
            cv = shift ? v[t] : cv;
            ci = shift ? id[t] : ci;
            v[t] = nv;
            id[t] = ni;
          }
        }
      }
    }
    int chosen[KM1];
#pragma unroll
    for (int rd = 0; rd < KM1; ++rd) {
      // wave-wide arg-max: DPP butterfly inside 16-lane rows, then lane swaps
      // across rows, all without LDS traffic
      float bv = v[0];
      int bi = id[0];
      argmax_row16(bv, bi);
      argmax_rows(bv, bi);
      chosen[rd] = bi;
      if (id[0] == bi) {  // the winning lane pops its head
#pragma unroll
        for (int t = 0; t + 1 < KM1; ++t) {
          v[t] = v[t + 1];
          id[t] = id[t + 1];
        }
        v[KM1 - 1] = -__builtin_inff();
        id[KM1 - 1] = 0x7fffffff;
      }
    }
#pragma unroll
    for (int a = 0; a < KM1; ++a) {
#pragma unroll
      for (int t = 0; t + 1 < KM1 - a; ++t) {
        const int lo = min(chosen[t], chosen[t + 1]);
        const int hi = max(chosen[t], chosen[t + 1]);
        chosen[t] = lo;
        chosen[t + 1] = hi;
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < KM1; ++u) out[u] = chosen[u];
      out[KM1] = b_loc;
    }
  }
}

// Few rows with very many candidates (long contexts): NW waves per row,
// ranked by select_row_rt (each wave's best k-1, then the row's best k-1
// among the NW*(k-1) survivors, which do not arrive in index order and are
// therefore compared by score and index in full).
template <int KM1, int NW>
__global__ __launch_bounds__(64 * NW) void k_select_multi(const float* __restrict__ sblk, int nb,
                                                          int32_t* __restrict__ sel, int64_t sel_gstride,
                                                          int64_t sel_rstride, int G, int64_t row0,
                                                          const int32_t* __restrict__ ctx_lens, int bk_shift) {
  static_assert(KM1 > 0, "k >= 2");
  __shared__ float sv[NW * (kMaxTopk - 1)];
  __shared__ int si[NW * (kMaxTopk - 1)];
  __shared__ int picks[kMaxTopk];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = blockIdx.x;
  const int64_t rr = r / G;
  const int g = (int)(r % G);
  const int b_loc = ctx_lens ? (ctx_lens[rr] - 1) >> bk_shift : (int)((row0 + rr) >> bk_shift);
  int32_t* out = sel + (int64_t)g * sel_gstride + rr * sel_rstride;
  if (b_loc <= KM1) {  // every block 0..b_loc is selected (uniform over the workgroup)
    if (wave == 0 && lane <= KM1) out[lane] = (lane <= b_loc) ? lane : -1;
    return;
  }
  select_row_rt<NW>(sblk + r * (int64_t)nb, b_loc, KM1, sv, si, picks);
  if (wave != 0) return;
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's picks are in LDS
  __builtin_amdgcn_wave_barrier();
  if (lane < KM1) out[lane] = picks[lane];
  if (lane == 0) out[KM1] = b_loc;
}

void launch_select(const LaunchSelect& a, hipStream_t st) {
  const int64_t rows = a.nrows * a.G;
  if (rows <= 0) return;
  // few rows: a wave per row (16 waves per row when the rows are long: at
  // 8 x 1M decode 53 -> ~10 us; 4 waves at 1024 candidates measured a few us
  // slower than one); many rows: 16 lanes per row (4 rows per wave)
  const bool per_wave = rows <= kWaveRowsMax;
  const int nw = !per_wave || a.topk < 2 ? 1 : a.nb >= 4096 ? 16 : 1;
  dim3 grid((unsigned)(per_wave ? rows : (rows + 15) / 16));
#define MSA_SEL_MULTI(K)                                                                                \
  hipLaunchKernelGGL((k_select_multi<K - 1, 16>), grid, dim3(1024), 0, st, a.sblk, a.nb, a.sel,         \
                     a.sel_gstride, a.sel_rstride, a.G, a.row0, a.ctx_lens, a.bk_shift);
#define MSA_SEL_CASE(K)                                                                                 \
  case K:                                                                                               \
    if (per_wave && nw > 1) {                                                                           \
      if constexpr (K > 1) { MSA_SEL_MULTI(K) }                                                         \
    } else if (per_wave) {                                                                              \
      hipLaunchKernelGGL(k_select_wave<K - 1>, grid, dim3(64), 0, st, a.sblk, a.nb, a.sel,              \
                         a.sel_gstride, a.sel_rstride, a.G, a.row0, a.ctx_lens, a.bk_shift);            \
    } else {                                                                                            \
      hipLaunchKernelGGL(k_select<K - 1>, grid, dim3(256), 0, st, a.sblk, a.nb, a.sel, a.sel_gstride,   \
                         a.sel_rstride, a.nrows, a.G, a.row0, a.ctx_lens, a.bk_shift);                  \
    }                                                                                                   \
    break;
  switch (a.topk) {
    MSA_SEL_CASE(1)
    MSA_SEL_CASE(2)
    MSA_SEL_CASE(3)
    MSA_SEL_CASE(4)
    MSA_SEL_CASE(5)
    MSA_SEL_CASE(6)
    MSA_SEL_CASE(7)
    MSA_SEL_CASE(8)
    MSA_SEL_CASE(9)
    MSA_SEL_CASE(10)
    MSA_SEL_CASE(11)
    MSA_SEL_CASE(12)
    MSA_SEL_CASE(13)
    MSA_SEL_CASE(14)
    MSA_SEL_CASE(15)
    MSA_SEL_CASE(16)
    default: break;
  }
#undef MSA_SEL_CASE
#undef MSA_SEL_MULTI
}

}  // namespace msa
