// Exp-free top-k block selection with the forced local block [pnsm, section 7;
// yhxrc, 二].
//
// Each index row (query i or decode sequence, group g) keeps the local block
// b_loc plus the k-1 best older blocks by pooled raw score, ties to the lower
// block index. Softmax preserves the order of the scores, so no max/exp/sum is
// evaluated; the specialised small-k register top-k follows the pages' kernel
// choice of a per-thread register list for small k [pnsm, section 7].
//
// One lane per row: the candidates b = 0..b_loc-1 are streamed in ascending
// order through an LDS tile (64 rows x 64 candidates, loaded coalesced), and
// each lane keeps its row's best k-1 (score, index) pairs in registers, sorted
// by (score descending, index ascending). A candidate enters only if it is
// strictly greater than the current (k-1)-th score and is placed after every
// equal score; since candidates arrive in ascending index order, among equal
// scores the lowest indices are kept. The chosen indices are sorted ascending at the
// end and written with b_loc last and -1 padding.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int64_t kWaveRowsMax = 16384;

template <int KM1>
__global__ __launch_bounds__(64) void k_select(const float* __restrict__ sblk, int nb,
                                               int32_t* __restrict__ sel, int64_t sel_gstride,
                                               int64_t sel_rstride, int64_t nrows, int G, int64_t row0,
                                               const int32_t* __restrict__ ctx_lens) {
  __shared__ float tile[64][65];
  const int lane = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int64_t r = r0 + lane;
  const bool valid = r < nrows * G;
  const int64_t rr = valid ? r / G : 0;
  const int g = valid ? (int)(r % G) : 0;
  int b_loc = 0;
  if (valid) b_loc = ctx_lens ? (ctx_lens[rr] - 1) / kBlock : (int)((row0 + rr) / kBlock);
  // candidates this lane must rank (0 when every older block is taken anyway)
  const int need = (KM1 > 0 && valid && b_loc > KM1) ? b_loc : 0;
  int maxneed = need;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) maxneed = max(maxneed, __shfl_xor(maxneed, m, 64));

  float v[KM1 > 0 ? KM1 : 1];
  int id[KM1 > 0 ? KM1 : 1];
#pragma unroll
  for (int t = 0; t < KM1; ++t) {
    v[t] = -__builtin_inff();
    id[t] = -1;
  }

  for (int c0 = 0; c0 < maxneed; c0 += 64) {
    // cooperative, coalesced staging of 64 rows x 64 candidates
    for (int q = 0; q < 64; ++q) {
      const int need_q = __shfl(need, q, 64);
      const int col = c0 + lane;
      float x = -__builtin_inff();
      if (col < need_q) x = sblk[(r0 + q) * (int64_t)nb + col];
      tile[q][lane] = x;
    }
    __syncthreads();
    const int cnt = min(64, need - c0);
    for (int j = 0; j < 64; ++j) {
      if constexpr (KM1 > 0) {
        float cv = tile[lane][j];
        if (j < cnt && cv > v[KM1 - 1]) {
          int ci = c0 + j;
          // Insert before the first strictly smaller score; from there on every
          // element shifts down one place (the displaced ones keep their order,
          // so equal scores stay in ascending index order).
          bool shift = false;
#pragma unroll
          for (int t = 0; t < KM1; ++t) {
            shift = shift || (cv > v[t]);
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
    __syncthreads();
  }

  if (!valid) return;
  int32_t* out = sel + (int64_t)g * sel_gstride + rr * sel_rstride;
  if (b_loc <= KM1) {
#pragma unroll
    for (int u = 0; u <= KM1; ++u) out[u] = (u <= b_loc) ? u : -1;
    return;
  }
  // ascending block ids (bubble network over the k-1 chosen indices)
#pragma unroll
  for (int a = 0; a < KM1; ++a) {
#pragma unroll
    for (int t = 0; t + 1 < KM1 - a; ++t) {
      const int lo = min(id[t], id[t + 1]);
      const int hi = max(id[t], id[t + 1]);
      id[t] = lo;
      id[t + 1] = hi;
    }
  }
#pragma unroll
  for (int u = 0; u < KM1; ++u) out[u] = id[u];
  out[KM1] = b_loc;
}

// Few rows with many candidates (decode): one wave per row. Lane l ranks the
// candidates b = l, l+64, ... (ascending, so the same register insertion keeps
// its k-1 best with ties to the lower index); the 64 lane lists are then merged
// by k-1 rounds of a wave-wide arg-max over the list heads, each round popping
// the winner's head.
template <int KM1>
__global__ __launch_bounds__(64) void k_select_wave(const float* __restrict__ sblk, int nb,
                                                    int32_t* __restrict__ sel, int64_t sel_gstride,
                                                    int64_t sel_rstride, int G, int64_t row0,
                                                    const int32_t* __restrict__ ctx_lens) {
  const int lane = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int64_t rr = r / G;
  const int g = (int)(r % G);
  const int b_loc = ctx_lens ? (ctx_lens[rr] - 1) / kBlock : (int)((row0 + rr) / kBlock);
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
    for (int b = lane; b < b_loc; b += 64) {
      float cv = row[b];
      if (cv > v[KM1 - 1]) {
        int ci = b;
        bool shift = false;
#pragma unroll
        for (int t = 0; t < KM1; ++t) {
          shift = shift || (cv > v[t]);
          const float nv = shift ? cv : v[t];
          const int ni = shift ? ci : id[t];
          cv = shift ? v[t] : cv;
          ci = shift ? id[t] : ci;
          v[t] = nv;
          id[t] = ni;
        }
      }
    }
    int chosen[KM1];
#pragma unroll
    for (int rd = 0; rd < KM1; ++rd) {
      float bv = v[0];
      int bi = id[0];
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        const bool take = ov > bv || (ov == bv && oi < bi);
        bv = take ? ov : bv;
        bi = take ? oi : bi;
      }
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

void launch_select(const LaunchSelect& a, hipStream_t st) {
  const int64_t rows = a.nrows * a.G;
  if (rows <= 0) return;
  // thread-per-row needs many rows to fill the GPU; below that, wave-per-row
  const bool per_wave = rows <= kWaveRowsMax;
  dim3 grid((unsigned)(per_wave ? rows : (rows + 63) / 64));
#define MSA_SEL_CASE(K)                                                                                 \
  case K:                                                                                               \
    if (per_wave)                                                                                       \
      hipLaunchKernelGGL(k_select_wave<K - 1>, grid, dim3(64), 0, st, a.sblk, a.nb, a.sel,              \
                         a.sel_gstride, a.sel_rstride, a.G, a.row0, a.ctx_lens);                        \
    else                                                                                                \
      hipLaunchKernelGGL(k_select<K - 1>, grid, dim3(64), 0, st, a.sblk, a.nb, a.sel, a.sel_gstride,    \
                         a.sel_rstride, a.nrows, a.G, a.row0, a.ctx_lens);                              \
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
}

}  // namespace msa
