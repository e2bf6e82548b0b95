// Reverse index ("query gather") and tile schedule for the KV-outer main branch
// [pnsm, section 7 and section 9: reverse index, query gather, pre-scheduled
// tile chunking].
//
// The selections of one window of query rows are inverted into, for every
// (group g, KV block b), the list of entries (i_rel << 4 | u) of the queries
// whose slot u selected b, ascending in i. The lists are built without global
// atomics and deterministically:
//   1. per (group, chunk of 64 rows): a 64-bit LDS mask per block marks which
//      rows of the chunk selected it; its popcount is the chunk's count;
//   2. one exclusive scan over counts laid out [g][b][chunk] gives every
//      (g, b, chunk) its output offset (and every list its start);
//   3. the chunk pass is repeated and each entry lands at offset + popcount of
//      the mask bits below its row.
// With the dense pass on, pairs whose 16-row unit selected the block at least
// kDenseMin times are left out: the dense pass computes them (k_csr_count also
// writes its per-unit lists); with it off, every pair is listed. Each list is
// then cut into tiles of at most `tile_q` queries, so a block hit by very many
// queries (a sink-like block) becomes many independent tiles.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kChunk = 64;       // rows per chunk (one 64-bit mask word)
constexpr int kScanTile = 4096;  // elements per scan workgroup (256 threads x 16)
constexpr int kUnit = 16;        // rows per dense unit
static_assert(kDenseMin >= 4 && kUnit * kMaxTopk / kDenseMin <= kDenseMax, "a dense list fits kDenseMax entries");

__device__ __forceinline__ void chunk_masks(const int32_t* __restrict__ sel, int64_t sel_gstride, int topk,
                                            int g, int i0, int nq, int bmax, unsigned long long* mask) {
  for (int b = threadIdx.x; b <= bmax; b += blockDim.x) mask[b] = 0ull;
  __syncthreads();
  const int32_t* s = sel + (int64_t)g * sel_gstride + (int64_t)i0 * topk;
  for (int e = threadIdx.x; e < nq * topk; e += blockDim.x) {
    const int b = s[e];
    if (b >= 0 && b <= bmax) atomicOr(&mask[b], 1ull << (e / topk));
  }
  __syncthreads();
}

// Bits of `m` (rows of the chunk that selected a block) that belong to 16-row
// units computing the block in the dense pass: at least min(kDenseMin, n) of
// the unit's n valid rows selected it. All the unit's rows are set, selecting
// or not (the dense pass masks the others).
__device__ __forceinline__ unsigned long long dense_bits(unsigned long long m, int nq, bool dense) {
  unsigned long long d = 0ull;
  if (!dense) return d;
#pragma unroll
  for (int s = 0; s < kChunk / kUnit; ++s) {
    const int r0 = s * kUnit;
    if (r0 >= nq) break;
    const int n = min(kUnit, nq - r0);
    const unsigned long long full = ((1ull << n) - 1ull) << r0;
    if (__popcll(m & full) >= min(kDenseMin, n)) d |= full;
  }
  return d;
}

__global__ __launch_bounds__(256) void k_csr_count(const int32_t* __restrict__ sel, int64_t sel_gstride,
                                                   int topk, int64_t row0, int nrows, int nbw, int nch,
                                                   int32_t* __restrict__ chunkcnt, int32_t* __restrict__ dense_cnt,
                                                   int32_t* __restrict__ dense_list, int32_t* __restrict__ dense_qmask,
                                                   int32_t* __restrict__ dense_slots, int nunits, bool dense,
                                                   int bk_shift) {
  extern __shared__ unsigned long long mask[];
  __shared__ int cand[kChunk / kUnit][kDenseMax];
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int i0 = chunk * kChunk;
  const int nq = min(kChunk, nrows - i0);
  const int bmax = (int)((row0 + i0 + nq - 1) >> bk_shift);
  chunk_masks(sel, sel_gstride, topk, g, i0, nq, bmax, mask);
  for (int b = threadIdx.x; b < nbw; b += blockDim.x) {
    int cnt = 0;
    if (b <= bmax) {
      const unsigned long long m = mask[b];
      cnt = __popcll(m & ~dense_bits(m, nq, dense));
    }
    chunkcnt[((int64_t)g * nbw + b) * nch + chunk] = cnt;
  }
  if (!dense) return;
  const int32_t* srow0 = sel + (int64_t)g * sel_gstride + (int64_t)i0 * topk;
  // per row: which of its slots the dense pass computes
  if ((int)threadIdx.x < nq) {
    const int t = threadIdx.x;
    int bits = 0;
    for (int u = 0; u < topk; ++u) {
      const int b = srow0[t * topk + u];
      if (b >= 0 && b <= bmax && ((dense_bits(mask[b], nq, true) >> t) & 1ull)) bits |= 1 << u;
    }
    dense_slots[(int64_t)g * nrows + i0 + t] = bits;
  }
  // dense list of each 16-row unit (wave s: unit s of the chunk): the distinct
  // blocks its rows selected often enough, each taken from the first row that
  // selected it, then ranked into ascending order
  const int s = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool active = s * kUnit < nq;
  const int n = active ? min(kUnit, nq - s * kUnit) : 0;
  const unsigned long long full = ((1ull << n) - 1ull) << (s * kUnit);
  int cnt = 0;
  if (active) {
    const int r = lane >> 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = 4 * (lane & 3) + j;
      bool keep = false;
      int b = -1;
      if (r < n && u < topk) {
        b = srow0[(s * kUnit + r) * topk + u];
        if (b >= 0 && b <= bmax) {
          const unsigned long long m = mask[b] & full;
          keep = __popcll(m) >= min(kDenseMin, n) && __builtin_ctzll(m) == s * kUnit + r;
        }
      }
      const unsigned long long bal = __ballot(keep);
      if (keep) cand[s][cnt + __popcll(bal & ((1ull << lane) - 1ull))] = b;
      cnt += __popcll(bal);
    }
  }
  __syncthreads();
  if (active) {
    const int64_t base = ((int64_t)g * nunits + (i0 >> 4) + s) * kDenseMax;
    if (lane < cnt) {
      const int x = cand[s][lane];
      int rank = 0;
      for (int j = 0; j < cnt; ++j) rank += cand[s][j] < x;
      dense_list[base + rank] = x;
      dense_qmask[base + rank] = (int)((mask[x] & full) >> (s * kUnit));
    }
    if (lane == 0) dense_cnt[g * nunits + (i0 >> 4) + s] = cnt;
  }
}

__global__ __launch_bounds__(256) void k_csr_scatter(const int32_t* __restrict__ sel, int64_t sel_gstride,
                                                     int topk, int64_t row0, int nrows, int nbw, int nch,
                                                     const int32_t* __restrict__ chunkoff,
                                                     int32_t* __restrict__ entries, bool dense, int bk_shift) {
  extern __shared__ unsigned long long mask[];
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int i0 = chunk * kChunk;
  const int nq = min(kChunk, nrows - i0);
  const int bmax = (int)((row0 + i0 + nq - 1) >> bk_shift);
  chunk_masks(sel, sel_gstride, topk, g, i0, nq, bmax, mask);
  const int32_t* s = sel + (int64_t)g * sel_gstride + (int64_t)i0 * topk;
  for (int e = threadIdx.x; e < nq * topk; e += blockDim.x) {
    const int b = s[e];
    if (b < 0 || b > bmax) continue;
    const int ql = e / topk, u = e % topk;
    const unsigned long long m = mask[b] & ~dense_bits(mask[b], nq, dense);
    if (!((m >> ql) & 1ull)) continue;  // handled by the dense pass
    const unsigned long long below = m & ((1ull << ql) - 1ull);
    const int64_t pos = chunkoff[((int64_t)g * nbw + b) * nch + chunk] + __popcll(below);
    entries[pos] = ((i0 + ql) << 4) | u;
  }
}

// ---- exclusive scan of int32 (three passes) ---------------------------------

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// block-wide exclusive scan of one value per thread (blockDim.x <= 1024)
__device__ int block_excl_scan(int x, int* total) {
  __shared__ int wsum[17];  // 16 wave offsets + the block total
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    int t = (lane < nw) ? wsum[lane] : 0;
    const int ti = wave_incl_scan(t);
    if (lane < nw) wsum[lane] = ti - t;
    if (lane == nw - 1) wsum[16] = ti;
  }
  __syncthreads();
  const int res = incl - x + wsum[w];
  if (total) *total = wsum[16];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(256) void k_scan_reduce(const int32_t* __restrict__ in, int64_t n,
                                                     int32_t* __restrict__ bsum) {
  const int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * 16;
  int s = 0;
#pragma unroll
  for (int t = 0; t < 16; ++t)
    if (base + t < n) s += in[base + t];
  int tot;
  block_excl_scan(s, &tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void k_scan_bsums(int32_t* __restrict__ bsum, int nblk) {
  // exclusive scan in place; nblk <= 1024 * 16
  const int per = (nblk + 1023) / 1024;
  const int b0 = threadIdx.x * per;
  int s = 0;
  for (int t = 0; t < per; ++t)
    if (b0 + t < nblk) s += bsum[b0 + t];
  int tot;
  int run = block_excl_scan(s, &tot);
  for (int t = 0; t < per; ++t) {
    if (b0 + t < nblk) {
      const int x = bsum[b0 + t];
      bsum[b0 + t] = run;
      run += x;
    }
  }
  if (threadIdx.x == 0) bsum[nblk] = tot;
}

__global__ __launch_bounds__(256) void k_scan_final(const int32_t* __restrict__ in, int64_t n,
                                                    const int32_t* __restrict__ bsum,
                                                    int32_t* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * 16;
  int v[16];
  int s = 0;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    v[t] = (base + t < n) ? in[base + t] : 0;
    s += v[t];
  }
  int run = block_excl_scan(s, nullptr) + bsum[blockIdx.x];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    if (base + t < n) out[base + t] = run;
    run += v[t];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) out[n] = bsum[gridDim.x];
}

// ---- tiles --------------------------------------------------------------------

// One workgroup: per list l = g*nbw + b, tiles = ceil(count / tile_q); exclusive
// scan into tile_start; tile_info[0] = total tiles, tile_info[1] = 0 (queue),
// [2] = lists, [3] = chunks per list, [5] = window rows, [6] = first row,
// [8..15] = 0 (the dense pass's item counters).
__global__ __launch_bounds__(1024) void k_tiles_count(const int32_t* __restrict__ chunkoff, int nch, int L,
                                                      int tile_q, int32_t* __restrict__ tile_start,
                                                      int32_t* __restrict__ tile_info, int nrows, int row0) {
  const int per = (L + 1023) / 1024;
  const int l0 = threadIdx.x * per;
  int s = 0;
  for (int t = 0; t < per; ++t) {
    const int l = l0 + t;
    if (l < L) {
      const int cnt = chunkoff[(int64_t)(l + 1) * nch] - chunkoff[(int64_t)l * nch];
      s += (cnt + tile_q - 1) / tile_q;
    }
  }
  int tot;
  int run = block_excl_scan(s, &tot);
  for (int t = 0; t < per; ++t) {
    const int l = l0 + t;
    if (l < L) {
      tile_start[l] = run;
      const int cnt = chunkoff[(int64_t)(l + 1) * nch] - chunkoff[(int64_t)l * nch];
      run += (cnt + tile_q - 1) / tile_q;
    }
  }
  if (threadIdx.x == 0) {
    tile_start[L] = tot;
    tile_info[0] = tot;
    tile_info[1] = 0;
    tile_info[2] = L;
    tile_info[3] = nch;
    tile_info[5] = nrows;
    tile_info[6] = row0;
  }
  if (threadIdx.x >= 8 && threadIdx.x < 16) tile_info[threadIdx.x] = 0;
}

__global__ __launch_bounds__(256) void k_tiles_fill(const int32_t* __restrict__ tile_start,
                                                    const int32_t* __restrict__ chunkoff, int nch, int L, int nbw,
                                                    int tile_q, const int32_t* __restrict__ tile_info,
                                                    int64_t tile_cap, int32_t* __restrict__ tiles,
                                                    int32_t* __restrict__ tile_visits) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int T = tile_info[0];
  if (t >= T || t >= tile_cap) return;
  if (tile_visits) tile_visits[t] = 0;
  // largest l with tile_start[l] <= t
  int lo = 0, hi = L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int l = lo;
  const int j = (int)(t - tile_start[l]);
  const int start = chunkoff[(int64_t)l * nch];
  const int cnt = chunkoff[(int64_t)(l + 1) * nch] - start;
  const int begin = start + j * tile_q;
  const int len = min(tile_q, cnt - j * tile_q);
  int32_t* o = tiles + t * 4;
  o[0] = l / nbw;  // group
  o[1] = begin;
  o[2] = len;
  o[3] = l % nbw;  // block
}

void launch_csr_and_tiles(const LaunchCsr& a, hipStream_t st) {
  const int nch = (a.nrows + kChunk - 1) / kChunk;
  const size_t lds = (size_t)a.nbw * sizeof(unsigned long long);
  dim3 grid(nch, a.G);
  hipLaunchKernelGGL(k_csr_count, grid, dim3(256), lds, st, a.sel, a.sel_gstride, a.topk, a.row0, a.nrows,
                     a.nbw, nch, a.chunkcnt, a.dense_cnt, a.dense_list, a.dense_qmask, a.dense_slots, a.nunits, a.dense,
                     a.bk_shift);
  const int64_t n = (int64_t)a.G * a.nbw * nch;
  const int nblk = (int)((n + kScanTile - 1) / kScanTile);
  hipLaunchKernelGGL(k_scan_reduce, dim3(nblk), dim3(256), 0, st, a.chunkcnt, n, a.bsum);
  hipLaunchKernelGGL(k_scan_bsums, dim3(1), dim3(1024), 0, st, a.bsum, nblk);
  hipLaunchKernelGGL(k_scan_final, dim3(nblk), dim3(256), 0, st, a.chunkcnt, n, a.bsum, a.chunkoff);
  hipLaunchKernelGGL(k_csr_scatter, grid, dim3(256), lds, st, a.sel, a.sel_gstride, a.topk, a.row0, a.nrows,
                     a.nbw, nch, a.chunkoff, a.entries, a.dense, a.bk_shift);
  const int L = a.G * a.nbw;
  hipLaunchKernelGGL(k_tiles_count, dim3(1), dim3(1024), 0, st, a.chunkoff, nch, L, a.tile_q, a.tile_start,
                     a.tile_info, a.nrows, (int)a.row0);
  const int fill_blocks = (int)((a.tile_cap + 255) / 256);
  hipLaunchKernelGGL(k_tiles_fill, dim3(fill_blocks), dim3(256), 0, st, a.tile_start, a.chunkoff, nch, L, a.nbw,
                     a.tile_q, a.tile_info, a.tile_cap, a.tiles, a.tile_visits);
}

}  // namespace msa
