// C ABI of libmsa: argument validation, workspace carving and the launch
// sequence of the MSA prefill and decode hot path on one MI355X.
//
// Prefill, per sequence and per window of up to kWindowMax query rows:
//   index scores -> top-k selection -> reverse index + tile schedule ->
//   persistent KV-outer attention -> query-stationary attention over the
//   blocks each 16-row unit shares, which merges the KV-outer partials
//   (combine).
// Windows bound the workspace (block scores and partials grow with the rows of
// a window, not with the sequence), which is what makes 1M-token prefill fit.
// Decode: index scores -> per-(sequence, group) selection and attention over
// the selected blocks in one kernel (online softmax across them; no partials).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <new>
#include <vector>

#include "api_internal.h"
#include "msa.h"
#include "msa_launch.h"

namespace {

using namespace msa;

constexpr int64_t kWindowMax = 65536;  // query rows per prefill window
constexpr int kTileQ = 16;             // queries per KV-outer tile
// longest sequence at B_k = 128: the reverse index keeps one 64-bit LDS mask
// per block (<= 8192); shorter blocks scale it down (and bound the pooled
// scores of a window, which grow with the number of blocks)
constexpr int64_t kMaxSeq = 1 << 20;
constexpr size_t kAlign = 256;

struct Shape {
  int Hq, G, k;
  int bk, bk_shift;  // B_k and log2 B_k
  int64_t max_seq;   // longest supported sequence / context
  float scale_log2;
};

msa_status check_params(const msa_params* p, Shape* s) {
  if (!p) return MSA_ERR_INVALID_ARG;
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0 || p->index_dim <= 0 ||
      p->block_size <= 0 || p->topk <= 0)
    return MSA_ERR_INVALID_ARG;
  if (p->num_q_heads % p->num_kv_heads != 0) return MSA_ERR_INVALID_ARG;
  if (p->head_dim != kHeadDim || p->index_dim != kIndexDim ||
      (p->block_size != 128 && p->block_size != 64 && p->block_size != 32) ||
      p->num_q_heads / p->num_kv_heads != kHpg || p->num_kv_heads > 8 || p->topk > kMaxTopk)
    return MSA_ERR_UNSUPPORTED;
  if (!std::isfinite(p->softmax_scale)) return MSA_ERR_INVALID_ARG;
  s->Hq = p->num_q_heads;
  s->G = p->num_kv_heads;
  s->k = p->topk;
  s->bk = p->block_size;
  s->bk_shift = p->block_size == 128 ? 7 : p->block_size == 64 ? 6 : 5;
  s->max_seq = kMaxSeq * p->block_size / kBlock;
  const float scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)p->head_dim);
  s->scale_log2 = scale * 1.4426950408889634f;
  return MSA_OK;
}

inline bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }
inline size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Workgroups of the persistent dense pass: one per CU (a multiple of the 8
// XCDs, at least 8, so that every XCD's range of items has one), no more
// than the items need.
int dense_grid(int64_t items) {
  const int64_t cap = std::max<int64_t>(8, cu_count() / 8 * 8);
  return (int)std::min<int64_t>(cap, std::max<int64_t>(8, (items + 7) / 8 * 8));
}

// entries of rows [a, b): G * sum_i min(k, floor(i/B_k) + 1)
int64_t entries_in(int64_t a, int64_t b, int G, int k, int bk) {
  int64_t e = 0;
  for (int64_t blk = a / bk; blk * bk < b; ++blk) {
    const int64_t lo = std::max(a, blk * bk), hi = std::min(b, (blk + 1) * bk);
    e += (hi - lo) * std::min<int64_t>(k, blk + 1);
  }
  return e * G;
}

struct PrefillLayout {
  int64_t W;  // window rows
  int nb;     // blocks of the sequence
  int nbs;    // row stride of the pooled scores (nb rounded up to 4: 16-byte aligned rows)
  int64_t nch, Lc, nblk, e_cap, tile_cap, slots;
  int64_t nunits;
  size_t sblk, sel, chunkcnt, chunkoff, bsum, entries, tile_start, tiles, tile_info, tile_visits, wg_trace, part_o,
      part_lse, dense_cnt, dense_list, dense_qmask, dense_slots, total;
};

// n_ctx: positions of the longest context; max_rows: most query rows of one
// sequence in the call.
bool prefill_layout(const Shape& s, int64_t n_ctx, int64_t max_rows, PrefillLayout* L) {
  if (n_ctx <= 0 || n_ctx > s.max_seq || max_rows <= 0 || max_rows > n_ctx) return false;
  L->nb = (int)cdiv(n_ctx, s.bk);
  L->nbs = (L->nb + 3) & ~3;
  L->W = std::min<int64_t>(cdiv(max_rows, kBlock) * kBlock, kWindowMax);
  L->nch = cdiv(L->W, 64);
  L->Lc = (int64_t)s.G * L->nb * L->nch;
  L->nblk = cdiv(L->Lc, 4096);
  if (L->nblk > 16384) return false;
  L->e_cap = L->W * s.G * s.k;
  L->tile_cap = cdiv(L->e_cap, kTileQ) + (int64_t)s.G * L->nb;
  L->slots = L->W * s.G * s.k;
  size_t off = 0;
  L->sblk = off;       off += up((size_t)L->W * s.G * L->nbs * sizeof(float));
  L->sel = off;        off += up((size_t)L->W * s.G * s.k * sizeof(int32_t));
  L->chunkcnt = off;   off += up((size_t)L->Lc * sizeof(int32_t));
  L->chunkoff = off;   off += up((size_t)(L->Lc + 1) * sizeof(int32_t));
  L->bsum = off;       off += up((size_t)(L->nblk + 1) * sizeof(int32_t));
  L->entries = off;    off += up((size_t)L->e_cap * sizeof(int32_t));
  L->tile_start = off; off += up((size_t)((int64_t)s.G * L->nb + 1) * sizeof(int32_t));
  L->tiles = off;      off += up((size_t)L->tile_cap * 4 * sizeof(int32_t));
  L->tile_info = off;  off += up(16 * sizeof(int32_t));
  L->tile_visits = off; off += up((size_t)L->tile_cap * sizeof(int32_t));
  L->wg_trace = off;   off += up((size_t)kMaxPersistent * 4 * sizeof(int64_t));
  L->part_o = off;     off += up((size_t)L->slots * kHpg * kHeadDim * sizeof(uint16_t));
  L->part_lse = off;   off += up((size_t)L->slots * kHpg * sizeof(float));
  L->nunits = cdiv(L->W, 16);
  L->dense_cnt = off;  off += up((size_t)s.G * L->nunits * sizeof(int32_t));
  L->dense_list = off; off += up((size_t)s.G * L->nunits * kDenseMax * sizeof(int32_t));
  L->dense_qmask = off; off += up((size_t)s.G * L->nunits * kDenseMax * sizeof(int32_t));
  L->dense_slots = off; off += up((size_t)s.G * L->W * sizeof(int32_t));
  L->total = off;
  return true;
}

// Workspace of the KL-alignment backward, per window of W rows.
constexpr int kKlChunk = 512;   // reverse-index entries per KL work item (1024: 9 % slower, 256: same)

struct KlLayout {
  int64_t W;
  int nb, nch;
  int64_t Lc, nblk, e_cap, chunk_cap, slots;
  size_t chunkcnt, chunkoff, bsum, entries, tile_start, chunks, chunk_info, part_m, part_l, loss_part, dq_part,
      lse_idx, dk_part, total;
};

bool kl_layout(const Shape& s, int64_t N, KlLayout* L) {
  if (N <= 0 || N > kMaxSeq || s.bk != kBlock) return false;
  L->nb = (int)cdiv(N, kBlock);
  L->W = std::min<int64_t>(cdiv(N, kBlock) * kBlock, kWindowMax);
  L->nch = (int)cdiv(L->W, 64);
  L->Lc = (int64_t)s.G * L->nb * L->nch;
  L->nblk = cdiv(L->Lc, 4096);
  if (L->nblk > 16384) return false;
  L->e_cap = L->W * s.G * s.k;
  L->chunk_cap = cdiv(L->e_cap, kKlChunk) + (int64_t)s.G * L->nb;
  L->slots = L->W * s.G * s.k;
  size_t off = 0;
  L->chunkcnt = off;   off += up((size_t)L->Lc * sizeof(int32_t));
  L->chunkoff = off;   off += up((size_t)(L->Lc + 1) * sizeof(int32_t));
  L->bsum = off;       off += up((size_t)(L->nblk + 1) * sizeof(int32_t));
  L->entries = off;    off += up((size_t)L->e_cap * sizeof(int32_t));
  L->tile_start = off; off += up((size_t)((int64_t)s.G * L->nb + 1) * sizeof(int32_t));
  L->chunks = off;     off += up((size_t)L->chunk_cap * 4 * sizeof(int32_t));
  L->chunk_info = off; off += up(16 * sizeof(int32_t));
  L->part_m = off;     off += up((size_t)L->slots * sizeof(float));
  L->part_l = off;     off += up((size_t)L->slots * sizeof(float));
  L->loss_part = off;  off += up((size_t)L->slots * sizeof(float));
  L->dq_part = off;    off += up((size_t)L->slots * kIndexDim * sizeof(float));
  L->lse_idx = off;    off += up((size_t)L->W * s.G * sizeof(float));
  L->dk_part = off;    off += up((size_t)L->chunk_cap * kBlock * kIndexDim * sizeof(float));
  L->total = off;
  return true;
}

struct DecodeLayout {
  int nb;
  size_t sblk, total;
};

// max_ctx beyond the longest supported context has no layout (the caller
// reports MSA_ERR_UNSUPPORTED)
bool decode_layout(const Shape& s, int32_t B, int64_t max_ctx, DecodeLayout* L) {
  if (B <= 0 || max_ctx <= 0 || max_ctx > s.max_seq) return false;
  L->nb = (int)cdiv(max_ctx, s.bk);
  size_t off = 0;
  L->sblk = off;     off += up((size_t)B * s.G * L->nb * sizeof(float));
  L->total = off;
  return true;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

msa_status finish() { return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP; }

// d_model: whole 64-wide slices; tokens bounded so every index stays well
// inside int64 and the grid inside its limits
bool project_args_ok(int64_t n_tokens, int32_t d_model) {
  return n_tokens > 0 && n_tokens <= (int64_t)1 << 28 && d_model >= 64 && d_model <= 65536 && d_model % 64 == 0;
}

msa_status run_index_project(const msa_params* p, int64_t n_tokens, int32_t d_model, const void* x,
                             const void* w_qi, const void* w_ki, const int32_t* ctx_lens, int64_t max_ctx,
                             void* q_idx, void* k_idx, void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  msa_status st = check_params(p, &s);
  if (st != MSA_OK) return st;
  if (!project_args_ok(n_tokens, d_model)) return n_tokens > 0 && d_model > 0 ? MSA_ERR_UNSUPPORTED
                                                                                : MSA_ERR_INVALID_ARG;
  for (const void* ptr : {x, w_qi, w_ki, (const void*)q_idx, (const void*)k_idx})
    if (!ptr || !aligned(ptr, 16)) return MSA_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, kAlign)) return MSA_ERR_INVALID_ARG;
  const ProjectPlan pl = plan_index_project(n_tokens, d_model, s.G);
  if (workspace_bytes < pl.part_floats * sizeof(float)) return MSA_ERR_WORKSPACE_TOO_SMALL;
  (void)hipGetLastError();
  LaunchProject a{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_qi),
                  static_cast<const uint16_t*>(w_ki), n_tokens, d_model, s.G, static_cast<uint16_t*>(q_idx),
                  static_cast<uint16_t*>(k_idx), ctx_lens, max_ctx, static_cast<float*>(workspace)};
  launch_index_project(a, static_cast<hipStream_t>(stream));
  return finish();
}

}  // namespace

extern "C" {

const char* msa_status_string(msa_status s) {
  switch (s) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

size_t msa_prefill_workspace_bytes(const msa_params* p, int32_t batch, int64_t seq_len) {
  Shape s;
  PrefillLayout L;
  if (batch <= 0 || check_params(p, &s) != MSA_OK || !prefill_layout(s, seq_len, seq_len, &L)) return 0;
  return L.total;
}

}  // extern "C"

namespace {

// Records a HIP event at every stage boundary when profiling (ev != nullptr).
struct StageClock {
  std::vector<hipEvent_t>* ev;
  hipStream_t st;
  void mark() {
    if (!ev) return;
    hipEvent_t e;
    if (hipEventCreate(&e) == hipSuccess) {
      (void)hipEventRecord(e, st);
      ev->push_back(e);
    }
  }
};

// One sequence's query rows [q_start, q_start + q_len); they attend to the
// positions < q_start + q_len of k, v and k_idx. The query-side pointers hold
// the q_len rows only; sel (optional) is sel[g*sel_gstride + (i - q_start)*k + u].
struct SeqIO {
  const uint16_t *q, *q_idx, *k, *v, *k_idx;
  uint16_t* out;
  int32_t* sel;
  int64_t sel_gstride;
  float* lse;
  int64_t q_start, q_len;
};

// The five stages on the window of rows [w0, w0 + Wn) of a sequence.
void prefill_window(const Shape& s, const PrefillLayout& L, const SeqIO& io, int64_t w0, int64_t Wn,
                    void* workspace, hipStream_t hs, StageClock& clk) {
  const int G = s.G, Hq = s.Hq, K = s.k;
  const int64_t n_ctx = io.q_start + io.q_len;
  const int64_t r0 = w0 - io.q_start;  // the window's first row among the call's rows
  const int nbw = (int)((w0 + Wn - 1) / s.bk + 1);
  const uint16_t* qw = io.q + r0 * Hq * kHeadDim;
  clk.mark();
  // 1. index scores for query blocks that have more than k-1 older blocks
  // 128-row query blocks with a row whose own block is >= k
  LaunchIndexPrefill ia{io.q_idx + r0 * G * kIndexDim, io.k_idx, at<float>(workspace, L.sblk), w0, w0 + Wn,
                        (int)std::max<int64_t>((int64_t)K * s.bk / kBlock, w0 / kBlock),
                        (int)((w0 + Wn - 1) / kBlock + 1), L.nbs, G, s.bk};
  launch_index_prefill(ia, hs);
  clk.mark();
  // 2. top-k selection
  int32_t* selw = io.sel ? io.sel + r0 * K : at<int32_t>(workspace, L.sel);
  const int64_t gstride = io.sel ? io.sel_gstride : L.W * K;
  LaunchSelect sa{at<float>(workspace, L.sblk), L.nbs, selw, gstride, K, Wn, G, K, w0, nullptr, s.bk_shift};
  launch_select(sa, hs);
  clk.mark();
  // 3. reverse index and tile schedule
  const int64_t e_w = entries_in(w0, w0 + Wn, G, K, s.bk);
  const int64_t tile_cap = cdiv(e_w, kTileQ) + (int64_t)G * nbw;
  const int nunits = (int)cdiv(Wn, 16);
  int32_t* dcnt = at<int32_t>(workspace, L.dense_cnt);
  int32_t* dlist = at<int32_t>(workspace, L.dense_list);
  LaunchCsr ca{selw, gstride, K, w0, (int)Wn, nbw, G,
               at<int32_t>(workspace, L.chunkcnt), at<int32_t>(workspace, L.chunkoff),
               at<int32_t>(workspace, L.bsum), at<int32_t>(workspace, L.entries),
               at<int32_t>(workspace, L.tile_start), at<int32_t>(workspace, L.tiles),
               at<int32_t>(workspace, L.tile_info), kTileQ, tile_cap, dcnt, dlist,
               at<int32_t>(workspace, L.dense_qmask), at<int32_t>(workspace, L.dense_slots), nunits, true,
               s.bk_shift, at<int32_t>(workspace, L.tile_visits)};
  launch_csr_and_tiles(ca, hs);
  clk.mark();
  // 4. KV-outer attention over the pairs not shared by a whole unit
  LaunchAttnPrefill aa{qw, io.k, io.v, at<int32_t>(workspace, L.entries), at<int32_t>(workspace, L.tiles),
                       at<int32_t>(workspace, L.tile_info), at<uint16_t>(workspace, L.part_o),
                       at<float>(workspace, L.part_lse), n_ctx, G, nbw, K, s.scale_log2,
                       (int)std::min<int64_t>({(int64_t)cu_count(), tile_cap, (int64_t)kMaxPersistent}), s.bk,
                       at<int32_t>(workspace, L.tile_visits), at<int64_t>(workspace, L.wg_trace)};
  launch_attn_prefill(aa, hs);
  clk.mark();
  // 5. query-stationary attention over the units' shared blocks + merge
  LaunchAttnDense da{qw, io.k, io.v, dcnt, dlist, at<int32_t>(workspace, L.dense_qmask),
                     at<int32_t>(workspace, L.dense_slots), at<uint16_t>(workspace, L.part_o),
                     at<float>(workspace, L.part_lse), io.out + r0 * Hq * kHeadDim,
                     io.lse ? io.lse + r0 * Hq : nullptr, n_ctx, w0, (int)Wn, nunits, G, K, s.scale_log2, s.bk,
                     at<int32_t>(workspace, L.tile_info), dense_grid((int64_t)nunits * G)};
  launch_attn_dense(da, hs);
  clk.mark();
}

// Windows of one sequence. The 16-row units of the dense pass must not
// straddle a key block (their rows share the local block), so a start that is
// not a multiple of 16 first gets a window of its own up to the next multiple
// of 16; the rest goes in windows of at most L.W rows.
void prefill_seq(const Shape& s, const PrefillLayout& L, const SeqIO& io, void* workspace, hipStream_t hs,
                 StageClock& clk) {
  const int64_t end = io.q_start + io.q_len;
  for (int64_t w0 = io.q_start; w0 < end;) {
    const int64_t head_end = (w0 + 15) / 16 * 16;
    const int64_t Wn = head_end != w0 ? std::min(head_end, end) - w0 : std::min(L.W, end - w0);
    prefill_window(s, L, io, w0, Wn, workspace, hs, clk);
    w0 += Wn;
  }
}

msa_status run_prefill(const msa_params* p, int32_t batch, int64_t seq_len, const void* q, const void* k,
                       const void* v, const void* q_idx, const void* k_idx, void* out, int32_t* sel_out,
                       float* lse_out, void* workspace, size_t workspace_bytes, void* stream,
                       std::vector<hipEvent_t>* ev) {
  Shape s;
  msa_status st = check_params(p, &s);
  if (st != MSA_OK) return st;
  if (batch <= 0 || seq_len <= 0) return MSA_ERR_INVALID_ARG;
  if (seq_len > s.max_seq) return MSA_ERR_UNSUPPORTED;
  for (const void* ptr : {q, k, v, q_idx, k_idx, (const void*)out})
    if (!ptr || !aligned(ptr, 16)) return MSA_ERR_INVALID_ARG;
  if ((sel_out && !aligned(sel_out, 4)) || (lse_out && !aligned(lse_out, 4))) return MSA_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, kAlign)) return MSA_ERR_INVALID_ARG;
  PrefillLayout L;
  if (!prefill_layout(s, seq_len, seq_len, &L)) return MSA_ERR_UNSUPPORTED;
  if (workspace_bytes < L.total) return MSA_ERR_WORKSPACE_TOO_SMALL;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  StageClock clk{ev, hs};
  const int64_t N = seq_len;
  const int G = s.G, Hq = s.Hq, K = s.k;
  for (int32_t bi = 0; bi < batch; ++bi) {
    SeqIO io;
    io.q = static_cast<const uint16_t*>(q) + (int64_t)bi * N * Hq * kHeadDim;
    io.k = static_cast<const uint16_t*>(k) + (int64_t)bi * N * G * kHeadDim;
    io.v = static_cast<const uint16_t*>(v) + (int64_t)bi * N * G * kHeadDim;
    io.q_idx = static_cast<const uint16_t*>(q_idx) + (int64_t)bi * N * G * kIndexDim;
    io.k_idx = static_cast<const uint16_t*>(k_idx) + (int64_t)bi * N * kIndexDim;
    io.out = static_cast<uint16_t*>(out) + (int64_t)bi * N * Hq * kHeadDim;
    io.sel = sel_out ? sel_out + (int64_t)bi * G * N * K : nullptr;
    io.sel_gstride = N * K;
    io.lse = lse_out ? lse_out + (int64_t)bi * N * Hq : nullptr;
    io.q_start = 0;
    io.q_len = N;
    prefill_seq(s, L, io, workspace, hs, clk);
  }
  return finish();
}

// Host-side checks of a variable-length call; *max_rows and *total get the
// longest q_len and the sum of q_len.
msa_status check_varlen(int32_t batch, int64_t max_ctx, const int64_t* q_start, const int64_t* q_len,
                        int64_t* max_rows, int64_t* total) {
  if (batch <= 0 || max_ctx <= 0 || !q_start || !q_len) return MSA_ERR_INVALID_ARG;
  if (max_ctx > kMaxSeq) return MSA_ERR_UNSUPPORTED;
  *max_rows = 0;
  *total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (q_start[b] < 0 || q_len[b] < 0 || q_len[b] > max_ctx - q_start[b]) return MSA_ERR_INVALID_ARG;
    *max_rows = std::max(*max_rows, q_len[b]);
    *total += q_len[b];
  }
  return MSA_OK;
}

msa_status run_prefill_varlen(const msa_params* p, int32_t batch, int64_t max_ctx, const int64_t* q_start,
                              const int64_t* q_len, const void* q, const void* q_idx, const void* k_cache,
                              const void* v_cache, const void* k_idx_cache, void* out, int32_t* sel_out,
                              float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  msa_status st = check_params(p, &s);
  if (st != MSA_OK) return st;
  int64_t max_rows = 0, total = 0;
  st = check_varlen(batch, max_ctx, q_start, q_len, &max_rows, &total);
  if (st != MSA_OK) return st;
  for (const void* ptr : {q, q_idx, k_cache, v_cache, k_idx_cache, (const void*)out})
    if (!ptr || !aligned(ptr, 16)) return MSA_ERR_INVALID_ARG;
  if ((sel_out && !aligned(sel_out, 4)) || (lse_out && !aligned(lse_out, 4))) return MSA_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, kAlign)) return MSA_ERR_INVALID_ARG;
  if (total == 0) return MSA_OK;
  PrefillLayout L;
  if (!prefill_layout(s, max_ctx, max_rows, &L)) return MSA_ERR_UNSUPPORTED;
  if (workspace_bytes < L.total) return MSA_ERR_WORKSPACE_TOO_SMALL;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  StageClock clk{nullptr, hs};
  const int G = s.G, Hq = s.Hq, K = s.k;
  int64_t r = 0;  // first packed row of sequence b
  for (int32_t b = 0; b < batch; ++b) {
    if (q_len[b] > 0) {
      SeqIO io;
      io.q = static_cast<const uint16_t*>(q) + r * Hq * kHeadDim;
      io.q_idx = static_cast<const uint16_t*>(q_idx) + r * G * kIndexDim;
      io.k = static_cast<const uint16_t*>(k_cache) + (int64_t)b * max_ctx * G * kHeadDim;
      io.v = static_cast<const uint16_t*>(v_cache) + (int64_t)b * max_ctx * G * kHeadDim;
      io.k_idx = static_cast<const uint16_t*>(k_idx_cache) + (int64_t)b * max_ctx * kIndexDim;
      io.out = static_cast<uint16_t*>(out) + r * Hq * kHeadDim;
      io.sel = sel_out ? sel_out + r * K : nullptr;
      io.sel_gstride = total * K;
      io.lse = lse_out ? lse_out + r * Hq : nullptr;
      io.q_start = q_start[b];
      io.q_len = q_len[b];
      prefill_seq(s, L, io, workspace, hs, clk);
    }
    r += q_len[b];
  }
  return finish();
}

// Sums the stage durations of a profiled call (marks come in groups of
// nstage + 1 per window) into stage_ms after synchronising on the last mark.
msa_status collect(std::vector<hipEvent_t>& ev, int nstage, float* stage_ms, msa_status st) {
  for (int i = 0; i < nstage; ++i) stage_ms[i] = 0.f;
  if (st == MSA_OK && !ev.empty()) {
    if (hipEventSynchronize(ev.back()) != hipSuccess) st = MSA_ERR_HIP;
    const size_t per = (size_t)nstage + 1;
    for (size_t w = 0; st == MSA_OK && w + per <= ev.size(); w += per) {
      for (int i = 0; i < nstage; ++i) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, ev[w + i], ev[w + i + 1]) != hipSuccess) st = MSA_ERR_HIP;
        stage_ms[i] += ms;
      }
    }
  }
  for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  return st;
}

}  // namespace

extern "C" {

msa_status msa_prefill(const msa_params* p, int32_t batch, int64_t seq_len, const void* q, const void* k,
                       const void* v, const void* q_idx, const void* k_idx, void* out, int32_t* sel_out,
                       float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  return run_prefill(p, batch, seq_len, q, k, v, q_idx, k_idx, out, sel_out, lse_out, workspace, workspace_bytes,
                     stream, nullptr);
}

}  // extern "C"

// Stage events of a *_timed call, read (and released) by msa_stage_timer_read.
struct msa_stage_timer {
  std::vector<hipEvent_t> ev;
  int nstage;
};

namespace {

msa_status keep_timer(std::vector<hipEvent_t>& ev, int nstage, msa_status st, msa_stage_timer** timer) {
  *timer = nullptr;
  if (st == MSA_OK) {
    msa_stage_timer* t = new (std::nothrow) msa_stage_timer{std::move(ev), nstage};
    if (t) {
      *timer = t;
      return MSA_OK;
    }
    st = MSA_ERR_HIP;
  }
  for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  return st;
}

}  // namespace

extern "C" {

msa_status msa_prefill_timed(const msa_params* p, int32_t batch, int64_t seq_len, const void* q, const void* k,
                             const void* v, const void* q_idx, const void* k_idx, void* out, int32_t* sel_out,
                             float* lse_out, void* workspace, size_t workspace_bytes, void* stream,
                             msa_stage_timer** timer) {
  if (!timer) return MSA_ERR_INVALID_ARG;
  std::vector<hipEvent_t> ev;
  msa_status st = run_prefill(p, batch, seq_len, q, k, v, q_idx, k_idx, out, sel_out, lse_out, workspace,
                              workspace_bytes, stream, &ev);
  return keep_timer(ev, 5, st, timer);
}

msa_status msa_stage_timer_read(msa_stage_timer* timer, float* stage_ms) {
  if (!timer || !stage_ms) return MSA_ERR_INVALID_ARG;
  msa_status st = collect(timer->ev, timer->nstage, stage_ms, MSA_OK);
  delete timer;
  return st;
}

msa_status msa_prefill_profiled(const msa_params* p, int32_t batch, int64_t seq_len, const void* q,
                                const void* k, const void* v, const void* q_idx, const void* k_idx, void* out,
                                int32_t* sel_out, float* lse_out, void* workspace, size_t workspace_bytes,
                                void* stream, float* stage_ms) {
  if (!stage_ms) return MSA_ERR_INVALID_ARG;
  std::vector<hipEvent_t> ev;
  msa_status st = run_prefill(p, batch, seq_len, q, k, v, q_idx, k_idx, out, sel_out, lse_out, workspace,
                              workspace_bytes, stream, &ev);
  return collect(ev, 5, stage_ms, st);
}

size_t msa_prefill_varlen_workspace_bytes(const msa_params* p, int64_t max_q_len, int64_t max_ctx) {
  Shape s;
  PrefillLayout L;
  if (check_params(p, &s) != MSA_OK || !prefill_layout(s, max_ctx, std::min(max_q_len, max_ctx), &L)) return 0;
  return L.total;
}

msa_status msa_prefill_schedule_layout(const msa_params* p, int64_t max_q_len, int64_t max_ctx,
                                       msa_prefill_schedule_map* m) {
  if (!m || max_q_len <= 0 || max_ctx <= 0) return MSA_ERR_INVALID_ARG;
  Shape s;
  msa_status st = check_params(p, &s);
  if (st != MSA_OK) return st;
  PrefillLayout L;
  if (!prefill_layout(s, max_ctx, std::min(max_q_len, max_ctx), &L)) return MSA_ERR_UNSUPPORTED;
  *m = msa_prefill_schedule_map{};
  m->tile_info = (int64_t)L.tile_info;
  m->chunk_off = (int64_t)L.chunkoff;
  m->entries = (int64_t)L.entries;
  m->tiles = (int64_t)L.tiles;
  m->tile_visits = (int64_t)L.tile_visits;
  m->wg_trace = (int64_t)L.wg_trace;
  m->dense_cnt = (int64_t)L.dense_cnt;
  m->dense_list = (int64_t)L.dense_list;
  m->dense_qmask = (int64_t)L.dense_qmask;
  m->dense_slots = (int64_t)L.dense_slots;
  m->dense_max = kDenseMax;
  m->tile_queries = kTileQ;
  m->claim = kTileClaim;
  m->dense_min = kDenseMin;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0)
    m->wall_clock_khz = khz;
  return MSA_OK;
}

msa_status msa_prefill_varlen(const msa_params* p, int32_t batch, int64_t max_ctx, const int64_t* q_start,
                              const int64_t* q_len, const void* q, const void* q_idx, const void* k_cache,
                              const void* v_cache, const void* k_idx_cache, void* out, int32_t* sel_out,
                              float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  return run_prefill_varlen(p, batch, max_ctx, q_start, q_len, q, q_idx, k_cache, v_cache, k_idx_cache, out,
                            sel_out, lse_out, workspace, workspace_bytes, stream);
}

size_t msa_decode_workspace_bytes(const msa_params* p, int32_t batch, int64_t max_ctx) {
  Shape s;
  DecodeLayout L;
  if (check_params(p, &s) != MSA_OK || !decode_layout(s, batch, max_ctx, &L)) return 0;
  return L.total;
}

}  // extern "C"

namespace msa {

// Host-side checks of a decode call, everything but the workspace; *need gets
// the workspace bytes the call takes.
msa_status decode_check(const msa_params* p, int32_t batch, int64_t max_ctx, const void* q, const void* q_idx,
                        const void* k_cache, const void* v_cache, const void* k_idx_cache, const int32_t* ctx_lens,
                        const void* out, const int32_t* sel_out, const float* lse_out, size_t* need) {
  Shape s;
  msa_status st = check_params(p, &s);
  if (st != MSA_OK) return st;
  if (batch <= 0 || max_ctx <= 0) return MSA_ERR_INVALID_ARG;
  if (max_ctx > s.max_seq) return MSA_ERR_UNSUPPORTED;
  for (const void* ptr : {q, q_idx, k_cache, v_cache, k_idx_cache, out})
    if (!ptr || !aligned(ptr, 16)) return MSA_ERR_INVALID_ARG;
  if (!ctx_lens || !aligned(ctx_lens, 4)) return MSA_ERR_INVALID_ARG;
  if ((sel_out && !aligned(sel_out, 4)) || (lse_out && !aligned(lse_out, 4))) return MSA_ERR_INVALID_ARG;
  DecodeLayout L;
  if (!decode_layout(s, batch, max_ctx, &L)) return MSA_ERR_INVALID_ARG;
  *need = L.total;
  return MSA_OK;
}

}  // namespace msa

namespace {

msa_status run_decode(const msa_params* p, int32_t batch, int64_t max_ctx, const void* q, const void* q_idx,
                      const void* k_cache, const void* v_cache, const void* k_idx_cache,
                      const int32_t* ctx_lens, void* out, int32_t* sel_out, float* lse_out, void* workspace,
                      size_t workspace_bytes, void* stream, std::vector<hipEvent_t>* ev) {
  size_t need = 0;
  msa_status st = msa::decode_check(p, batch, max_ctx, q, q_idx, k_cache, v_cache, k_idx_cache, ctx_lens, out, sel_out,
                               lse_out, &need);
  if (st != MSA_OK) return st;
  if (!workspace || !aligned(workspace, kAlign)) return MSA_ERR_INVALID_ARG;
  if (workspace_bytes < need) return MSA_ERR_WORKSPACE_TOO_SMALL;
  Shape s;
  check_params(p, &s);
  DecodeLayout L;
  decode_layout(s, batch, max_ctx, &L);

  hipStream_t hs = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  StageClock clk{ev, hs};
  clk.mark();
  LaunchIndexDecode ia{static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx_cache), ctx_lens,
                       at<float>(workspace, L.sblk), max_ctx, L.nb, batch, s.G, s.k, s.bk};
  launch_index_decode(ia, hs);
  clk.mark();
  // selection and attention in one kernel
  LaunchAttnDecode aa{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                      static_cast<const uint16_t*>(v_cache), ctx_lens, at<float>(workspace, L.sblk), L.nb, sel_out,
                      static_cast<uint16_t*>(out), lse_out, max_ctx, batch, s.G, s.k, s.scale_log2, s.bk};
  launch_attn_decode(aa, hs);
  clk.mark();
  return finish();
}

}  // namespace

extern "C" {

msa_status msa_decode(const msa_params* p, int32_t batch, int64_t max_ctx, const void* q, const void* q_idx,
                      const void* k_cache, const void* v_cache, const void* k_idx_cache,
                      const int32_t* ctx_lens, void* out, int32_t* sel_out, float* lse_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return run_decode(p, batch, max_ctx, q, q_idx, k_cache, v_cache, k_idx_cache, ctx_lens, out, sel_out, lse_out,
                    workspace, workspace_bytes, stream, nullptr);
}

msa_status msa_decode_profiled(const msa_params* p, int32_t batch, int64_t max_ctx, const void* q,
                               const void* q_idx, const void* k_cache, const void* v_cache,
                               const void* k_idx_cache, const int32_t* ctx_lens, void* out, int32_t* sel_out,
                               float* lse_out, void* workspace, size_t workspace_bytes, void* stream,
                               float* stage_ms) {
  if (!stage_ms) return MSA_ERR_INVALID_ARG;
  std::vector<hipEvent_t> ev;
  msa_status st = run_decode(p, batch, max_ctx, q, q_idx, k_cache, v_cache, k_idx_cache, ctx_lens, out, sel_out,
                             lse_out, workspace, workspace_bytes, stream, &ev);
  return collect(ev, 2, stage_ms, st);
}

msa_status msa_decode_timed(const msa_params* p, int32_t batch, int64_t max_ctx, const void* q, const void* q_idx,
                            const void* k_cache, const void* v_cache, const void* k_idx_cache,
                            const int32_t* ctx_lens, void* out, int32_t* sel_out, float* lse_out, void* workspace,
                            size_t workspace_bytes, void* stream, msa_stage_timer** timer) {
  if (!timer) return MSA_ERR_INVALID_ARG;
  std::vector<hipEvent_t> ev;
  msa_status st = run_decode(p, batch, max_ctx, q, q_idx, k_cache, v_cache, k_idx_cache, ctx_lens, out, sel_out,
                             lse_out, workspace, workspace_bytes, stream, &ev);
  return keep_timer(ev, 2, st, timer);
}

size_t msa_index_kl_workspace_bytes(const msa_params* p, int64_t seq_len) {
  Shape s;
  KlLayout L;
  if (check_params(p, &s) != MSA_OK || !kl_layout(s, seq_len, &L)) return 0;
  return L.total;
}

msa_status msa_index_kl_backward(const msa_params* p, int64_t seq_len, const void* q, const void* k,
                                 const void* q_idx, const void* k_idx, const int32_t* sel, const float* lse,
                                 float* loss, float* dq_idx, float* dk_idx, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  Shape s;
  msa_status st = check_params(p, &s);
  if (st != MSA_OK) return st;
  if (seq_len <= 0) return MSA_ERR_INVALID_ARG;
  if (seq_len > kMaxSeq) return MSA_ERR_UNSUPPORTED;
  for (const void* ptr : {q, k, q_idx, k_idx, (const void*)lse, (const void*)dq_idx, (const void*)dk_idx})
    if (!ptr || !aligned(ptr, 16)) return MSA_ERR_INVALID_ARG;
  if (!sel || !aligned(sel, 4) || !loss || !aligned(loss, 4)) return MSA_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, kAlign)) return MSA_ERR_INVALID_ARG;
  KlLayout L;
  if (!kl_layout(s, seq_len, &L)) return MSA_ERR_UNSUPPORTED;
  if (workspace_bytes < L.total) return MSA_ERR_WORKSPACE_TOO_SMALL;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t N = seq_len;
  const int G = s.G, Hq = s.Hq, K = s.k;
  launch_zero_f32(dk_idx, N * kIndexDim, hs);
  for (int64_t w0 = 0; w0 < N; w0 += L.W) {
    const int64_t Wn = std::min(L.W, N - w0);
    const int nbw = (int)((w0 + Wn - 1) / kBlock + 1);
    const int32_t* selw = sel + w0 * K;
    const int64_t e_w = entries_in(w0, w0 + Wn, G, K, kBlock);
    const int64_t chunk_cap = cdiv(e_w, kKlChunk) + (int64_t)G * nbw;
    // every selected pair, in chunks of up to kKlChunk queries per (group, block)
    LaunchCsr ca{selw, N * K, K, w0, (int)Wn, nbw, G,
                 at<int32_t>(workspace, L.chunkcnt), at<int32_t>(workspace, L.chunkoff),
                 at<int32_t>(workspace, L.bsum), at<int32_t>(workspace, L.entries),
                 at<int32_t>(workspace, L.tile_start), at<int32_t>(workspace, L.chunks),
                 at<int32_t>(workspace, L.chunk_info), kKlChunk, chunk_cap, nullptr, nullptr, nullptr, nullptr,
                 (int)cdiv(Wn, 16), false, 7};
    launch_csr_and_tiles(ca, hs);
    LaunchKl ka{static_cast<const uint16_t*>(q) + w0 * Hq * kHeadDim, static_cast<const uint16_t*>(k),
                static_cast<const uint16_t*>(q_idx) + w0 * G * kIndexDim, static_cast<const uint16_t*>(k_idx),
                lse + w0 * Hq, at<int32_t>(workspace, L.entries), at<int32_t>(workspace, L.chunks),
                at<int32_t>(workspace, L.chunk_info), chunk_cap, at<float>(workspace, L.part_m),
                at<float>(workspace, L.part_l), at<float>(workspace, L.loss_part), at<float>(workspace, L.dq_part),
                at<float>(workspace, L.lse_idx), loss, dq_idx + w0 * G * kIndexDim, dk_idx,
                at<float>(workspace, L.dk_part), at<int32_t>(workspace, L.tile_start), N, w0, (int)Wn, nbw, G, K,
                s.scale_log2};
    launch_kl_window(ka, hs);
  }
  return finish();
}

size_t msa_index_project_workspace_bytes(const msa_params* p, int64_t n_tokens, int32_t d_model) {
  Shape s;
  if (check_params(p, &s) != MSA_OK || !project_args_ok(n_tokens, d_model)) return 0;
  return up(std::max<size_t>(1, plan_index_project(n_tokens, d_model, s.G).part_floats * sizeof(float)));
}

msa_status msa_index_project(const msa_params* p, int64_t n_tokens, int32_t d_model, const void* x,
                             const void* w_qi, const void* w_ki, void* q_idx, void* k_idx, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return run_index_project(p, n_tokens, d_model, x, w_qi, w_ki, nullptr, 0, q_idx, k_idx, workspace,
                           workspace_bytes, stream);
}

msa_status msa_index_project_decode(const msa_params* p, int32_t batch, int64_t max_ctx, int32_t d_model,
                                    const void* x, const void* w_qi, const void* w_ki, const int32_t* ctx_lens,
                                    void* q_idx, void* k_idx_cache, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (batch <= 0 || max_ctx <= 0 || !ctx_lens || !aligned(ctx_lens, 4)) return MSA_ERR_INVALID_ARG;
  return run_index_project(p, batch, d_model, x, w_qi, w_ki, ctx_lens, max_ctx, q_idx, k_idx_cache, workspace,
                           workspace_bytes, stream);
}

msa_status msa_index_scores(const msa_params* p, int64_t seq_len, const void* q_idx, const void* k_idx,
                            float* scores, void* stream) {
  Shape s;
  msa_status st = check_params(p, &s);
  if (st != MSA_OK) return st;
  if (seq_len <= 0) return MSA_ERR_INVALID_ARG;
  if (seq_len > s.max_seq) return MSA_ERR_UNSUPPORTED;
  if (!q_idx || !k_idx || !scores || !aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(scores, 4))
    return MSA_ERR_INVALID_ARG;
  (void)hipGetLastError();
  const int nb = (int)cdiv(seq_len, s.bk);
  // 128-row query blocks holding a row whose own block is >= k
  LaunchIndexPrefill ia{static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx), scores, 0,
                        seq_len, (int)((int64_t)s.k * s.bk / kBlock), (int)cdiv(seq_len, kBlock), nb, s.G, s.bk};
  launch_index_prefill(ia, static_cast<hipStream_t>(stream));
  return finish();
}

msa_status msa_select_blocks(const msa_params* p, int64_t seq_len, const float* scores, int32_t* sel_out,
                             void* stream) {
  Shape s;
  msa_status st = check_params(p, &s);
  if (st != MSA_OK) return st;
  if (seq_len <= 0) return MSA_ERR_INVALID_ARG;
  if (!scores || !sel_out || !aligned(scores, 4) || !aligned(sel_out, 4)) return MSA_ERR_INVALID_ARG;
  (void)hipGetLastError();
  if (seq_len > s.max_seq) return MSA_ERR_UNSUPPORTED;
  const int nb = (int)cdiv(seq_len, s.bk);
  LaunchSelect sa{scores, nb, sel_out, seq_len * s.k, s.k, seq_len, s.G, s.k, 0, nullptr, s.bk_shift};
  launch_select(sa, static_cast<hipStream_t>(stream));
  return finish();
}

}  // extern "C"
