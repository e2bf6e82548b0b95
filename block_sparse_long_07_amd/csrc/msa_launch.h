// Host-side launch descriptors of the MSA kernels (internal to libmsa).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kHeadDim = 128;  // d
constexpr int kIndexDim = 64;  // d_idx
constexpr int kBlock = 128;    // B_k
constexpr int kHpg = 16;       // query heads per GQA group
constexpr int kMaxTopk = 16;
// A 16-row unit's block goes to the query-stationary (dense) pass when at
// least kDenseMin of the unit's rows selected it (all rows, if the unit has
// fewer): the rows that did not are masked there, which costs less than
// their KV-outer partials would. At most 16*16/kDenseMin blocks qualify.
constexpr int kDenseMin = 5;
constexpr int kDenseMax = 64;
constexpr int kMaxPersistent = 1024;  // workgroups of the persistent KV-outer pass, at most
constexpr int kTileClaim = 4;         // tiles a KV-outer workgroup claims from the queue at a time

// Per-query arrays of a prefill window (q, q_idx, out, lse, selection) start
// at the window's first row row0; key-side arrays (k, v, k_idx) at position 0.
struct LaunchIndexPrefill {
  const uint16_t* q_idx;  // [(i - row0)*G + g][64]: the window's rows
  const uint16_t* k_idx;  // [position][64]
  float* sblk;            // rows (i - row0)*G + g, row stride nb
  int64_t row0, row_end;  // the window's rows [row0, row_end)
  int qb_begin, qb_end;   // 128-row query blocks scored: [qb_begin, qb_end)
  int nb;                 // row stride of sblk
  int G;
  int bk;                 // B_k: 128, 64 or 32 (pooled scores per B_k keys)
};
void launch_index_prefill(const LaunchIndexPrefill& a, hipStream_t st);

struct LaunchIndexDecode {
  const uint16_t* q_idx;  // [batch, G, 64]
  const uint16_t* k_idx;  // [batch, max_ctx, 64]
  const int32_t* ctx_lens;
  float* sblk;            // [(s*G + g)*nb + b]
  int64_t max_ctx;
  int nb, batch, G, topk;
  int bk;                 // B_k: 128, 64 or 32
};
void launch_index_decode(const LaunchIndexDecode& a, hipStream_t st);

// Selection over rows r = rr*G + g of sblk (row stride nb). b_loc of row rr is
// (row0 + rr)/128 (prefill) or (ctx_lens[rr] - 1)/128 (decode, ctx_lens != null).
struct LaunchSelect {
  const float* sblk;
  int nb;
  int32_t* sel;           // sel[g*sel_gstride + rr*sel_rstride + u]
  int64_t sel_gstride, sel_rstride;
  int64_t nrows;          // rr count
  int G, topk;
  int64_t row0;
  const int32_t* ctx_lens;
  int bk_shift;           // log2 B_k
};
void launch_select(const LaunchSelect& a, hipStream_t st);

// Reverse index (CSR) of one window's selections: for each (g, b) the entries
// (i_rel << 4 | u) of the queries that selected b, ascending in i.
struct LaunchCsr {
  const int32_t* sel;     // sel[g*sel_gstride + i_rel*topk + u]
  int64_t sel_gstride;
  int topk;
  int64_t row0;           // absolute first row of the window
  int nrows;              // window rows
  int nbw;                // blocks visible to the window: (row0 + nrows - 1)/128 + 1
  int G;
  int32_t* chunkcnt;      // [G*nbw*nch]
  int32_t* chunkoff;      // [G*nbw*nch + 1]
  int32_t* bsum;          // scan scratch
  int32_t* entries;
  int32_t* tile_start;    // [G*nbw + 1]
  int32_t* tiles;         // [T_cap][4] = (group, begin, len, block)
  int32_t* tile_info;     // [16]: [0] tiles, [1] queue counter, [2] lists (G*nbw), [3] chunks per list,
                          // [4] workgroups of the KV-outer pass (written by it), [5] rows, [6] row0,
                          // [7] workgroups of the dense pass (written by it), [8..15] its per-XCD
                          // item counters (zeroed here)
  int tile_q;             // queries per tile
  int64_t tile_cap;
  int32_t* dense_cnt;     // [G][nunits]: blocks a 16-row unit computes in the dense pass
  int32_t* dense_list;    // [G][nunits][kDenseMax], ascending
  int32_t* dense_qmask;   // [G][nunits][kDenseMax]: bit r = row r of the unit selected the block
  int32_t* dense_slots;   // [G][nrows]: bit u = slot u of the row is computed in the dense pass
  int nunits;             // ceil(nrows / 16)
  bool dense;             // split off the dense pass's pairs (else list every pair; dense_* unused)
  int bk_shift;           // log2 B_k
  int32_t* tile_visits;   // [T_cap] (optional): zeroed for the tiles scheduled
};
void launch_csr_and_tiles(const LaunchCsr& a, hipStream_t st);

struct LaunchAttnPrefill {
  const uint16_t* q;      // [i - row0][Hq][128]
  const uint16_t* k;      // [position][G][128]
  const uint16_t* v;
  const int32_t* entries;
  const int32_t* tiles;
  int32_t* tile_info;
  uint16_t* part_o;       // [slot][2048] bf16 in fragment order, slot = (i_rel*G + g)*topk + u
  float* part_lse;        // [slot][16], log2 domain
  int64_t n_tokens;       // keys that exist (positions < n_tokens)
  int G, nbw, topk;
  float scale_log2;
  int grid;               // persistent workgroups (<= kMaxPersistent)
  int bk;                 // B_k: 128, 64 or 32
  int32_t* tile_visits;   // [T]: +1 for every claim of a tile
  int64_t* wg_trace;      // [grid][4]: hardware id, tiles drained, wall clock at start and end
};
void launch_attn_prefill(const LaunchAttnPrefill& a, hipStream_t st);

struct LaunchAttnDense {
  const uint16_t* q;      // [i - row0][Hq][128]
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* dense_cnt;
  const int32_t* dense_list;
  const int32_t* dense_qmask;
  const int32_t* dense_slots;
  const uint16_t* part_o; // KV-outer partials, merged into the output here
  const float* part_lse;
  uint16_t* out;          // window's first row
  float* lse_out;         // optional, window's first row
  int64_t n_tokens, row0;
  int nrows, nunits, G, topk;
  float scale_log2;
  int bk;
  int32_t* tile_info;     // [7]: grid (written), [8..15]: per-XCD item counters, zero before the pass
  int grid;               // persistent workgroups: a multiple of kXcd (8), at least 8
};
void launch_attn_dense(const LaunchAttnDense& a, hipStream_t st);

struct LaunchAttnDecode {
  const uint16_t* q;      // [batch, Hq, 128]
  const uint16_t* k;      // [batch, max_ctx, G, 128]
  const uint16_t* v;
  const int32_t* ctx_lens;
  const float* sblk;      // pooled index scores, row s*G + g of nb
  int nb;
  int32_t* sel_out;       // optional [(s*G + g)*topk + u]
  uint16_t* out;          // [batch, Hq, 128]
  float* lse_out;         // optional [batch, Hq]
  int64_t max_ctx;
  int batch, G, topk;
  float scale_log2;
  int bk;
};
void launch_attn_decode(const LaunchAttnDecode& a, hipStream_t st);

// Index Branch KL alignment, one window of rows [row0, row0 + nrows) of one
// sequence. Per-query arrays start at the window's first row; k, k_idx, loss
// and dk_idx are indexed by position.
struct LaunchKl {
  const uint16_t* q;      // [i - row0][Hq][128]
  const uint16_t* k;      // [position][G][128]
  const uint16_t* q_idx;  // [i - row0][G][64]
  const uint16_t* k_idx;  // [position][64]
  const float* lse;       // [i - row0][Hq], natural log
  const int32_t* entries; // reverse index of every selected pair
  const int32_t* chunks;  // [chunk][4] = (group, begin, len, block)
  const int32_t* chunk_info;  // [0] chunks
  int64_t chunk_cap;      // grid size (>= chunks)
  float* part_m;          // [slot], slot = (i_rel*G + g)*topk + u
  float* part_l;
  float* loss_part;
  float* dq_part;         // [slot][64]
  float* lse_idx;         // [i_rel*G + g]
  float* loss;            // [G][n_tokens]
  float* dq_idx;          // [i - row0][G][64]
  float* dk_idx;          // [position][64], accumulated over windows
  float* dk_part;         // [chunk][128][64]: each chunk's dk_idx rows
  const int32_t* tile_start;  // [G*nbw + 1]: first chunk of each (group, block) list
  int64_t n_tokens, row0;
  int nrows, nbw, G, topk;
  float scale_log2;
};
void launch_kl_window(const LaunchKl& a, hipStream_t st);
void launch_zero_f32(float* p, int64_t n, hipStream_t st);

// Index Branch projections (one GEMM for the G query heads and the key head).
struct LaunchProject {
  const uint16_t* x;      // [n][d_model]
  const uint16_t* w_qi;   // [G*64][d_model]
  const uint16_t* w_ki;   // [64][d_model]
  int64_t n;
  int d_model, G;
  uint16_t* q_idx;        // [n][G][64]
  uint16_t* k_idx;        // key head rows: t, or t*max_ctx + ctx_lens[t]-1 when ctx_lens is set
  const int32_t* ctx_lens;
  int64_t max_ctx;
  float* part;            // fp32 partials when d_model is split (plan.part_floats floats)
};
struct ProjectPlan {
  int parts, nc;          // column parts and 64-column units per workgroup
  int64_t m_tiles;        // 128-token tiles
  int splits, stages_per_split;
  size_t part_floats;     // scratch for split partials (0: none)
  bool ws = false;        // many tokens, d_model a multiple of 256: k_index_project_ws
};
ProjectPlan plan_index_project(int64_t n, int d_model, int G);
void launch_index_project(const LaunchProject& a, hipStream_t st);


}  // namespace msa
