/*
 * msa.h - C ABI of the MI355X (gfx950) MiniMax Sparse Attention hot path.
 *
 * MSA replaces dense causal attention with two branches [yifor, 設計核心;
 * yhxrc, 二 "MSA是怎么做的"; pnsm, section 2]:
 *   Index Branch - for every query token i and GQA group g, raw (exp-free)
 *     scores q_idx[i,g] . k_idx[j] over earlier keys, max-pooled per block of
 *     B_k keys; the query's own block floor(i/B_k) is always selected and the
 *     other k-1 blocks are the best-scoring older blocks (ties: lower index).
 *   Main Branch - exact softmax attention of the group's query heads over the
 *     tokens j <= i of the selected blocks only.
 * The prefill main branch is organised KV-outer ("outer gather Q") [pnsm,
 * section 7; yhxrc, 二; yololab, "KV Outer Gather Q是什麼？"]: each selected
 * (group, KV block) is staged once and every query that selected it is
 * computed against it, producing softmax partials that a second pass merges
 * without atomics ("two-phase combine", [pnsm, section 7]).
 *
 * Page keys used in citations:
 *   [pnsm]    "MiniMax Sparse Attention：一篇读懂百万上下文时代的稀疏注意力工程化路线" (pnsm.cn)
 *   [yifor]   "MiniMax Sparse Attention (MSA): a Two-Branch Block-Sparse Attention Trained
 *             on a 109B-Parameter MoE With a 3T-Token Budget" (yifor-blog)
 *   [yhxrc]   MSA/NSA/DSA/MoBA comparison article (yhxrc.cn)
 *   [yololab] MiniMax M3 / MSA overview (yololab.net)
 *
 * Conventions for every entry point:
 *   - All tensors are device pointers to contiguous row-major memory, 16-byte
 *     aligned; bf16 means IEEE bfloat16 stored as uint16.
 *   - The caller owns every buffer (inputs, outputs, workspace). The library
 *     never allocates or frees device memory; all work is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream) and the call returns at once
 *     (the *_profiled variants below are the exception: they create HIP
 *     events and synchronise on them before returning).
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error status nothing has been launched. MSA_ERR_HIP reports a failed
 *     launch (hipGetLastError); asynchronous device faults surface at the
 *     caller's next synchronisation.
 *   - Calls are reentrant; concurrent calls need distinct workspaces.
 *   - Supported shapes: head_dim 128, index_dim 64, block_size 128, 64 or 32
 *     (the block sizes the pages ablate [pnsm, section 8: block-size ablation
 *     in its evidence table]), num_q_heads / num_kv_heads == 16,
 *     1 <= num_kv_heads <= 8, 1 <= topk <= 16. Sequences and contexts hold at
 *     most 2^20 * block_size / 128 positions (2^20, 2^19, 2^18). The
 *     KL-alignment backward takes block_size 128 only. Anything else returns
 *     MSA_ERR_UNSUPPORTED.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1,        /* null/misaligned pointer, non-positive size, Hq % Hkv != 0 */
  MSA_ERR_UNSUPPORTED = -2,        /* a shape outside the supported set above */
  MSA_ERR_WORKSPACE_TOO_SMALL = -3,
  MSA_ERR_HIP = -4
} msa_status;

typedef struct {
  int32_t num_q_heads;   /* Hq: query heads (64 in the pages' model, section 8 of [pnsm]) */
  int32_t num_kv_heads;  /* G: KV heads = GQA groups = index query heads (4) */
  int32_t head_dim;      /* d = 128 */
  int32_t index_dim;     /* d_idx = 64: width of q_idx / k_idx */
  int32_t block_size;    /* B_k keys per selectable block: 128 [pnsm, section 2], 64 or 32 */
  int32_t topk;          /* k blocks per (query, group), the forced local block included (16) */
  float softmax_scale;   /* main-branch logit scale; <= 0 selects 1/sqrt(head_dim) */
} msa_params;

/* Bytes of device workspace msa_prefill needs for `batch` sequences of
 * `seq_len` tokens (the same for any batch: sequences are processed in turn).
 * Returns 0 for invalid or unsupported arguments. Query rows are processed in
 * windows of at most 65536; the workspace is dominated by the KV-outer
 * partials, sized for every (row, group, slot) of one window (4160 bytes
 * each: 16 heads x 128 bf16 plus 16 fp32 lse), and by the pooled block scores
 * of a window, which grow with the sequence. At 4 groups and k = 16: 1.0 GiB
 * at 4K tokens, 8.3 GiB at 32K, 16.8 GiB at 64K, 17.3 GiB at 128K, 24.5 GiB
 * at 1M. */
size_t msa_prefill_workspace_bytes(const msa_params* p, int32_t batch, int64_t seq_len);

/* Causal MSA prefill of `batch` independent sequences of `seq_len` tokens: for
 * every query row and group, the Index Branch selects the own block plus the
 * k-1 best-scoring older blocks, and the Main Branch computes exact softmax
 * attention over the selected blocks' tokens at or before the row [pnsm,
 * section 2: group-specific block selection; yhxrc, 二 "MSA是怎么做的"].
 *   q      bf16 [batch, seq_len, Hq, d]       query heads; head h belongs to group h / 16
 *   k, v   bf16 [batch, seq_len, G, d]        main-branch keys / values
 *   q_idx  bf16 [batch, seq_len, G, d_idx]    one index query head per group
 *   k_idx  bf16 [batch, seq_len, d_idx]       the shared index key head
 *   out    bf16 [batch, seq_len, Hq, d]       attention output (fp32 accumulation,
 *                                              rounded to nearest even)
 *   sel_out  optional int32 [batch, G, seq_len, topk]: selected block ids per
 *            (group, query), ascending, padded with -1 (NULL: not written)
 *   lse_out  optional fp32 [batch, seq_len, Hq]: natural-log sum of exp of the
 *            scaled logits over the attended tokens (NULL: not written)
 *   workspace  >= msa_prefill_workspace_bytes(p, batch, seq_len) bytes
 * Block selection is exact for index projections whose dot products are exact
 * in fp32 (e.g. small integers); ties go to the lower block index. */
msa_status msa_prefill(const msa_params* p, int32_t batch, int64_t seq_len,
                       const void* q, const void* k, const void* v,
                       const void* q_idx, const void* k_idx,
                       void* out, int32_t* sel_out, float* lse_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace msa_prefill_varlen needs when no sequence has more
 * than max_q_len query rows and caches hold max_ctx positions. Returns 0 for
 * invalid or unsupported arguments. */
size_t msa_prefill_varlen_workspace_bytes(const msa_params* p, int64_t max_q_len, int64_t max_ctx);

/* Prefill of `batch` sequences of different lengths, each a chunk of query
 * rows that continues an existing cache: sequence b's rows are the positions
 * [q_start[b], q_start[b] + q_len[b]), and each attends causally to the cache
 * positions 0 .. its own position. q_start[b] = 0 is a fresh prompt; a chunk
 * split into pieces gives every row the same result as one call over the
 * whole (up to fp32 rounding order in the attention; the selection is the
 * same), since row i depends only on positions <= i [yifor, 設計核心;
 * pnsm, section 2]. As in decode, the chunk's K, V and k_idx must already be
 * in the caches at its positions.
 *   q_start, q_len  HOST int64 [batch]: q_start >= 0, q_len >= 0 (0: nothing for
 *                   that sequence), q_start + q_len <= max_ctx
 *   q      bf16 [T, Hq, d] with T = sum of q_len: the sequences' rows packed in
 *          order (sequence b starts at row sum_{b'<b} q_len[b'])
 *   q_idx  bf16 [T, G, d_idx]
 *   k_cache, v_cache  bf16 [batch, max_ctx, G, d]
 *   k_idx_cache       bf16 [batch, max_ctx, d_idx]
 *   out      bf16 [T, Hq, d]
 *   sel_out  optional int32 [G, T, topk] (ascending, -1 padded)
 *   lse_out  optional fp32 [T, Hq]
 *   workspace  >= msa_prefill_varlen_workspace_bytes(p, max q_len, max_ctx) bytes
 * T = 0 returns MSA_OK at once. max_ctx above the longest supported context
 * (2^20 at block_size 128) is MSA_ERR_UNSUPPORTED. */
msa_status msa_prefill_varlen(const msa_params* p, int32_t batch, int64_t max_ctx,
                              const int64_t* q_start, const int64_t* q_len,
                              const void* q, const void* q_idx,
                              const void* k_cache, const void* v_cache, const void* k_idx_cache,
                              void* out, int32_t* sel_out, float* lse_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ---- Schedule inspection ---------------------------------------------------
 * Where a prefill workspace keeps the reverse index and the tile schedule of
 * the KV-outer pass [pnsm, section 7 "outer gather Q" and section 9: reverse
 * index, pre-scheduled tile chunking, persistent work queue], for checks and
 * load-balance diagnostics. Once a msa_prefill / msa_prefill_varlen call has
 * completed on its stream, these arrays describe the LAST window it processed
 * (a window is a run of at most 65536 query rows of one sequence; a call of one
 * sequence of up to 65536 rows starting at a multiple of 16 has exactly one).
 * All offsets are bytes from the start of the workspace; n is the window's rows,
 * nbw the blocks its rows can see, nch = ceil(n / 64), units = ceil(n / 16).
 * Nothing here is read by the library after the call: writing it is harmless. */
typedef struct {
  int64_t tile_info;   /* int32 [16]: [0] tiles T, [1] the queue counter after the pass
                          (claims * claim), [2] lists = G * nbw, [3] nch,
                          [4] workgroups of the KV-outer pass, [5] n, [6] first row,
                          [7] workgroups of the dense pass, [8 + r] the claim counter
                          of its item range r (r < 8; G * units items in 8 ranges
                          of floor or ceil(G * units / 8) items, range r >= its
                          size after the pass: failed claims count too) */
  int64_t chunk_off;   /* int32 [lists * nch + 1]: exclusive scan of the KV-outer pair
                          counts of each (group g, block b, chunk of 64 rows), list
                          l = g * nbw + b first; list l holds entries
                          [chunk_off[l * nch], chunk_off[(l + 1) * nch]) */
  int64_t entries;     /* int32: row in the window << 4 | slot u, rows ascending in a list */
  int64_t tiles;       /* int32 [T][4]: group, first entry, entry count (<= tile_queries), block */
  int64_t tile_visits; /* int32 [T]: how many times the KV-outer pass computed each tile */
  int64_t wg_trace;    /* int64 [workgroups][4] of the KV-outer pass: hardware id
                          (xcc << 6 | shader engine << 4 | compute unit), tiles it
                          computed, wall clock at its start and at its end */
  int64_t dense_cnt;   /* int32 [G][units]: blocks the 16-row unit computes in the
                          query-stationary (dense) pass */
  int64_t dense_list;  /* int32 [G][units][dense_max]: those blocks, ascending */
  int64_t dense_qmask; /* int32 [G][units][dense_max]: bit r = row r of the unit selected it */
  int64_t dense_slots; /* int32 [G][n]: bit u = slot u of the row is computed in the dense pass */
  int32_t dense_max;
  int32_t tile_queries;
  int32_t claim;       /* tiles per claim from the queue */
  int32_t dense_min;   /* a unit's block goes to the dense pass when at least
                          min(dense_min, rows of the unit) of its rows selected it */
  int64_t wall_clock_khz; /* rate of the wg_trace clock (0 if the device does not report it) */
} msa_prefill_schedule_map;

/* Fills *m for the workspace of a prefill whose longest sequence has max_q_len
 * query rows and whose longest context is max_ctx positions (msa_prefill:
 * max_q_len = max_ctx = seq_len). MSA_ERR_INVALID_ARG for a NULL m or
 * non-positive sizes, MSA_ERR_UNSUPPORTED where the workspace-size functions
 * return 0. Host only; wall_clock_khz is queried from the current device. */
msa_status msa_prefill_schedule_layout(const msa_params* p, int64_t max_q_len, int64_t max_ctx,
                                       msa_prefill_schedule_map* m);

/* Bytes of device workspace msa_decode needs. Returns 0 on invalid arguments
 * and for max_ctx above the longest supported context. */
size_t msa_decode_workspace_bytes(const msa_params* p, int32_t batch, int64_t max_ctx);

/* One decode step for `batch` sequences. Decode is prefill's last row: the new
 * token's K, V and k_idx must already be appended to the caches at row
 * ctx_lens[b]-1, and its query attends causally to rows 0..ctx_lens[b]-1
 * [yhxrc, 二: the index re-scores and re-selects blocks for every new token].
 *   q            bf16 [batch, Hq, d]           the new token's query heads
 *   q_idx        bf16 [batch, G, d_idx]        the new token's index query heads
 *   k_cache, v_cache  bf16 [batch, max_ctx, G, d]
 *   k_idx_cache  bf16 [batch, max_ctx, d_idx]
 *   ctx_lens     device int32 [batch], 1 <= ctx_lens[b] <= max_ctx (device values
 *                are not checked on the host; out-of-range values are undefined);
 *                cache positions >= ctx_lens[b] are never read
 *   out          bf16 [batch, Hq, d]
 *   sel_out      optional int32 [batch, G, topk] (ascending, -1 padded)
 *   lse_out      optional fp32 [batch, Hq]
 * max_ctx above the longest supported context (2^20 * block_size / 128) is
 * MSA_ERR_UNSUPPORTED. */
msa_status msa_decode(const msa_params* p, int32_t batch, int64_t max_ctx,
                      const void* q, const void* q_idx,
                      const void* k_cache, const void* v_cache, const void* k_idx_cache,
                      const int32_t* ctx_lens,
                      void* out, int32_t* sel_out, float* lse_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- Decode without allocation -------------------------------------------
 * For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): msa_decode with
 * the same arguments minus the workspace, which comes from a fixed device
 * array of MSA_DECODE_NOALLOC_WORKSPACE_BYTES that the library holds on each
 * device it runs on (from the first call there until the process ends). A
 * call whose msa_decode_workspace_bytes exceeds it returns
 * MSA_ERR_UNSUPPORTED (the pooled block scores: 64 sequences at 128K
 * positions take 1 MiB, 8 at 1M 1 MiB; at most 512 sequences of 128K fit).
 * Calls on one device share the array: calls that overlap in time on one
 * device race (serialise them on one stream). The results are those of
 * msa_decode: the same kernels run. */
#define MSA_DECODE_NOALLOC_WORKSPACE_BYTES ((size_t)8 << 20)
msa_status msa_decode_noalloc(const msa_params* p, int32_t batch, int64_t max_ctx,
                              const void* q, const void* q_idx,
                              const void* k_cache, const void* v_cache, const void* k_idx_cache,
                              const int32_t* ctx_lens,
                              void* out, int32_t* sel_out, float* lse_out, void* stream);

/* ---- Profiling variants -------------------------------------------------
 * Same work and arguments as msa_prefill / msa_decode, plus HIP events recorded
 * on `stream` at every stage boundary. They synchronise on the last event and
 * return in stage_ms the duration of each stage, summed over sequences and
 * windows:
 *   prefill (5): index scores, top-k selection, reverse index + tile schedule,
 *                KV-outer attention, attention over the blocks each 16-row
 *                unit shares with the merge of the KV-outer partials (combine)
 *   decode  (2): index scores; top-k selection with the attention over the
 *                selected blocks of each sequence and group (one kernel:
 *                each workgroup ranks its own row, then merges the blocks
 *                as they stream)
 * stage_ms must not be NULL (MSA_ERR_INVALID_ARG).
 *
 * The *_timed variants record the same stage events but return at once,
 * without synchronising (so back-to-back calls keep the GPU busy): *timer
 * receives a handle that msa_stage_timer_read later turns into stage_ms
 * (waiting for the call's last event) and releases. Every handle must be
 * read exactly once; on an error status no handle is returned. */
msa_status msa_prefill_profiled(const msa_params* p, int32_t batch, int64_t seq_len,
                                const void* q, const void* k, const void* v,
                                const void* q_idx, const void* k_idx,
                                void* out, int32_t* sel_out, float* lse_out,
                                void* workspace, size_t workspace_bytes, void* stream,
                                float* stage_ms);
typedef struct msa_stage_timer msa_stage_timer;
msa_status msa_prefill_timed(const msa_params* p, int32_t batch, int64_t seq_len,
                             const void* q, const void* k, const void* v,
                             const void* q_idx, const void* k_idx,
                             void* out, int32_t* sel_out, float* lse_out,
                             void* workspace, size_t workspace_bytes, void* stream,
                             msa_stage_timer** timer);
msa_status msa_decode_timed(const msa_params* p, int32_t batch, int64_t max_ctx,
                            const void* q, const void* q_idx,
                            const void* k_cache, const void* v_cache, const void* k_idx_cache,
                            const int32_t* ctx_lens,
                            void* out, int32_t* sel_out, float* lse_out,
                            void* workspace, size_t workspace_bytes, void* stream,
                            msa_stage_timer** timer);
msa_status msa_stage_timer_read(msa_stage_timer* timer, float* stage_ms);
msa_status msa_decode_profiled(const msa_params* p, int32_t batch, int64_t max_ctx,
                               const void* q, const void* q_idx,
                               const void* k_cache, const void* v_cache, const void* k_idx_cache,
                               const int32_t* ctx_lens,
                               void* out, int32_t* sel_out, float* lse_out,
                               void* workspace, size_t workspace_bytes, void* stream,
                               float* stage_ms);

/* ---- Index Branch training signal ------------------------------------------
 * KL alignment of the Index Branch to the Main Branch [pnsm, section 4: the
 * main branch's attention on the selected support is the teacher, gradients
 * reach only the index projections; yhxrc, 二]. For one sequence, per query
 * row i and group g with support T = {j <= i : floor(j/B_k) in sel[g, i]}:
 *   P_main(j) = mean over the group's query heads h of exp(scale q[i,h].k[j,g] - lse[i,h])
 *   P_idx(j)  = softmax over T of q_idx[i,g] . k_idx[j]
 *   loss[g, i] = KL(P_main || P_idx)
 * and the gradients of sum_{g,i} loss[g, i] with respect to q_idx and k_idx
 * only: dq_idx[i,g] = sum_T (P_idx - P_main)(j) k_idx[j] and
 * dk_idx[j] = sum over (i, g) with j in T of (P_idx - P_main)(j) q_idx[i,g].
 *   q, k      bf16 [seq_len, Hq, d], [seq_len, G, d]   (as passed to msa_prefill)
 *   q_idx     bf16 [seq_len, G, d_idx];  k_idx bf16 [seq_len, d_idx]
 *   sel       int32 [G, seq_len, topk]  msa_prefill's sel_out (ascending, -1 padded)
 *   lse       fp32 [seq_len, Hq]        msa_prefill's lse_out (natural log), 16-byte aligned
 *   loss      fp32 [G, seq_len]
 *   dq_idx    fp32 [seq_len, G, d_idx]  (written)
 *   dk_idx    fp32 [seq_len, d_idx]     (written; summed in a fixed order, so the
 *                                        result is the same on every call)
 *   workspace >= msa_index_kl_workspace_bytes(p, seq_len) bytes
 * The teacher uses the forward's lse, so P_main is the forward's attention
 * distribution up to its rounding. Returns 0 / an error status as above. */
size_t msa_index_kl_workspace_bytes(const msa_params* p, int64_t seq_len);
msa_status msa_index_kl_backward(const msa_params* p, int64_t seq_len,
                                 const void* q, const void* k, const void* q_idx, const void* k_idx,
                                 const int32_t* sel, const float* lse,
                                 float* loss, float* dq_idx, float* dk_idx,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ---- Index Branch projections ----------------------------------------------
 * The index heads are linear maps of the layer's hidden states: one index query
 * head per group and one index key head shared by all groups [yhxrc, 二; yifor,
 * 工程實踐啟示: the branch adds two projection matrices]. One call computes
 * both from one read of x (no bias or activation; fp32 accumulation, outputs
 * rounded to bf16, nearest even):
 *   q_idx[t, g, :] = W_qi[g] x[t],   k_idx row of token t = W_ki x[t]
 *   x      bf16 [n_tokens, d_model]      hidden states; d_model a multiple of 64,
 *                                        64 .. 65536 (else MSA_ERR_UNSUPPORTED)
 *   w_qi   bf16 [G, d_idx, d_model]      (out_features x in_features)
 *   w_ki   bf16 [d_idx, d_model]
 *   q_idx  bf16 [n_tokens, G, d_idx]     written
 *   k_idx  bf16 [n_tokens, d_idx]        written (msa_index_project), or
 *   k_idx_cache bf16 [batch, max_ctx, d_idx]: row ctx_lens[b]-1 of sequence b
 *                                        written, no other row touched
 *                                        (msa_index_project_decode: the decode
 *                                        step's key appended to its cache)
 *   workspace  >= msa_index_project_workspace_bytes(p, n_tokens, d_model) bytes
 *              (scratch for small n_tokens, where d_model is split across
 *              workgroups and the partials summed in a fixed order)
 * Every pointer 16-byte aligned, the workspace 256-byte aligned. n_tokens up
 * to 2^28. For a chunk of a longer sequence, pass k_idx at its first cache
 * row. Results do not depend on the stream's other work or on earlier calls. */
size_t msa_index_project_workspace_bytes(const msa_params* p, int64_t n_tokens, int32_t d_model);
msa_status msa_index_project(const msa_params* p, int64_t n_tokens, int32_t d_model,
                             const void* x, const void* w_qi, const void* w_ki,
                             void* q_idx, void* k_idx,
                             void* workspace, size_t workspace_bytes, void* stream);
msa_status msa_index_project_decode(const msa_params* p, int32_t batch, int64_t max_ctx, int32_t d_model,
                                    const void* x, const void* w_qi, const void* w_ki,
                                    const int32_t* ctx_lens, void* q_idx, void* k_idx_cache,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ---- Stage entry points (Index Branch only) ------------------------------
 * For callers that need the selection alone, and for per-stage parity tests. */

/* Pooled index scores [yifor, 設計核心: max-pooling per block] of one sequence:
 *   scores fp32 [seq_len, G, nb] with nb = ceil(seq_len / block_size).
 * For every query row i whose own block b_loc = i / B_k is >= topk (rows that
 * have more than k-1 older blocks to choose from), scores[i, g, b] for
 * b < b_loc is max over keys j of block b of q_idx[i,g] . k_idx[j]. Every other
 * entry is left untouched. No workspace. */
msa_status msa_index_scores(const msa_params* p, int64_t seq_len,
                            const void* q_idx, const void* k_idx,
                            float* scores, void* stream);

/* Top-k selection [pnsm, section 7: exp-free top-k; yhxrc, 二] from pooled
 * scores laid out as msa_index_scores writes them:
 *   sel_out int32 [G, seq_len, topk]: the block b_loc plus the topk-1 best older
 *   blocks (ties: lower index), ascending, -1 padded. Rows with b_loc < topk
 *   select every block 0..b_loc and never read `scores`. No workspace. */
msa_status msa_select_blocks(const msa_params* p, int64_t seq_len,
                             const float* scores, int32_t* sel_out, void* stream);

/* Human-readable name of a status code (static storage). */
const char* msa_status_string(msa_status s);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
