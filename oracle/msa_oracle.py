"""Plain float64 CPU oracle for MiniMax Sparse Attention (MSA): block selection
(Index Branch) and exact softmax attention over the selected blocks (Main Branch).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
this module: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg use it. It shares no code with the HIP path; the only common dependency is
the seeded input generator module ``msa_synth``.

Sources (the pages the method is defined on; cited below by short key):

  [pnsm]  "MiniMax Sparse Attention：一篇读懂百万上下文时代的稀疏注意力工程化路线"
          (pnsm.cn explainer), sections 2 (group-specific block selection),
          7 (kernel design) and 9 (efficiency).
  [yifor] "MiniMax Sparse Attention (MSA): a Two-Branch Block-Sparse Attention
          Trained on a 109B-Parameter MoE With a 3T-Token Budget" (yifor-blog),
          section "設計核心" (two branches) and "從 O(N) 降至 O(kB_k)".
  [yhxrc] yhxrc.cn comparison of MSA/NSA/DSA/MoBA, section 二 "MSA是怎么做的".

What is computed, per query row i (0-based position), for each GQA group g:

 1. Score [pnsm §7; yhxrc §二]: raw index scores s_j = q_idx[i,g,:] . k_idx[j,:]
    for every key j in a block older than i's own block. No scale, no softmax:
    softmax keeps the order of the scores, so ranking on raw scores selects the
    same blocks.
 2. Pool [yifor "設計核心"; yhxrc §二]: the score of block b is the maximum of
    s_j over the B_k keys of block b (block max-pooling).
 3. Select [pnsm §2; yhxrc §二]: the block holding i, b_loc = floor(i/B_k), is
    always selected and counts inside the k; the other k-1 are the highest
    pooled scores among blocks 0..b_loc-1. Readings where the pages are silent:
    ties go to the lower block index; with fewer than k-1 older blocks all of
    them are taken. The selection is emitted ascending, padded with -1.
 4. Attend [pnsm §2; yifor "設計核心"; yhxrc §二]: exact softmax attention of
    each query head h of group g (h in [g*hpg, (g+1)*hpg)) over the token set
    T = {j <= i : floor(j/B_k) in Sel}; z_j = scale * q[i,h,:] . k[j,g,:],
    out = sum_T softmax(z)_j v[j,g,:], lse = ln sum_T exp(z_j). Evaluated with
    the maximum subtracted (the log-sum-exp identity) in float64.

Decode is the same computation for the single row i = ctx_len - 1 of each
sequence, over that sequence's cache.

Pins (tests/test_oracle_pins.py, tests/golden/): dense causal GQA attention when
k covers every block (checked against an independent textbook implementation
and torch's scaled_dot_product_attention in float64), brute-force selection by
subset enumeration on tiny tied inputs, invariants, planted-needle recall, a
hand-derived worked case in tests/golden/, metamorphic checks, the k=1 and
B_k=1 special cases, and masked-SDPA equality in the general case.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np


def to_f64(x) -> np.ndarray:
    """Exact upcast of a bfloat16/float tensor (torch or numpy) to float64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Index Branch
# ---------------------------------------------------------------------------

def block_scores(q_idx_row: np.ndarray, k_idx_prefix: np.ndarray, block_size: int) -> np.ndarray:
    """Steps 1-2 for one query row.

    q_idx_row: [G, d_idx]; k_idx_prefix: [n_blocks*B_k, d_idx], the keys of the
    blocks older than the query's own block. Returns S [G, n_blocks] with
    S[g, b] = max over j in block b of q_idx_row[g] . k_idx[j].
    """
    G = q_idx_row.shape[0]
    J = k_idx_prefix.shape[0]
    assert J % block_size == 0
    nblk = J // block_size
    if nblk == 0:
        return np.zeros((G, 0))
    s = k_idx_prefix @ q_idx_row.T                    # [J, G] raw scores
    return s.reshape(nblk, block_size, G).max(axis=1).T  # [G, n_blocks]


def select_blocks(S_g: np.ndarray, b_loc: int, k: int) -> np.ndarray:
    """Step 3 for one (row, group): local block plus the top k-1 older blocks.

    S_g: pooled scores of blocks 0..b_loc-1. Returns int array [k], ascending,
    -1 padded.
    """
    cand = np.arange(b_loc)
    if b_loc <= k - 1:
        chosen = cand
    else:
        order = np.lexsort((cand, -S_g[:b_loc]))  # primary: score desc; ties: index asc
        chosen = cand[order[:k - 1]]
    sel = np.sort(np.concatenate([chosen, [b_loc]]).astype(np.int64))
    out = np.full(k, -1, dtype=np.int64)
    out[:sel.size] = sel
    return out


# ---------------------------------------------------------------------------
# Main Branch
# ---------------------------------------------------------------------------

def token_set(sel: np.ndarray, i: int, block_size: int) -> np.ndarray:
    """T = {j <= i : floor(j / B_k) in sel}, ascending."""
    js = []
    for b in sel:
        if b < 0:
            continue
        lo = b * block_size
        hi = min((b + 1) * block_size, i + 1)
        if hi > lo:
            js.append(np.arange(lo, hi))
    return np.concatenate(js) if js else np.zeros(0, dtype=np.int64)


def attend(q_heads: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Exact softmax attention of several heads over one token set.

    q_heads [H, d], keys [T, d], values [T, d] -> (out [H, d], lse [H]).
    """
    z = scale * (q_heads @ keys.T)              # [H, T]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    denom = e.sum(axis=1, keepdims=True)
    out = (e @ values) / denom
    lse = (m + np.log(denom))[:, 0]
    return out, lse


# ---------------------------------------------------------------------------
# Whole rows
# ---------------------------------------------------------------------------

def prefill_rows(rows: Sequence[int], q_rows: np.ndarray, q_idx_rows: np.ndarray,
                 k_idx: np.ndarray, k: np.ndarray, v: np.ndarray, *,
                 block_size: int, topk: int, scale: Optional[float] = None,
                 want_scores: bool = False) -> Dict[str, np.ndarray]:
    """Oracle for the given query rows of one sequence.

    q_rows [R, Hq, d] and q_idx_rows [R, G, d_idx] hold the sampled rows only;
    k_idx [>=N, d_idx], k and v [>=N, G, d] hold the whole sequence (only
    positions <= max(rows) are read). Returns sel [R, G, topk] (int64),
    out [R, Hq, d], lse [R, Hq] and, if asked, the pooled scores as a list of
    [G, b_loc] arrays.
    """
    rows = [int(r) for r in rows]
    R = len(rows)
    Hq, d = q_rows.shape[1], q_rows.shape[2]
    G = q_idx_rows.shape[1]
    hpg = Hq // G
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sel = np.full((R, G, topk), -1, dtype=np.int64)
    out = np.zeros((R, Hq, d))
    lse = np.zeros((R, Hq))
    scores = []
    for r, i in enumerate(rows):
        b_loc = i // block_size
        S = block_scores(q_idx_rows[r], k_idx[:b_loc * block_size], block_size)
        if want_scores:
            scores.append(S)
        for g in range(G):
            sel[r, g] = select_blocks(S[g], b_loc, topk)
            T = token_set(sel[r, g], i, block_size)
            heads = slice(g * hpg, (g + 1) * hpg)
            o, l = attend(q_rows[r, heads], k[T, g], v[T, g], scale)
            out[r, heads] = o
            lse[r, heads] = l
    res = {"sel": sel, "out": out, "lse": lse}
    if want_scores:
        res["scores"] = scores
    return res


def decode_seq(q: np.ndarray, q_idx: np.ndarray, k_idx_cache: np.ndarray,
               k_cache: np.ndarray, v_cache: np.ndarray, ctx_len: int, *,
               block_size: int, topk: int, scale: Optional[float] = None,
               want_scores: bool = False) -> Dict[str, np.ndarray]:
    """Oracle for one decode step of one sequence: the new token is cache row
    ctx_len-1 (already appended), so decode equals prefill row i = ctx_len-1.

    q [Hq, d], q_idx [G, d_idx]; caches hold at least ctx_len rows.
    Returns sel [G, topk], out [Hq, d], lse [Hq] (and scores [G, b_loc]).
    """
    res = prefill_rows([ctx_len - 1], q[None], q_idx[None], k_idx_cache, k_cache, v_cache,
                       block_size=block_size, topk=topk, scale=scale, want_scores=want_scores)
    out = {"sel": res["sel"][0], "out": res["out"][0], "lse": res["lse"][0]}
    if want_scores:
        out["scores"] = res["scores"][0]
    return out
