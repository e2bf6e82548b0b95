"""Plain float64 CPU oracle of the Index Branch's KL-alignment training signal.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
this module: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg use it. It shares no code with the HIP path.

Sources (cited by short key, as in msa_oracle):
  [pnsm]  "MiniMax Sparse Attention：一篇读懂百万上下文时代的稀疏注意力工程化路线"
          (pnsm.cn), section 4 (training signals: KL alignment and gradient
          detach).
  [yhxrc] yhxrc.cn comparison of MSA/NSA/DSA/MoBA, section 二 (the index branch
          takes the main branch's attention distribution as its teacher, KL
          alignment on the selected blocks, gradients kept out of the backbone).

What is computed, per query row i and GQA group g, on the support
T = T(i, g) = {j <= i : floor(j / B_k) in Sel[g, i]} chosen by the Index Branch:

  teacher  P_main(j) = (1/hpg) * sum over the group's query heads h of
                       softmax_{j in T}(scale * q[i,h] . k[j,g])
  student  P_idx(j)  = softmax_{j in T}(q_idx[i,g] . k_idx[j])
  loss     L(i, g)   = KL(P_main || P_idx) = sum_T P_main * (log P_main - log P_idx)

and the gradients of sum_{i,g} L(i, g) with respect to q_idx and k_idx only
(the main branch is detached [pnsm section 4; yhxrc 二]):

  dL/ds_j      = P_idx(j) - P_main(j)                 (s_j = q_idx[i,g] . k_idx[j])
  dq_idx[i,g]  = sum_{j in T} (P_idx(j) - P_main(j)) k_idx[j]
  dk_idx[j]   += (P_idx(j) - P_main(j)) q_idx[i,g]    for every (i, g) with j in T(i, g)

Readings where the pages are silent (listed in the design notes too): the
teacher is the mean of the group's head distributions (one index head serves
the group); the student's logits are the raw index scores the selection ranks
(no temperature); the divergence is teacher-to-student; the loss is summed
over (i, g). Terms with P_main(j) = 0 contribute 0.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from oracle.msa_oracle import block_scores, select_blocks, token_set


def _softmax(x: np.ndarray) -> np.ndarray:
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def row_terms(q_heads: np.ndarray, keys: np.ndarray, q_idx_g: np.ndarray, k_idx_T: np.ndarray,
              scale: float):
    """KL terms of one (row, group) on its support T.

    q_heads [hpg, d] (the group's query heads), keys [T, d], q_idx_g [d_idx],
    k_idx_T [T, d_idx]. Returns (loss, grad_s [T]) with grad_s = P_idx - P_main.
    """
    p_main = _softmax(scale * (q_heads @ keys.T)).mean(axis=0)   # [T]
    s = k_idx_T @ q_idx_g                                        # [T]
    log_p_idx = s - (s.max() + np.log(np.exp(s - s.max()).sum()))
    pos = p_main > 0
    loss = float(np.sum(p_main[pos] * (np.log(p_main[pos]) - log_p_idx[pos])))
    return loss, np.exp(log_p_idx) - p_main


def index_kl(q: np.ndarray, k: np.ndarray, q_idx: np.ndarray, k_idx: np.ndarray, *, block_size: int,
             topk: int, scale: Optional[float] = None, sel: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """KL alignment of one sequence: every row, every group.

    q [N, Hq, d], k [N, G, d], q_idx [N, G, d_idx], k_idx [N, d_idx] (float64).
    sel [N, G, topk] (optional): the selection to use; computed here from the
    index scores (msa_oracle's steps 1-3) when not given.
    Returns loss [G, N], dq_idx [N, G, d_idx], dk_idx [N, d_idx], sel [N, G, topk].
    """
    N, Hq, d = q.shape
    G = k.shape[1]
    hpg = Hq // G
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    loss = np.zeros((G, N))
    dq = np.zeros(q_idx.shape)
    dk = np.zeros(k_idx.shape)
    sel_out = np.full((N, G, topk), -1, dtype=np.int64)
    for i in range(N):
        b_loc = i // block_size
        if sel is None:
            S = block_scores(q_idx[i], k_idx[:b_loc * block_size], block_size)
        for g in range(G):
            sg = select_blocks(S[g], b_loc, topk) if sel is None else np.asarray(sel[i, g])
            sel_out[i, g] = sg
            T = token_set(sg, i, block_size)
            l, gs = row_terms(q[i, g * hpg:(g + 1) * hpg], k[T, g], q_idx[i, g], k_idx[T], scale)
            loss[g, i] = l
            dq[i, g] = gs @ k_idx[T]
            dk[T] += np.outer(gs, q_idx[i, g])
    return {"loss": loss, "dq_idx": dq, "dk_idx": dk, "sel": sel_out}


def index_kl_rows(rows, q_rows: np.ndarray, q_idx_rows: np.ndarray, k: np.ndarray, k_idx: np.ndarray, *,
                  block_size: int, topk: int, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Loss [R, G] and dq_idx [R, G, d_idx] of the given rows only (each row's
    terms depend on its own inputs and the keys before it). k_idx and k hold
    the whole sequence; q_rows [R, Hq, d], q_idx_rows [R, G, d_idx]."""
    R = len(rows)
    Hq, d = q_rows.shape[1], q_rows.shape[2]
    G = q_idx_rows.shape[1]
    hpg = Hq // G
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    loss = np.zeros((R, G))
    dq = np.zeros(q_idx_rows.shape)
    for r, i in enumerate(int(x) for x in rows):
        b_loc = i // block_size
        S = block_scores(q_idx_rows[r], k_idx[:b_loc * block_size], block_size)
        for g in range(G):
            T = token_set(select_blocks(S[g], b_loc, topk), i, block_size)
            l, gs = row_terms(q_rows[r, g * hpg:(g + 1) * hpg], k[T, g], q_idx_rows[r, g], k_idx[T], scale)
            loss[r, g] = l
            dq[r, g] = gs @ k_idx[T]
    return {"loss": loss, "dq_idx": dq}
