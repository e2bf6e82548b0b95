"""Textbook dense attention references used to pin the MSA oracle.

TEST INFRASTRUCTURE ONLY (same rule as msa_oracle: only tests/, smoke() and
bench.py's cpu_baseline leg may use it). Written independently of msa_oracle:
it forms the full N x N score matrix per head and applies an explicit boolean
mask, the plain definition of (masked) causal grouped-query attention.

Head h reads KV head h // (Hq // G) (contiguous grouping of query heads onto KV
heads, the GQA layout of [pnsm §2]: 64 query heads sharing 4 KV heads).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def masked_gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                         mask: Optional[np.ndarray] = None,
                         scale: Optional[float] = None):
    """q [N, Hq, d], k/v [N, G, d]; mask [G, N, N] bool (True = attend) or None
    for plain causal. Returns out [N, Hq, d], lse [N, Hq] (float64)."""
    N, Hq, d = q.shape
    G = k.shape[1]
    hpg = Hq // G
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    causal = np.tril(np.ones((N, N), dtype=bool))
    out = np.zeros((N, Hq, d))
    lse = np.zeros((N, Hq))
    for h in range(Hq):
        g = h // hpg
        allowed = causal if mask is None else (causal & mask[g])
        scores = scale * (q[:, h, :] @ k[:, g, :].T)
        scores = np.where(allowed, scores, -np.inf)
        row_max = scores.max(axis=1, keepdims=True)
        w = np.exp(scores - row_max)
        w = np.where(allowed, w, 0.0)
        tot = w.sum(axis=1, keepdims=True)
        out[:, h, :] = (w / tot) @ v[:, g, :]
        lse[:, h] = (row_max + np.log(tot))[:, 0]
    return out, lse


def block_mask_from_selection(sel: np.ndarray, n: int, block_size: int) -> np.ndarray:
    """sel [N, G, k] block ids (-1 pad) -> mask [G, N, N]: mask[g, i, j] is True
    when the block of key j is among query i's selected blocks for group g."""
    N, G, _ = sel.shape
    assert N == n
    key_block = np.arange(n) // block_size
    m = np.zeros((G, n, n), dtype=bool)
    for g in range(G):
        for i in range(n):
            chosen = sel[i, g][sel[i, g] >= 0]
            m[g, i] = np.isin(key_block, chosen)
    return m
