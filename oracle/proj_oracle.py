"""Plain float64 CPU oracle of the Index Branch's two projections: the index
query heads (one per GQA group) and the one shared index key head are linear
maps of the layer's hidden states.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
this module: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg use it. It shares no code with the HIP path.

Sources:
  [yhxrc] yhxrc.cn comparison of MSA/NSA/DSA/MoBA, section 二: the index branch
          has one scoring (query) head per attention group plus one key head
          shared by the whole model layer.
  [yifor] yifor-blog, section "工程實踐啟示" (engineering takeaways): the
          index branch adds only two projection matrices.

Readings (the pages give the head counts and the two matrices, nothing more):
  - Each projection is a plain linear map with no bias, activation,
    normalisation or position encoding: q_idx[t, g] = W_qi[g] x[t] and
    k_idx[t] = W_ki x[t].
  - Weights use the (out_features, in_features) layout of a linear layer:
    W_qi [G, d_idx, d_model], W_ki [d_idx, d_model].
  - The projections' outputs feed the index scores in bf16, so the product
    path rounds them to bf16 (nearest even); `round_bf16` applies the same
    rounding to the exact result when a test compares bit for bit.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np
import torch


def index_project(x: np.ndarray, w_qi: np.ndarray, w_ki: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """x [n, d_model], w_qi [G, d_idx, d_model], w_ki [d_idx, d_model] (float64)
    -> q_idx [n, G, d_idx], k_idx [n, d_idx] in float64 [yhxrc, 二; yifor, 工程實踐啟示]."""
    x = np.asarray(x, dtype=np.float64)
    w_qi = np.asarray(w_qi, dtype=np.float64)
    w_ki = np.asarray(w_ki, dtype=np.float64)
    n, dm = x.shape
    G, di, dm2 = w_qi.shape
    assert dm2 == dm and w_ki.shape == (di, dm)
    q_idx = np.empty((n, G, di))
    for g in range(G):
        q_idx[:, g, :] = x @ w_qi[g].T
    k_idx = x @ w_ki.T
    return q_idx, k_idx


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even) -> float64, by torch's CPU
    conversion. Exact for values that are exact in fp32 (the bit-exact tests
    keep every sum an integer below 2^24, so no double rounding occurs)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def fp32_error_bound(x: np.ndarray, w_qi: np.ndarray, w_ki: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-output bound on the fp32 accumulation error of a d_model-term dot
    product, (d_model * 2^-24) * sum_k |x_k w_k| (first order of the standard
    bound for recursive summation, for any order of the additions)."""
    ax, aq, ak = np.abs(x), np.abs(w_qi), np.abs(w_ki)
    dm = x.shape[1]
    sq, sk = index_project(ax, aq, ak)
    c = dm * 2.0 ** -24
    return c * sq, c * sk
