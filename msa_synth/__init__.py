"""Seeded synthetic inputs for the MSA prefill and decode hot path.

This module only *makes arrays*: it holds none of the method's arithmetic (no
scoring, pooling, selection or attention). Both the GPU path (tests, bench) and
the float64 oracle draw their inputs from here, and nothing else is shared
between them.

Every value is a pure function of (seed, stream, flat element index), built
from integer hashing plus exactly representable float steps, so one row can be
regenerated alone on the CPU and equals the same row generated on the GPU bit
for bit:

* hash: the MurmurHash3 32-bit finaliser ("fmix32", Austin Appleby's public
  MurmurHash3) applied to (key ^ low word), then (that ^ high word ^ key2).
  All products are taken modulo 2**32 with 16-bit limbs in int64, so no
  intermediate overflows on any device.
* "~N(0,1)" values: the classical Irwin-Hall approximation, the sum of twelve
  uniform variates minus six. Here the twelve variates are the 16-bit halves of
  six 32-bit words (the element's hash h0 and fmix32(h0 ^ c_t), t = 1..5); z = (2*S - 12*65535) * 2**-17 is exact in float32 (|2S-...| <
  2**20), has mean 0 and variance (2**32-1)/2**32, and is rounded once to
  bfloat16 (round-to-nearest-even, the same rule on CPU and GPU).
* integer-valued index projections: hash mod (hi-lo+1) + lo.

Workload recipes (block size B_k = 128 unless stated):

* ``tiny``: one GQA group, q_idx/k_idx i.i.d. integers in [-3, 3].
* ``planted``: background q_idx/k_idx in {-1,0,1}; group g's index-query slice
  (dims [g*s, (g+1)*s), s = d_idx/G) is 3; for each group, ``n_planted``
  distinct far blocks in [0, nb/4) each hold one needle key row that is 3 on the
  group's slice and 0 elsewhere. A needle scores 3*3*s = 144 (s = 16) against
  any background block's <= 3*s + (d_idx - s) = 96, so every planted block older
  than the query's own block is among its top blocks.
* ``skewed``: the planted recipe with ``n_planted`` per group plus ``n_hot``
  blocks shared by every group (block 0, a sink-like block, and n_hot-1 seeded
  blocks in [1, nb/8)); a hot needle row is 3 in every dim, and non-slice
  q_idx dims are drawn from {0, 1} so a hot needle scores >= 144 for every
  group. Hot blocks are then selected by nearly every later query.
* decode: per sequence s the planted recipe with seed ``seed*1000 + s`` over
  the cache rows; the new token's q_idx follows the same query recipe.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

MASK32 = 0xFFFFFFFF

# stream ids: one per generated tensor
S_Q, S_K, S_V, S_QIDX, S_KIDX = 1, 2, 3, 4, 5


def _fmix32_int(h: int) -> int:
    h &= MASK32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & MASK32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & MASK32
    h ^= h >> 16
    return h


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2**32 for int64 x in [0, 2**32), exact (no int64 overflow)."""
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + ((hi * (c & 0xFFFF)) << 16)) & MASK32


def _fmix32(h: torch.Tensor) -> torch.Tensor:
    h = h ^ (h >> 16)
    h = _mul32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = _mul32(h, 0xC2B2AE35)
    h = h ^ (h >> 16)
    return h


def _keys(seed: int, stream: int):
    k1 = _fmix32_int(seed * 0x9E3779B1 + stream * 0x85EBCA77 + 0x165667B1)
    k2 = _fmix32_int(k1 ^ 0x27D4EB2F ^ (seed >> 32))
    return k1, k2


def hash32(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """Counter-based 32-bit hash of int64 counters idx (0 <= idx < 2**62)."""
    k1, k2 = _keys(seed, stream)
    lo = idx & MASK32
    hi = idx >> 32
    h = _fmix32(lo ^ k1)
    h = _fmix32(h ^ hi ^ k2)
    return h


def normal_bf16(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """Irwin-Hall(12) approximately standard normal values, as bfloat16."""
    h0 = hash32(seed, stream, idx)
    s = (h0 & 0xFFFF) + (h0 >> 16)
    for t in range(1, 6):
        h = _fmix32(h0 ^ _fmix32_int(0x5BD1E995 + t))
        s = s + (h & 0xFFFF) + (h >> 16)
    z = (2 * s - 12 * 65535).to(torch.float32) * (2.0 ** -17)
    return z.to(torch.bfloat16)


def uniform_int(seed: int, stream: int, idx: torch.Tensor, lo: int, hi: int) -> torch.Tensor:
    """Integers uniform (up to a 2**-32 relative bias) in [lo, hi], as int64."""
    h = hash32(seed, stream, idx)
    return h % (hi - lo + 1) + lo


_CHUNK = 1 << 24


def _gen_rows(fn, rows: torch.Tensor, row_elems: int, device) -> torch.Tensor:
    """Evaluate fn(flat_idx) for every element of the given rows, chunked."""
    rows = rows.to(device=device, dtype=torch.int64)
    out = []
    rows_per_chunk = max(1, _CHUNK // max(1, row_elems))
    col = torch.arange(row_elems, device=device, dtype=torch.int64)
    for s in range(0, rows.numel(), rows_per_chunk):
        r = rows[s:s + rows_per_chunk]
        idx = (r[:, None] * row_elems + col[None, :]).reshape(-1)
        out.append(fn(idx).reshape(r.numel(), row_elems))
    if not out:
        return fn(torch.zeros(0, dtype=torch.int64, device=device)).reshape(0, row_elems)
    return torch.cat(out, 0)


def _as_rows(rows, n: int, device) -> torch.Tensor:
    if rows is None:
        return torch.arange(n, dtype=torch.int64, device=device)
    if isinstance(rows, slice):
        return torch.arange(n, dtype=torch.int64, device=device)[rows]
    return torch.as_tensor(np.asarray(rows, dtype=np.int64), device=device)


@dataclasses.dataclass
class Dims:
    num_q_heads: int = 64
    num_kv_heads: int = 4
    head_dim: int = 128
    index_dim: int = 64
    block_size: int = 128
    topk: int = 16

    @property
    def hpg(self) -> int:
        return self.num_q_heads // self.num_kv_heads


class PrefillInputs:
    """One sequence of N tokens; rows are token positions."""

    def __init__(self, n: int, dims: Dims, seed: int, recipe: str = "planted",
                 n_planted: int = 8, n_hot: int = 0):
        assert recipe in ("tiny", "planted", "skewed")
        self.n, self.dims, self.seed, self.recipe = n, dims, seed, recipe
        self.n_planted, self.n_hot = n_planted, n_hot
        G, di, bk = dims.num_kv_heads, dims.index_dim, dims.block_size
        nb = (n + bk - 1) // bk
        self.nb = nb
        self.slice = di // G
        # needle rows: dict row -> ("group", g) or ("hot", -1)
        self.needles: dict = {}
        self.planted: dict = {g: [] for g in range(G)}
        self.hot: list = []
        if recipe == "tiny":
            return
        rng = np.random.default_rng(np.random.PCG64(seed))
        used_blocks = set()
        if recipe == "skewed" and n_hot > 0:
            hot = [0]
            hi = max(2, nb // 8)
            while len(hot) < n_hot:
                b = int(rng.integers(1, hi))
                if b not in hot:
                    hot.append(b)
            self.hot = sorted(hot)
            for b in self.hot:
                r = b * bk + int(rng.integers(0, bk))
                self.needles[r] = ("hot", -1)
                used_blocks.add(b)
        lim = max(1, nb // 4)
        for g in range(G):
            blocks = []
            tries = 0
            while len(blocks) < min(n_planted, lim) and tries < 10000:
                tries += 1
                b = int(rng.integers(0, lim))
                if b in blocks or b in used_blocks:
                    continue
                r = b * bk + int(rng.integers(0, bk))
                if r >= n or r in self.needles:
                    continue
                blocks.append(b)
                self.needles[r] = ("group", g)
            self.planted[g] = sorted(blocks)

    # -- main-branch tensors ------------------------------------------------
    def q(self, rows=None, device="cpu") -> torch.Tensor:
        d = self.dims
        r = _as_rows(rows, self.n, device)
        e = d.num_q_heads * d.head_dim
        t = _gen_rows(lambda i: normal_bf16(self.seed, S_Q, i), r, e, device)
        return t.reshape(-1, d.num_q_heads, d.head_dim)

    def k(self, rows=None, device="cpu") -> torch.Tensor:
        d = self.dims
        r = _as_rows(rows, self.n, device)
        e = d.num_kv_heads * d.head_dim
        t = _gen_rows(lambda i: normal_bf16(self.seed, S_K, i), r, e, device)
        return t.reshape(-1, d.num_kv_heads, d.head_dim)

    def v(self, rows=None, device="cpu") -> torch.Tensor:
        d = self.dims
        r = _as_rows(rows, self.n, device)
        e = d.num_kv_heads * d.head_dim
        t = _gen_rows(lambda i: normal_bf16(self.seed, S_V, i), r, e, device)
        return t.reshape(-1, d.num_kv_heads, d.head_dim)

    # -- index-branch tensors -----------------------------------------------
    def q_idx(self, rows=None, device="cpu") -> torch.Tensor:
        d = self.dims
        G, di, s = d.num_kv_heads, d.index_dim, self.slice
        r = _as_rows(rows, self.n, device)
        e = G * di
        if self.recipe == "tiny":
            t = _gen_rows(lambda i: uniform_int(self.seed, S_QIDX, i, -3, 3), r, e, device)
            return t.to(torch.bfloat16).reshape(-1, G, di)
        lo = 0 if self.recipe == "skewed" else -1
        t = _gen_rows(lambda i: uniform_int(self.seed, S_QIDX, i, lo, 1), r, e, device)
        t = t.reshape(-1, G, di)
        for g in range(G):
            t[:, g, g * s:(g + 1) * s] = 3
        return t.to(torch.bfloat16)

    def k_idx(self, rows=None, device="cpu") -> torch.Tensor:
        d = self.dims
        di, s = d.index_dim, self.slice
        r = _as_rows(rows, self.n, device)
        if self.recipe == "tiny":
            t = _gen_rows(lambda i: uniform_int(self.seed, S_KIDX, i, -3, 3), r, di, device)
            return t.to(torch.bfloat16)
        t = _gen_rows(lambda i: uniform_int(self.seed, S_KIDX, i, -1, 1), r, di, device)
        if self.needles:
            rl = r.cpu().numpy()
            needle_rows = np.array(sorted(self.needles), dtype=np.int64)
            for p in np.nonzero(np.isin(rl, needle_rows))[0].tolist():
                kind, g = self.needles[int(rl[p])]
                if kind == "hot":
                    t[p, :] = 3
                else:
                    t[p, :] = 0
                    t[p, g * s:(g + 1) * s] = 3
        return t.to(torch.bfloat16)


class DecodeInputs:
    """B sequences with a KV cache of max_ctx rows each and ctx_lens[b] valid rows
    (the last valid row is the new token)."""

    def __init__(self, batch: int, max_ctx: int, dims: Dims, seed: int,
                 ctx_lens: Optional[Sequence[int]] = None, n_planted: int = 8):
        self.batch, self.max_ctx, self.dims, self.seed = batch, max_ctx, dims, seed
        self.ctx_lens = list(ctx_lens) if ctx_lens is not None else [max_ctx] * batch
        assert len(self.ctx_lens) == batch and all(1 <= c <= max_ctx for c in self.ctx_lens)
        # per-sequence index recipe: the planted prefill recipe over the cache rows
        self.seqs = [PrefillInputs(max_ctx, dims, seed * 1000 + b, "planted", n_planted=n_planted)
                     for b in range(batch)]

    def q(self, b: int, device="cpu") -> torch.Tensor:
        L = self.ctx_lens[b]
        return self.seqs[b].q([L - 1], device)[0]

    def q_idx(self, b: int, device="cpu") -> torch.Tensor:
        L = self.ctx_lens[b]
        return self.seqs[b].q_idx([L - 1], device)[0]

    def k_cache(self, b: int, rows=None, device="cpu") -> torch.Tensor:
        return self.seqs[b].k(rows, device)

    def v_cache(self, b: int, rows=None, device="cpu") -> torch.Tensor:
        return self.seqs[b].v(rows, device)

    def k_idx_cache(self, b: int, rows=None, device="cpu") -> torch.Tensor:
        return self.seqs[b].k_idx(rows, device)


def stratified_rows(n: int, count: int, block_size: int, seed: int, k: int,
                    extra: Sequence[int] = ()) -> np.ndarray:
    """Sorted unique query rows for sampled parity: rows before (k-1)*B_k, rows at
    block starts and ends, the last row, rows in/after the given blocks, rest
    uniform."""
    rng = np.random.default_rng(np.random.PCG64(seed + 7919))
    picks = set()
    early = min(n, (k - 1) * block_size)
    if early > 0:
        picks.update(rng.integers(0, early, size=min(early, count // 8)).tolist())
    nb = (n + block_size - 1) // block_size
    starts = rng.integers(0, nb, size=count // 8) * block_size
    picks.update(int(x) for x in starts if x < n)
    ends = rng.integers(0, nb, size=count // 8) * block_size + block_size - 1
    picks.update(int(x) for x in ends if x < n)
    picks.add(n - 1)
    for b in extra:
        for off in (0, 1, block_size - 1, block_size, block_size + 1):
            r = b * block_size + off
            if 0 <= r < n:
                picks.add(r)
    while len(picks) < min(count, n):
        picks.update(rng.integers(0, n, size=count - len(picks)).tolist())
    out = np.array(sorted(picks), dtype=np.int64)
    return out[:max(count, len(out))]
