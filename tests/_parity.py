"""Shared helpers of the GPU parity tests: build seeded inputs on the device,
run the oracle on the host for the same rows, compare."""
from __future__ import annotations

import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import msa_synth as syn
from oracle import msa_oracle as mo

OUT_MAX_ABS = 2e-2      # bf16 in/out, fp32 accumulation
OUT_REL_L2 = 5e-3
# lse: the attention weights P enter both P.V and the denominator rounded to
# bf16 (unit roundoff u = 2^-8), so the denominator can be off by a relative u
# when one key dominates a row: |d lse| <= ln(1 + 2^-8) = 3.9e-3, plus fp32
# accumulation (~1e-6).
LSE_MAX_ABS = 4e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def prefill_device_inputs(inp: syn.PrefillInputs, device="cuda"):
    q = inp.q(device=device)[None].contiguous()
    k = inp.k(device=device)[None].contiguous()
    v = inp.v(device=device)[None].contiguous()
    qi = inp.q_idx(device=device)[None].contiguous()
    ki = inp.k_idx(device=device)[None].contiguous()
    return q, k, v, qi, ki


def oracle_prefill(inp: syn.PrefillInputs, rows, topk, want_scores=False, kv_host=None, threads=16, scale=None):
    """Oracle on the given rows; inputs regenerated on the CPU from the seed
    (kv_host: optional pre-generated (k_idx, k, v) float64 arrays)."""
    rows = np.asarray(rows, dtype=np.int64)
    if kv_host is None:
        kv_host = (mo.to_f64(inp.k_idx()), mo.to_f64(inp.k()), mo.to_f64(inp.v()))
    ki, k, v = kv_host
    q = mo.to_f64(inp.q(rows))
    qi = mo.to_f64(inp.q_idx(rows))
    bk = inp.dims.block_size
    parts = np.array_split(np.arange(len(rows)), max(1, min(4 * threads, len(rows) // 16)))

    done = [0]
    t0 = time.time()

    def run(ix):
        r = mo.prefill_rows(rows[ix], q[ix], qi[ix], ki, k, v, block_size=bk, topk=topk,
                            want_scores=want_scores, scale=scale)
        done[0] += len(ix)
        if len(rows) >= 1024:
            log(f"    oracle rows {done[0]}/{len(rows)} ({time.time() - t0:.0f}s)")
        return r

    try:  # one BLAS thread per worker: the workers already use every core
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limit = None
    try:
        with ThreadPoolExecutor(min(threads, len(parts))) as ex:
            res = list(ex.map(run, parts))
    finally:
        if limit is not None:
            limit.unregister()
    out = {key: np.concatenate([r[key] for r in res]) for key in ("sel", "out", "lse")}
    if want_scores:
        out["scores"] = [s for r in res for s in r["scores"]]
    return out


def compare_out(got: torch.Tensor, want: np.ndarray, what: str):
    g = got.detach().to("cpu", torch.float64).numpy()
    diff = g - want
    max_abs = float(np.abs(diff).max())
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-30))
    log(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= OUT_MAX_ABS, f"{what}: max abs {max_abs}"
    assert rel <= OUT_REL_L2, f"{what}: rel L2 {rel}"
    return max_abs, rel


def compare_lse(got: torch.Tensor, want: np.ndarray, what: str):
    g = got.detach().to("cpu", torch.float64).numpy()
    err = float(np.abs(g - want).max())
    log(f"  {what}: lse max_abs={err:.3e}")
    assert err <= LSE_MAX_ABS, f"{what}: lse err {err}"


def timed(label):
    class _T:
        def __enter__(self):
            self.t = time.time()
            return self

        def __exit__(self, *a):
            log(f"  [{label}] {time.time() - self.t:.1f}s")
    return _T()
