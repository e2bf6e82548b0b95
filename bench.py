"""Benchmark of the MSA hot path on one MI355X.

One step = one MSA prefill of a 32768-token sequence (64 query heads, 4 KV
heads, head_dim 128, index dim 64, B_k 128, k 16, planted-needle index keys)
followed by one decode step of 64 sequences with 131072-token caches (same
heads; planted index keys per sequence). Inputs are generated on the device
before timing and stay resident in HBM.

Prints one JSON line. `value` is the prefill sparse-attention throughput
F_main / t_prefill, where F_main = 4 * d * hpg * sum over (query, group) of the
attended token count and t_prefill is the whole prefill call (index branch
included). Decode KV GB/s (algorithmic bytes / whole decode call) is reported
alongside, with per-stage times from the profiled entry points and the
roofline of the dominant kernel. The timed calls' own outputs (no selection
or lse output, reused workspace) are checked against the float64 oracle on
sampled prefill rows and 8 decode sequences (`parity`; the run exits with
status 3 on a miss); the same oracle rows, timed on the host cores, are the
`cpu_baseline`. Side measurements (not part of a step): cold-cache timings
(after a 512 MiB write), measured ceilings (bf16 matmul, device copy), the
top-k kernel beside torch.topk, chunked and variable-length prefill, the
Index Branch KL-alignment backward, prefill / decode at B_k 64 and 32, the
Index Branch projections from hidden states, and the long configurations
(`configs`: 128K prefill with hot blocks, 1M prefill, 8 x 1M decode).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MSA prefill sparse-attn TFLOP/s (% MFMA peak) + decode KV GB/s @128K ctx"
MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E

# Bench workload
N_PREFILL, HQ, G, D, DI, BK, TOPK = 32768, 64, 4, 128, 64, 128, 16
DEC_B, DEC_L = 64, 131072


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- algorithmic work ------------------------------------------------------

def attended_tokens(i: int, topk: int, bk: int = BK) -> int:
    """|T| for query row i: every selected block older than the own block is
    full, the own block contributes i % bk + 1 keys, and |Sel| = min(k, b_loc+1)."""
    b_loc = i // bk
    return bk * (min(topk, b_loc + 1) - 1) + (i % bk + 1)


def prefill_flops(rows, n_groups=G, hpg=HQ // G, d=D, topk=TOPK):
    t = sum(attended_tokens(int(i), topk) for i in rows)
    return 4.0 * d * hpg * n_groups * t


def prefill_flops_full(n, **kw):
    # closed form summed per block for speed
    topk = kw.get("topk", TOPK)
    bk = kw.get("bk", BK)
    tot = 0
    for blk in range((n + bk - 1) // bk):
        lo, hi = blk * bk, min(n, (blk + 1) * bk)
        cnt = hi - lo
        tot += cnt * bk * (min(topk, blk + 1) - 1) + sum(range(1, cnt + 1))
    return 4.0 * kw.get("d", D) * kw.get("hpg", HQ // G) * kw.get("n_groups", G) * tot


def index_flops_full(n, topk=TOPK):
    tot = 0
    for i_blk in range((n + BK - 1) // BK):
        cnt = min(n, (i_blk + 1) * BK) - i_blk * BK
        if i_blk >= topk:
            tot += cnt * BK * i_blk
    return 2.0 * DI * G * tot


def decode_bytes(ctx_lens, topk=TOPK, bk=BK):
    tot = 0
    for L in ctx_lens:
        i = L - 1
        b_loc = i // bk
        scored = bk * b_loc if b_loc >= topk else 0
        tot += scored * DI * 2                                # k_idx keys scored
        tot += G * attended_tokens(i, topk, bk) * 2 * D * 2   # K and V of the attended tokens
        tot += HQ * D * 2 * 2 + G * DI * 2                    # q, out, q_idx
    return float(tot)


# A 16-row unit's block is computed by the dense pass when at least this many
# of the unit's rows selected it (all of them, if the unit has fewer); the
# library's split rule (kDenseMin in its launch header).
DENSE_MIN = 5


def pair_stats(torch, sel, n, bk=BK, d=D, hpg=HQ // G, window=65536):
    """Split the selected (query, group, block) pairs of a prefill into the
    two attention passes, as the library does: a pair is "dense" when at least
    min(DENSE_MIN, rows of the unit) rows of its 16-row unit selected the block,
    else it is computed KV-outer. Returns per-pass pair counts, algorithmic
    flops (4*d*hpg per attended key), the number of distinct (group, block) K/V
    blocks each pass touches, and the dense pass's (unit, block) count (it
    computes all 16 rows of a unit against each, masking those that did not
    select it). sel: [G, n, k] int32 on the device (-1 = no selection). Rows
    are taken `window` at a time (a multiple of 16) to bound the memory."""
    ng, _, k = sel.shape
    dev = sel.device
    nb = (n + bk - 1) // bk
    st = {"dense_pairs": 0, "sparse_pairs": 0, "F_dense": 0.0, "F_sparse": 0.0, "kv_dense": 0, "kv_sparse": 0,
          "dense_unit_blocks": 0}
    for g in range(ng):
        used_d = torch.zeros(nb, dtype=torch.bool, device=dev)
        used_s = torch.zeros(nb, dtype=torch.bool, device=dev)
        for r0 in range(0, n, window):
            r1 = min(n, r0 + window)
            w = r1 - r0
            nunits = (w + 15) // 16
            rows = torch.arange(r0, r1, device=dev)
            unit_rows = torch.clamp(w - torch.arange(nunits, device=dev) * 16, max=16)
            s = sel[g, r0:r1].long()
            valid = s >= 0
            rr = rows[:, None].expand(w, k)[valid]
            bb = s[valid]
            key = ((rr - r0) // 16) * nb + bb
            cnt = torch.bincount(key, minlength=nunits * nb).view(nunits, nb)
            dense_ub = cnt >= torch.clamp(unit_rows, max=DENSE_MIN)[:, None]
            dense = dense_ub.view(-1)[key]
            st["dense_unit_blocks"] += int((dense_ub & (cnt > 0)).sum())
            keys = torch.where(bb == rr // bk, rr % bk + 1, torch.full_like(rr, bk)).double()
            fl = 4.0 * d * hpg * keys
            st["F_dense"] += float(fl[dense].sum())
            st["F_sparse"] += float(fl[~dense].sum())
            st["dense_pairs"] += int(dense.sum())
            st["sparse_pairs"] += int((~dense).sum())
            used_d[bb[dense]] = True
            used_s[bb[~dense]] = True
            del s, valid, rr, bb, key, cnt, dense_ub, dense, keys, fl
        st["kv_dense"] += int(used_d.sum())
        st["kv_sparse"] += int(used_s.sum())
    return st


# HBM traffic per launch of the attention kernels on this workload, from
# rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by a 1 GiB calibration kernel
# (profiles/bench_step_hbm_bytes.txt). Valid only for the kernel sources they
# were taken on: keyed by the hash that source_hash() computes.
MEASURED_TRAFFIC = {
    "source": "84c9f377dc1e50b0",
    "k_attn_prefill (KV-outer)": 4.175e9,
    "k_attn_dense (dense + merge)": 3.520e9,
}


def source_hash():
    """sha256 of the attention kernels' sources with comments and blank lines
    removed (a change of comments alone leaves the kernels, and so their
    measured traffic, as they were)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("attn.hip", "msa_device.h", "msa_launch.h"):
        with open(os.path.join(ROOT, "block_sparse_long_07_amd", "csrc", f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update("\n".join(l.rstrip() for l in src.split("\n") if l.strip()).encode())
    return h.hexdigest()[:16]


def kernel_roofline(name, ms, flops, nbytes, measured=True):
    """Roofline position of one kernel: the bound is whichever of the MFMA
    time (flops at the bf16 peak) and the HBM time (algorithmic bytes at the
    HBM peak) is larger; achieved and frac are in that bound's unit.
    measured=False: no counter figures exist for this launch configuration."""
    t = ms * 1e-3
    mfma_bound = flops / (MFMA_PEAK_TFLOPS * 1e12) >= nbytes / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        ach, peak, unit = flops / t / 1e12, MFMA_PEAK_TFLOPS, "TFLOP/s"
    else:
        ach, peak, unit = nbytes / t / 1e9, HBM_PEAK_GBS, "GB/s"
    traffic = MEASURED_TRAFFIC.get(name) if measured and MEASURED_TRAFFIC["source"] == source_hash() else None
    return {"kernel": name, "bound": "mfma" if mfma_bound else "hbm", "achieved": round(ach, 2), "peak": peak,
            "unit": unit, "frac": round(ach / peak, 4), "traffic": traffic, "ms": round(ms, 4),
            "algorithmic_tflop": round(flops / 1e12, 4), "algorithmic_gb": round(nbytes / 1e9, 4),
            "tflops": round(flops / t / 1e12, 2), "GB/s": round(nbytes / t / 1e9, 1)}


def attention_rooflines(torch, sel, n, stage, bk=BK, topk=TOPK, measured=True):
    """Both attention kernels' roofline positions from the actual selection
    sel [G, n, k]: algorithmic flops per attended key, algorithmic bytes = each
    pass's K/V blocks once, the (query, group) inputs and outputs, and the
    KV-outer partials written once and read once. "executed_tflop" counts the
    MFMA work as issued: every key of each selected block (the causal tail of
    the own block included) and, in the dense pass, all 16 rows of a unit
    against each of its listed blocks."""
    ps = pair_stats(torch, sel, n, bk=bk)
    q_bytes = HQ // G * D * 2                     # one (query, group): 16 heads x 128 dims, bf16
    part_bytes = q_bytes + HQ // G * 4            # normalised bf16 partial + fp32 lse per head
    kv_block = 2 * bk * D * 2                     # K and V of one block of one group
    b_kv = ps["sparse_pairs"] * (q_bytes + part_bytes) + ps["kv_sparse"] * kv_block
    b_dm = (n * G * (2 * q_bytes + topk * 4) + ps["kv_dense"] * kv_block + ps["sparse_pairs"] * part_bytes)
    kernels = [kernel_roofline("k_attn_prefill (KV-outer)", stage["kv_outer_attn"], ps["F_sparse"], b_kv, measured),
               kernel_roofline("k_attn_dense (dense + merge)", stage["dense_attn_merge"], ps["F_dense"], b_dm,
                               measured)]
    kernels[0]["executed_tflop"] = round(ps["sparse_pairs"] * 4.0 * D * (HQ // G) * bk / 1e12, 4)
    # the dense pass's MFMA work including the masked rows of its unit blocks
    kernels[1]["executed_tflop"] = round(ps["dense_unit_blocks"] * 16 * 4.0 * D * (HQ // G) * bk / 1e12, 4)
    return ps, kernels


def block_size_variants(torch, msa, pre, dec_in, ctx_lens, topk, reps, sizes=(64, 32)):
    """The bench prefill and decode at the smaller block sizes the pages
    ablate (same inputs, same k: a budget of k * B_k keys per query). Prefill
    TFLOP/s counts the attended keys (F_main at that B_k); decode GB/s its
    algorithmic bytes at that B_k."""
    n = pre[0].shape[1]
    res = {}
    for bk in sizes:
        p = msa.params(HQ, G, D, DI, bk, topk)
        ws = torch.empty(msa.prefill_workspace_bytes(p, 1, n), dtype=torch.uint8, device=pre[0].device)
        out = torch.empty_like(pre[0])
        ms = _time_calls(torch, lambda: msa.prefill(*pre, topk=topk, block_size=bk, workspace=ws, out=out), reps)
        st = stage_times(msa, lambda **kw: msa.prefill(*pre, topk=topk, block_size=bk, workspace=ws, out=out, **kw),
                         reps)
        stage = dict(zip(msa.PREFILL_STAGES, (float(v) for v in st)))
        _, sel, _ = msa.prefill(*pre, topk=topk, block_size=bk, workspace=ws, out=out, want_sel=True)
        ps, kernels = attention_rooflines(torch, sel[0], n, stage, bk=bk, topk=topk, measured=False)
        del sel, ws, out
        f = prefill_flops_full(n, topk=topk, bk=bk)
        assert abs(ps["F_dense"] + ps["F_sparse"] - f) <= 1e-9 * f, "pair split does not cover F_main"
        wsd = torch.empty(msa.decode_workspace_bytes(p, dec_in[0].shape[0], dec_in[2].shape[1]), dtype=torch.uint8,
                          device=pre[0].device)
        outd = torch.empty_like(dec_in[0])
        dms = _time_calls(torch, lambda: msa.decode(*dec_in, topk=topk, block_size=bk, workspace=wsd, out=outd),
                          reps)
        db = decode_bytes(ctx_lens, topk, bk)
        del wsd, outd
        res[str(bk)] = {"prefill": {"ms": round(ms, 4), "F_main_tflop": round(f / 1e12, 4),
                                    "tflops": round(f / (ms * 1e-3) / 1e12, 2),
                                    "stage_ms": {k: round(v, 4) for k, v in stage.items()}, "kernels": kernels},
                        "decode": {"ms": round(dms, 4), "bytes_gb": round(db / 1e9, 4),
                                   "GB/s": round(db / (dms * 1e-3) / 1e9, 1)}}
    return res


# The hidden size the index projections read: the pages give the head layout
# (64 query heads of 128) but not the model width; this reading takes
# d_model = 64 * 128.
D_MODEL = 8192


def projection_measure(torch, msa, n, batch, reps, d_model=D_MODEL):
    """Index Branch projections (G index query heads + the shared key head,
    one GEMM) for the n-token prefill and for one decode step of `batch`
    sequences (key appended to each cache). Algorithmic work: 2 n d_model
    64 (G+1) flops; bytes: x once, the weights once, the bf16 outputs once."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(5)
    cols = 64 * (G + 1)
    x = torch.randn((n, d_model), generator=g, device=dev).to(torch.bfloat16)
    wq = (torch.randn((G, DI, d_model), generator=g, device=dev) * d_model ** -0.5).to(torch.bfloat16)
    wk = (torch.randn((DI, d_model), generator=g, device=dev) * d_model ** -0.5).to(torch.bfloat16)
    qi = torch.empty((n, G, DI), dtype=torch.bfloat16, device=dev)
    ki = torch.empty((n, DI), dtype=torch.bfloat16, device=dev)
    p = msa.params(HQ, G, D, DI)
    ws = torch.empty(max(msa.index_project_workspace_bytes(p, n, d_model),
                         msa.index_project_workspace_bytes(p, batch, d_model)), dtype=torch.uint8, device=dev)
    res = {"d_model": d_model}
    ms = _time_calls(torch, lambda: msa.index_project(x, wq, wk, q_idx=qi, k_idx=ki, workspace=ws), reps)
    fl = 2.0 * n * d_model * cols
    nb = (n * d_model + cols * d_model + n * cols) * 2
    t_mfma, t_hbm = fl / (MFMA_PEAK_TFLOPS * 1e12), nb / (HBM_PEAK_GBS * 1e9)
    res["prefill"] = {"tokens": n, "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                      "GB/s": round(nb / (ms * 1e-3) / 1e9, 1), "bound": "mfma" if t_mfma >= t_hbm else "hbm",
                      "frac": round(max(t_mfma, t_hbm) / (ms * 1e-3), 4)}
    # measured ceiling for this shape: the vendor GEMM (torch.matmul, hipBLASLt)
    # of the same x against the stacked weights into a plain [n, cols] output
    # (no cache-row scatter), as a reference point for the analytic bound
    wst = torch.cat([wq.reshape(G * DI, d_model), wk]).t()
    ref = torch.empty((n, cols), dtype=torch.bfloat16, device=dev)
    ms_v = _time_calls(torch, lambda: torch.matmul(x, wst, out=ref), reps)
    res["prefill"]["vendor_gemm"] = {"ms": round(ms_v, 4), "tflops": round(fl / (ms_v * 1e-3) / 1e12, 2),
                                     "frac": round(max(t_mfma, t_hbm) / (ms_v * 1e-3), 4),
                                     "what": "torch.matmul (hipBLASLt) of the same shape, plain output"}
    cache = torch.zeros((batch, 4096, DI), dtype=torch.bfloat16, device=dev)
    lens = torch.full((batch,), 4096, dtype=torch.int32, device=dev)
    xd = x[:batch].contiguous()
    qd = torch.empty((batch, G, DI), dtype=torch.bfloat16, device=dev)
    ms = _time_calls(torch, lambda: msa.index_project_decode(xd, wq, wk, cache, lens, q_idx=qd, workspace=ws), reps)
    fl = 2.0 * batch * d_model * cols
    nb = (batch * d_model + cols * d_model + batch * cols) * 2
    res["decode"] = {"batch": batch, "ms": round(ms, 4), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1), "bound": "hbm",
                     "frac": round(nb / (HBM_PEAK_GBS * 1e9) / (ms * 1e-3), 4)}
    return res


# ---- rocprofv3 summaries -------------------------------------------------------

def summarize_rocprof(d):
    """Text summary of rocprofv3 CSV output (kernel stats and per-dispatch
    counters) for the msa kernels and the calibration kernel."""
    import csv
    import glob
    from collections import defaultdict

    def keep(name):
        return "msa::" in name or "neg_kernel" in name

    lines = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        lines.append(f"## kernel stats ({os.path.basename(f)})")
        lines.append(f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_ms':>10s}")
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if keep(r["Name"]):
                    lines.append(f"{r['Name'][:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                                 f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                                 f"{float(r['TotalDurationNs']) / 1e6:10.3f}")
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        # the same kernel runs at several shapes in one process: split by grid
        lines.append(f"## dispatches by grid ({os.path.basename(f)})")
        lines.append(f"{'kernel':60s} {'grid':>18s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
        by = defaultdict(list)
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if keep(r["Kernel_Name"]):
                    grid = "x".join(r.get(k, "?") for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"))
                    t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
                    by[(r["Kernel_Name"][:60], grid)].append((t0, (t1 - t0) / 1e3))
        for (name, grid), ev in sorted(by.items()):
            us = [d for _, d in ev]
            lines.append(f"{name:60s} {grid:>18s} {len(us):6d} {np.mean(us):10.2f} {min(us):10.2f} {max(us):10.2f}")
        lines.append(f"## attention dispatches in launch order, us ({os.path.basename(f)})")
        for (name, grid), ev in sorted(by.items()):
            if "k_attn_" in name and len(ev) <= 24:
                lines.append(f"{name[:60]:60s} " + " ".join(f"{d:.1f}" for _, d in sorted(ev)))
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        lines.append(f"## counters per dispatch ({os.path.basename(f)})")
        agg = defaultdict(list)
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if keep(r["Kernel_Name"]):
                    agg[(r["Kernel_Name"][:60], r["Counter_Name"])].append(float(r["Counter_Value"]))
        for (name, ctr), vals in sorted(agg.items()):
            lines.append(f"{name:60s} {ctr:14s} n={len(vals):3d} mean={np.mean(vals):.6g} "
                         f"min={min(vals):.6g} max={max(vals):.6g}")
    return "\n".join(lines)


# ---- device inputs -----------------------------------------------------------

def make_inputs(torch, dev):
    import msa_synth as syn
    dims = syn.Dims(num_q_heads=HQ, num_kv_heads=G, head_dim=D, index_dim=DI, block_size=BK, topk=TOPK)
    pin = syn.PrefillInputs(N_PREFILL, dims, 0, "planted", n_planted=8)
    pre = [t(device=dev)[None].contiguous() for t in (pin.q, pin.k, pin.v, pin.q_idx, pin.k_idx)]
    dec = syn.DecodeInputs(DEC_B, DEC_L, dims, 0)
    q = torch.stack([dec.q(b, dev) for b in range(DEC_B)]).contiguous()
    qi = torch.stack([dec.q_idx(b, dev) for b in range(DEC_B)]).contiguous()
    kc = torch.empty((DEC_B, DEC_L, G, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    kic = torch.empty((DEC_B, DEC_L, DI), dtype=torch.bfloat16, device=dev)
    for b in range(DEC_B):
        kc[b] = dec.k_cache(b, device=dev)
        vc[b] = dec.v_cache(b, device=dev)
        kic[b] = dec.k_idx_cache(b, device=dev)
    lens = torch.tensor(dec.ctx_lens, dtype=torch.int32, device=dev)
    return pin, pre, (q, qi, kc, vc, kic, lens), dec


# ---- CPU baseline (the oracle) and parity of the timed calls -----------------------

def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def _row_cost(rows, bk=BK, topk=TOPK):
    """Per-row oracle work model: index scoring over b_loc(i) older blocks
    plus attention over |T(i)| keys (both as flops)."""
    rows = np.asarray(rows, dtype=np.int64)
    b_loc = rows // bk
    t = bk * (np.minimum(topk, b_loc + 1) - 1) + rows % bk + 1
    return 2.0 * DI * G * bk * b_loc + 4.0 * D * HQ * t


def cpu_oracle(pin, rows, budget_s=15.0):
    """The float64 oracle on as many of `rows` (in the given order) as fit in
    the budget: half of it in one process with the default BLAS threads, half
    in a pool of one-BLAS-thread workers over all host cores. Returns the
    timing record and the oracle results of the rows done (for parity)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import msa_oracle as mo
    cores = len(os.sched_getaffinity(0))
    blas = _blas_threads()
    f = mo.to_f64
    t0 = time.time()
    ki, k, v = f(pin.k_idx()), f(pin.k()), f(pin.v())
    log(f"cpu_baseline: host inputs {time.time() - t0:.1f}s")
    chunk = 16
    done_rows, sel, out = [], [], []

    def run(rr):
        q, qi = f(pin.q(rr)), f(pin.q_idx(rr))
        return mo.prefill_rows(rr, q, qi, ki, k, v, block_size=BK, topk=TOPK)

    # one process, default BLAS threads
    single_flops, single_s, pos = 0.0, 0.0, 0
    while single_s < budget_s / 2 and pos < len(rows):
        rr = np.sort(rows[pos:pos + chunk])
        t = time.time()
        r = run(rr)
        single_s += time.time() - t
        single_flops += prefill_flops(rr)
        done_rows.append(rr), sel.append(r["sel"]), out.append(r["out"])
        pos += len(rr)
    # pool over all cores, one BLAS thread each
    pool_flops, pool_s = 0.0, 0.0
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limit = None
    try:
        with ThreadPoolExecutor(cores) as ex:
            while pool_s < budget_s / 2 and pos < len(rows):
                batch = [np.sort(rows[p:p + chunk]) for p in range(pos, min(len(rows), pos + chunk * cores), chunk)]
                t = time.time()
                res = list(ex.map(run, batch))
                pool_s += time.time() - t
                for rr, r in zip(batch, res):
                    pool_flops += prefill_flops(rr)
                    done_rows.append(rr), sel.append(r["sel"]), out.append(r["out"])
                pos += sum(len(rr) for rr in batch)
    finally:
        if limit is not None:
            limit.unregister()
    rows_done = np.concatenate(done_rows)
    # extrapolation of the full 32K prefill from the per-row work model
    all_rows = np.arange(N_PREFILL)
    scale = _row_cost(all_rows).sum() / _row_cost(rows_done).sum()
    pool_rate = pool_flops / pool_s if pool_s > 0 else 0.0
    rec = {"value": (pool_rate or single_flops / max(single_s, 1e-9)) / 1e12, "unit": "TFLOP/s", "cores": cores,
           "kind": "oracle",
           "sample": f"{len(rows_done)} stratified random rows of the 32768-token prefill workload (selection + "
                     f"attention, float64 numpy); value from the pool leg",
           "blas_threads": blas,
           "single_process": {"s": round(single_s, 2), "tflops": round(single_flops / max(single_s, 1e-9) / 1e12, 5)},
           "pool": {"workers": cores, "s": round(pool_s, 2), "tflops": round(pool_rate / 1e12, 5)},
           "extrapolated_full_prefill_s": round((single_s + pool_s) * scale, 1),
           "extrapolated_note": "extrapolated: sample time x (work model of all 32768 rows / of the sampled rows)"}
    return rec, rows_done, np.concatenate(sel), np.concatenate(out)


def prefill_parity(torch, got_sel, got_out, ref_sel, ref_out):
    """Bit-exact selection and max-abs / relative-L2 output error against the
    oracle on the same rows (bar: 2e-2 / 5e-3)."""
    g = got_out.astype(np.float64)
    diff = g - ref_out
    max_abs = float(np.abs(diff).max())
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref_out), 1e-30))
    sel_exact = bool(np.array_equal(got_sel, ref_sel))
    return {"rows": int(ref_out.shape[0]), "sel_exact": sel_exact, "max_abs": max_abs, "rel_l2": rel,
            "ok": sel_exact and max_abs <= 2e-2 and rel <= 5e-3}


def decode_parity(torch, dec, dec_in, out_d, seqs):
    """The timed decode call's outputs for `seqs` against the oracle (caches
    read row-wise from the device; q, q_idx regenerated on the host)."""
    from oracle import msa_oracle as mo
    q, qi, kc, vc, kic, lens = dec_in

    class Rows:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, idx):
            if isinstance(idx, tuple):
                idx = tuple(torch.as_tensor(np.asarray(i), device=self.t.device)
                            if not isinstance(i, (int, slice)) else i for i in idx)
            elif not isinstance(idx, (int, slice)):
                idx = torch.as_tensor(np.asarray(idx), device=self.t.device)
            return mo.to_f64(self.t[idx])

    import block_sparse_long_07_amd as msa
    _, sel_all, _ = msa.decode(q, qi, kc, vc, kic, lens, topk=TOPK, want_sel=True)
    max_abs, num, den, sel_exact = 0.0, 0.0, 0.0, True
    for b in seqs:
        L = dec.ctx_lens[b]
        ref = mo.decode_seq(mo.to_f64(dec.q(b)), mo.to_f64(dec.q_idx(b)), mo.to_f64(kic[b, :L]), Rows(kc[b]),
                            Rows(vc[b]), L, block_size=BK, topk=TOPK)
        got = out_d[b].double().cpu().numpy()
        d = got - ref["out"]
        max_abs = max(max_abs, float(np.abs(d).max()))
        num += float((d ** 2).sum())
        den += float((ref["out"] ** 2).sum())
        sel_exact &= bool(np.array_equal(sel_all[b].cpu().numpy(), ref["sel"]))
    rel = (num / max(den, 1e-30)) ** 0.5
    return {"seqs": len(seqs), "sel_exact": sel_exact, "max_abs": max_abs, "rel_l2": rel,
            "ok": sel_exact and max_abs <= 2e-2 and rel <= 5e-3}


# ---- context measurements ------------------------------------------------------

def ceilings(torch, reps=10):
    """Measured ceilings on this GPU: a bf16 torch.matmul (8192^3) and a 1 GiB
    device copy (1 GiB read + 1 GiB written)."""
    dev = torch.device("cuda:0")
    a = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    b = torch.randn((8192, 8192), device=dev).to(torch.bfloat16).t().contiguous()
    ms = _time_calls(torch, lambda: torch.matmul(a, b), reps)
    mm = 2.0 * 8192 ** 3 / (ms * 1e-3) / 1e12
    del a, b
    src = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    ms = _time_calls(torch, lambda: dst.copy_(src), reps)
    cp = 2.0 * (1 << 30) / (ms * 1e-3) / 1e9
    del src, dst
    return {"matmul_bf16_tflops": round(mm, 1), "matmul_frac_of_peak": round(mm / MFMA_PEAK_TFLOPS, 3),
            "copy_GB/s": round(cp, 1), "copy_frac_of_peak": round(cp / HBM_PEAK_GBS, 3)}


def topk_context(torch, msa, pre, reps):
    """The pages compare their top-k kernel with a generic top-k (3-5x). Here:
    msa_select_blocks against torch.topk (k-1 of the older blocks, the others
    masked to -inf beforehand, untimed) on the same pooled scores of the bench
    prefill. Context only: torch.topk neither forces the own block nor fixes
    the order of ties."""
    q, k, v, qi, ki = (t[0] for t in pre)
    n = qi.shape[0]
    sc = msa.index_scores(qi, ki, topk=TOPK)
    nb = sc.shape[-1]
    rows = torch.arange(n, device=sc.device)
    valid = torch.arange(nb, device=sc.device)[None, :] < (rows // BK)[:, None]
    masked = torch.where(valid[:, None, :], sc, torch.full_like(sc, float("-inf")))
    sel = torch.empty((G, n, TOPK), dtype=torch.int32, device=sc.device)
    ms_msa = _time_calls(torch, lambda: msa.select_blocks(sc, topk=TOPK, sel=sel), reps)
    ms_t = _time_calls(torch, lambda: torch.topk(masked, TOPK - 1, dim=-1), reps)
    del sc, masked, sel, valid
    return {"msa_topk_ms": round(ms_msa, 4), "torch_topk_ms": round(ms_t, 4),
            "torch_over_msa": round(ms_t / ms_msa, 2), "rows": n * G, "candidates_max": nb}


def _flush(torch, buf):
    buf.zero_()


def time_cold(torch, fn, reps, flush_bytes=512 << 20):
    """Mean time of fn after writing a 512 MiB buffer (evicts the 256 MB
    last-level cache and the L2s), events around fn only."""
    buf = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    ts = []
    for _ in range(reps):
        _flush(torch, buf)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del buf
    return float(np.mean(ts))


# ---- the longer configurations ------------------------------------------------------

def queue_spread(torch, msa, ws, p, n):
    """Balance of the persistent KV-outer pass over the last window of the
    latest prefill on `ws`: per-workgroup busy time (its own wall clock from
    start to exit) and tiles drained, and how many compute units held one."""
    torch.cuda.synchronize()
    m = msa.prefill_schedule_layout(p, n, n)
    sc = msa.read_prefill_schedule(ws, m, G)
    wg = sc["wg_trace"].numpy().astype(np.int64)
    info = sc["tile_info"].numpy()
    if len(wg) == 0 or m.wall_clock_khz <= 0:
        return None
    us = 1e3 / m.wall_clock_khz
    busy = (wg[:, 3] - wg[:, 2]) * us
    tiles = wg[:, 1]
    return {"window_rows": int(info[5]), "first_row": int(info[6]), "tiles": int(info[0]),
            "workgroups": int(len(wg)), "compute_units_used": int(len(np.unique(wg[:, 0]))),
            "visits_all_one": bool((sc["tile_visits"].numpy() == 1).all()),
            "busy_us": {"min": round(float(busy.min()), 1), "median": round(float(np.median(busy)), 1),
                        "max": round(float(busy.max()), 1), "max_over_mean": round(float(busy.max() / busy.mean()), 3)},
            "tiles_per_wg": {"min": int(tiles.min()), "median": float(np.median(tiles)), "max": int(tiles.max())},
            "first_exit_to_last_exit_us": round(float((wg[:, 3].max() - wg[:, 3].min()) * us), 1),
            "span_us": round(float((wg[:, 3].max() - wg[:, 2].min()) * us), 1),
            "clock_khz": int(m.wall_clock_khz)}


def config_prefill(torch, msa, label, inp, reps):
    """One prefill configuration: warm (mean of reps) and cold timings, the
    per-stage times, the attention kernels' roofline positions from the actual
    selection, and the index stage's rate."""
    dev = torch.device("cuda:0")
    n = inp.n
    t0 = time.time()
    pre = [fn(device=dev)[None].contiguous() for fn in (inp.q, inp.k, inp.v, inp.q_idx, inp.k_idx)]
    torch.cuda.synchronize()
    log(f"{label}: inputs ready in {time.time() - t0:.1f}s")
    p = msa.params(HQ, G, D, DI, BK, TOPK)
    ws = torch.empty(msa.prefill_workspace_bytes(p, 1, n), dtype=torch.uint8, device=dev)
    out = torch.empty_like(pre[0])
    run = lambda: msa.prefill(*pre, topk=TOPK, workspace=ws, out=out)
    ms = _time_calls(torch, run, reps)
    ms_cold = time_cold(torch, run, max(2, reps // 2))
    x = stage_times(msa, lambda **kw: msa.prefill(*pre, topk=TOPK, workspace=ws, out=out, **kw), max(2, reps // 2))
    stage = dict(zip(msa.PREFILL_STAGES, (float(v) for v in x)))
    _, sel, _ = msa.prefill(*pre, topk=TOPK, workspace=ws, out=out, want_sel=True)
    queue = queue_spread(torch, msa, ws, p, n)
    del ws, out, pre
    torch.cuda.empty_cache()
    ps, kernels = attention_rooflines(torch, sel[0], n, stage, measured=False)
    del sel
    torch.cuda.empty_cache()
    f_main, f_idx = prefill_flops_full(n), index_flops_full(n)
    dom = max(kernels, key=lambda r: r["ms"])
    log(f"{label}: {ms:.2f} ms warm, {ms_cold:.2f} ms cold")
    return {"workload": label, "ms": round(ms, 3), "ms_cold": round(ms_cold, 3),
            "F_main_tflop": round(f_main / 1e12, 3), "F_idx_tflop": round(f_idx / 1e12, 3),
            "tflops": round(f_main / (ms * 1e-3) / 1e12, 2),
            "end_to_end_tflops": round((f_main + f_idx) / (ms * 1e-3) / 1e12, 2),
            "index_tflops": round(f_idx / (stage["index_score"] * 1e-3) / 1e12, 2),
            "stage_ms": {k: round(v, 3) for k, v in stage.items()},
            "roofline": {k: dom[k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac", "traffic")},
            "kernels": kernels,
            "pairs": {k: ps[k] for k in ("dense_pairs", "sparse_pairs", "kv_dense", "kv_sparse",
                                         "dense_unit_blocks")},
            "kv_outer_queue": queue}


def config_decode(torch, msa, label, B, L, seed, reps):
    dev = torch.device("cuda:0")
    import msa_synth as syn
    dims = syn.Dims()
    t0 = time.time()
    dec = syn.DecodeInputs(B, L, dims, seed)
    q = torch.stack([dec.q(b, dev) for b in range(B)]).contiguous()
    qi = torch.stack([dec.q_idx(b, dev) for b in range(B)]).contiguous()
    kc = torch.empty((B, L, G, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    kic = torch.empty((B, L, DI), dtype=torch.bfloat16, device=dev)
    for b in range(B):
        kc[b] = dec.k_cache(b, device=dev)
        vc[b] = dec.v_cache(b, device=dev)
        kic[b] = dec.k_idx_cache(b, device=dev)
    lens = torch.tensor(dec.ctx_lens, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"{label}: inputs ready in {time.time() - t0:.1f}s")
    p = msa.params(HQ, G, D, DI, BK, TOPK)
    ws = torch.empty(msa.decode_workspace_bytes(p, B, L), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    run = lambda: msa.decode(q, qi, kc, vc, kic, lens, topk=TOPK, workspace=ws, out=out)
    ms = _time_calls(torch, run, reps)
    ms_cold = time_cold(torch, run, max(2, reps // 2))
    x = stage_times(msa, lambda **kw: msa.decode(q, qi, kc, vc, kic, lens, topk=TOPK, workspace=ws, out=out, **kw),
                    reps)
    db = decode_bytes(dec.ctx_lens)
    gbs = db / (ms * 1e-3) / 1e9
    del q, qi, kc, vc, kic, ws, out
    torch.cuda.empty_cache()
    return {"workload": label, "ms": round(ms, 4), "ms_cold": round(ms_cold, 4), "bytes_gb": round(db / 1e9, 4),
            "GB/s": round(gbs, 1), "GB/s_cold": round(db / (ms_cold * 1e-3) / 1e9, 1),
            "roofline": {"kernel": "decode (index + select + attention)", "bound": "hbm",
                         "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
            "stage_ms": {k: round(float(v), 4) for k, v in zip(msa.DECODE_STAGES, x)}}


def long_configs(torch, msa, reps):
    """The long-context configurations: the 128K prefill with hot blocks
    shared by most queries, the 1M-token prefill, and decode of 8 sequences
    with 1M-token caches."""
    import msa_synth as syn
    res = []
    inp = syn.PrefillInputs(131072, syn.Dims(), 3, "skewed", n_planted=4, n_hot=4)
    res.append(config_prefill(torch, msa, "prefill N=131072, skewed (4 hot blocks shared by all groups)", inp, reps))
    inp = syn.PrefillInputs(1 << 20, syn.Dims(), 4, "planted", n_planted=8)
    res.append(config_prefill(torch, msa, "prefill N=1048576", inp, max(2, reps // 4)))
    res.append(config_decode(torch, msa, "decode 8 x 1048576", 8, 1 << 20, 5, reps))
    return res


# ---- serving shapes (msa_prefill_varlen) --------------------------------------

def stage_times(msa, fn, reps):
    """Mean per-stage milliseconds of reps back-to-back calls fn(stage_timers=...)
    (the library's stage events on the launch stream; no synchronisation
    between the calls)."""
    timers = []
    for _ in range(reps):
        fn(stage_timers=timers)
    return np.mean(np.array(msa.read_stage_timers(timers)), axis=0)


def _time_calls(torch, fn, reps):
    fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        fn()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def serving_shapes(torch, msa, pre, topk, reps, n_chunks=4, varlen_lens=(8192, 6144, 4096, 2048)):
    """The 32K sequence prefilled as n_chunks chunks, each against the cache
    the previous ones filled, and a batch of prompts of mixed lengths (rows of
    the same tensors, one cache per prompt). Throughput = attended-token flops
    (the same F_main definition) / wall time of the calls."""
    q, k, v, qi, ki = (t[0] for t in pre)
    n = q.shape[0]
    step = n // n_chunks
    bounds = [(a, min(n, a + step)) for a in range(0, n, step)]
    p = msa.params(HQ, G, D, DI, BK, topk)
    ws = torch.empty(msa.prefill_varlen_workspace_bytes(p, step, n), dtype=torch.uint8, device=q.device)
    outs = [torch.empty((b - a, HQ, D), dtype=torch.bfloat16, device=q.device) for a, b in bounds]
    qs = [q[a:b].contiguous() for a, b in bounds]
    qis = [qi[a:b].contiguous() for a, b in bounds]

    def chunks():
        for (a, b), qc, qic, o in zip(bounds, qs, qis, outs):
            msa.prefill_varlen(qc, qic, k[None], v[None], ki[None], [a], [b - a], topk=topk, workspace=ws, out=o)

    ms_c = _time_calls(torch, chunks, reps)
    f_c = prefill_flops_full(n, topk=topk)
    chunked = {"chunks": len(bounds), "chunk_rows": step, "ms": round(ms_c, 4),
               "tflops": round(f_c / (ms_c * 1e-3) / 1e12, 2)}

    seg = max(varlen_lens)
    B = len(varlen_lens)
    assert B * seg <= n
    kc, vc, kic = (t[:B * seg].reshape((B, seg) + tuple(t.shape[1:])) for t in (k, v, ki))
    vq = torch.cat([q[b * seg:b * seg + L] for b, L in enumerate(varlen_lens)]).contiguous()
    vqi = torch.cat([qi[b * seg:b * seg + L] for b, L in enumerate(varlen_lens)]).contiguous()
    ws2 = torch.empty(msa.prefill_varlen_workspace_bytes(p, seg, seg), dtype=torch.uint8, device=q.device)
    vout = torch.empty_like(vq)

    def batch():
        msa.prefill_varlen(vq, vqi, kc, vc, kic, [0] * B, list(varlen_lens), topk=topk, workspace=ws2, out=vout)

    ms_v = _time_calls(torch, batch, reps)
    f_v = sum(prefill_flops_full(L, topk=topk) for L in varlen_lens)
    varlen = {"q_lens": list(varlen_lens), "ms": round(ms_v, 4), "tflops": round(f_v / (ms_v * 1e-3) / 1e12, 2)}
    return chunked, varlen


# ---- Index Branch KL-alignment backward ------------------------------------------

def kl_backward_measure(torch, msa, pre, topk, reps):
    """KL alignment of the Index Branch (loss, dq_idx, dk_idx) on the bench
    prefill, with the forward's selection and lse. Algorithmic HBM bytes per
    selected (row, group, block) pair: the query's 16 heads (4 KiB, pass 2),
    its index query twice (2 x 128 B), its 16 lse values (64 B), and the slot
    partials written and read back (2 x 268 B); per (group, block) its K block
    (32 KiB) and its k_idx block twice (2 x 16 KiB); per row and group the
    outputs (dq_idx 256 B, loss 4 B); per key dk_idx (256 B)."""
    q, k, v, qi, ki = pre
    _, sel, lse = msa.prefill(q, k, v, qi, ki, topk=topk, want_sel=True, want_lse=True)
    sel, lse = sel[0].contiguous(), lse[0].contiguous()
    q0, k0, qi0, ki0 = q[0], k[0], qi[0], ki[0]
    p = msa.params(HQ, G, D, DI, BK, topk)
    n = q0.shape[0]
    ws = torch.empty(msa.index_kl_workspace_bytes(p, n), dtype=torch.uint8, device=q0.device)
    ms = _time_calls(torch, lambda: msa.index_kl_backward(q0, k0, qi0, ki0, sel, lse, topk=topk, workspace=ws), reps)
    nb = (n + BK - 1) // BK
    pairs = G * sum(min(BK, n - blk * BK) * min(topk, blk + 1) for blk in range(nb))
    nbytes = (pairs * (4096 + 2 * 128 + 64 + 2 * 268) + G * nb * (32768 + 2 * 16384)
              + n * G * (256 + 4) + n * 256)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "pairs": int(pairs), "Mpairs/s": round(pairs / (ms * 1e-3) / 1e6, 1),
            "algorithmic_gb": round(nbytes / 1e9, 4), "GB/s": round(gbs, 1), "bound": "hbm",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


# ---- main ---------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--profile-reps", type=int, default=5, help="repetitions of the cold-cache timings")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after the run, stream 1 GiB through a plain elementwise kernel (torch.neg on int32, "
                         "1 GiB read + 1 GiB written) to scale rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="no GPU work: condense the rocprofv3 CSV output under DIR to text and exit")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-serving", action="store_true",
                    help="skip the chunked / variable-length prefill, KL-backward, B_k 64 / 32 and projection "
                         "measurements "
                         "(profiling runs use this so that per-kernel averages cover the headline workload only)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the long configurations (128K skewed prefill, 1M prefill, 8 x 1M decode) and the "
                         "context measurements (ceilings, top-k comparison)")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle check of the timed calls' outputs (profiling runs)")
    ap.add_argument("--configs-only", action="store_true",
                    help="run only the long configurations and print their JSON (profiling runs of those shapes)")
    args = ap.parse_args()
    if args.summarize_rocprof:
        print(summarize_rocprof(args.summarize_rocprof))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_long_07_amd as msa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    msa.load()
    dev = torch.device("cuda:0")
    if args.configs_only:
        print(json.dumps({"configs": long_configs(torch, msa, args.steps)}), flush=True)
        return
    t0 = time.time()
    pin, pre, dec_in, dec = make_inputs(torch, dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")

    p = msa.params(HQ, G, D, DI, BK, TOPK)
    ws_p = torch.empty(msa.prefill_workspace_bytes(p, 1, N_PREFILL), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(msa.decode_workspace_bytes(p, DEC_B, DEC_L), dtype=torch.uint8, device=dev)
    out_p = torch.empty_like(pre[0])
    out_d = torch.empty_like(dec_in[0])

    def step(evs=None, timers=None):
        if evs:
            evs[0].record()
        msa.prefill(*pre, topk=TOPK, workspace=ws_p, out=out_p, stage_timers=timers)
        if evs:
            evs[1].record()
        msa.decode(*dec_in, topk=TOPK, workspace=ws_d, out=out_d)
        if evs:
            evs[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed steps: torch events around each call, and the library's own
    # stage events for the prefill (recorded on the launch stream between its
    # kernels, read after the loop) for the per-kernel durations. The decode
    # call, 40x shorter, is timed without them (its three stage events cost
    # about 10 us of its 245); its stages come from a second loop below.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    timers = []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for e in evs:
        step(e, timers)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    stage_runs = msa.read_stage_timers(timers)
    pre_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    step_ms = wall * 1e3 / args.steps

    # the timed calls' own outputs, kept for the oracle comparison below
    import msa_synth as syn
    planted = sorted({b for g in pin.planted.values() for b in g})
    par_rows = syn.stratified_rows(N_PREFILL, 4096, BK, 0, TOPK, extra=planted)
    np.random.default_rng(1).shuffle(par_rows)
    timed_out_rows = out_p[0][torch.as_tensor(par_rows, device=dev)].float().cpu().numpy()
    timed_out_d = out_d.clone()

    # per-stage times: the prefill's from the timed steps, the decode's from
    # as many back-to-back decode calls with stage events
    pst = np.mean(np.array(stage_runs), axis=0)
    for _ in range(args.steps):
        msa.decode(*dec_in, topk=TOPK, workspace=ws_d, out=out_d, stage_timers=timers)
    dst = np.mean(np.array(msa.read_stage_timers(timers)), axis=0)

    f_main = prefill_flops_full(N_PREFILL)
    f_idx = index_flops_full(N_PREFILL)
    dbytes = decode_bytes(dec.ctx_lens)
    value = f_main / (pre_ms * 1e-3) / 1e12
    stage = dict(zip(msa.PREFILL_STAGES, (float(x) for x in pst)))
    t_main_ms = stage["reverse_index"] + stage["kv_outer_attn"] + stage["dense_attn_merge"]
    dec_gbs = dbytes / (dec_ms * 1e-3) / 1e9
    dec_idx_bytes = sum((BK * ((L - 1) // BK) if (L - 1) // BK >= TOPK else 0) * DI * 2 for L in dec.ctx_lens)

    # roofline of the two attention kernels from the actual selection
    _, sel, _ = msa.prefill(*pre, topk=TOPK, workspace=ws_p, out=out_p, want_sel=True)
    ps, kernels = attention_rooflines(torch, sel[0], N_PREFILL, stage)
    par_sel = sel[0][:, torch.as_tensor(par_rows, device=dev)].permute(1, 0, 2).cpu().numpy()
    del sel
    queue = queue_spread(torch, msa, ws_p, p, N_PREFILL)
    assert abs(ps["F_dense"] + ps["F_sparse"] - f_main) <= 1e-9 * f_main, "pair split does not cover F_main"
    dom = max(kernels, key=lambda r: r["ms"])

    cold = {"prefill_ms": round(time_cold(torch, lambda: msa.prefill(*pre, topk=TOPK, workspace=ws_p, out=out_p),
                                          args.profile_reps), 4),
            "decode_ms": round(time_cold(torch, lambda: msa.decode(*dec_in, topk=TOPK, workspace=ws_d, out=out_d),
                                         args.profile_reps), 4)}
    cold["prefill_tflops"] = round(prefill_flops_full(N_PREFILL) / (cold["prefill_ms"] * 1e-3) / 1e12, 2)
    cold["decode_GB/s"] = round(decode_bytes(dec.ctx_lens) / (cold["decode_ms"] * 1e-3) / 1e9, 1)
    context = None
    if not args.no_configs:
        context = {"ceilings": ceilings(torch), "topk": topk_context(torch, msa, pre, args.steps)}

    chunked, varlen = (None, None) if args.no_serving else serving_shapes(torch, msa, pre, TOPK, args.steps)
    kl = None if args.no_serving else kl_backward_measure(torch, msa, pre, TOPK, args.steps)
    variants = (None if args.no_serving else
                block_size_variants(torch, msa, pre, dec_in, dec.ctx_lens, TOPK, args.steps))
    proj = None if args.no_serving else projection_measure(torch, msa, N_PREFILL, DEC_B, args.steps)

    parity = None
    if not args.no_parity:
        dpar = decode_parity(torch, dec, dec_in, timed_out_d, [0, 9, 18, 27, 36, 45, 54, 63])
    del ws_p, ws_d, out_p, out_d, timed_out_d, pre, dec_in
    torch.cuda.empty_cache()
    configs = None if args.no_configs else long_configs(torch, msa, args.steps)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded Irwin-Hall ~N(0,1) bf16 Q/K/V, integer index keys with planted needles",
        "config": {"workload": "prefill N=32768 (64q/4kv, d=128, d_idx=64, B_k=128, k=16) + decode 64 x 131072",
                   "global_batch": 1, "seq_len": N_PREFILL, "decode_batch": DEC_B, "decode_ctx": DEC_L,
                   "parallelism": "single GPU"},
        "pct_of_mfma_peak": round(100 * value / MFMA_PEAK_TFLOPS, 2),
        "prefill": {"ms": round(pre_ms, 4), "F_main_tflop": round(f_main / 1e12, 4),
                    "F_idx_tflop": round(f_idx / 1e12, 4),
                    "stage_ms": {k: round(x, 4) for k, x in stage.items()},
                    "stage_ms_source": "HIP events the library records on the launch stream between its kernels, "
                                       "in every timed step (mean over the steps)",
                    "main_branch_tflops": round(f_main / (t_main_ms * 1e-3) / 1e12, 2),
                    "end_to_end_tflops": round((f_main + f_idx) / (pre_ms * 1e-3) / 1e12, 2),
                    "index_tflops": round(f_idx / (float(pst[0]) * 1e-3) / 1e12, 2)},
        "decode": {"ms": round(dec_ms, 4), "bytes_gb": round(dbytes / 1e9, 4), "GB/s": round(dec_gbs, 1),
                   "pct_of_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 2),
                   "stage_ms": {k: round(float(x), 4) for k, x in zip(msa.DECODE_STAGES, dst)},
                   "index_GB/s": round(dec_idx_bytes / (float(dst[0]) * 1e-3) / 1e9, 1)},
        "roofline": {"kernel": dom["kernel"], "bound": dom["bound"], "achieved": dom["achieved"],
                     "peak": dom["peak"], "unit": dom["unit"], "frac": dom["frac"], "traffic": dom["traffic"],
                     "traffic_unit": "HBM bytes per launch (rocprofv3, calibrated)",
                     "algorithmic_bytes": round(dom["algorithmic_gb"] * 1e9)},
        "kernels": kernels,
        "pairs": {k: ps[k] for k in ("dense_pairs", "sparse_pairs", "kv_dense", "kv_sparse", "dense_unit_blocks")},
        "chunked_prefill": chunked,
        "varlen_prefill": varlen,
        "index_kl_backward": kl,
        "block_size_variants": variants,
        "index_projection": proj,
        "cold_cache": cold,
        "kv_outer_queue": queue,
        "context": context,
        "configs": configs,
    }
    if not (args.no_parity and args.no_cpu_baseline):
        rec, rows_done, ref_sel, ref_out = cpu_oracle(pin, par_rows, args.cpu_budget)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = rec
        if not args.no_parity:
            pos = {int(r): i for i, r in enumerate(par_rows)}
            ix = np.array([pos[int(r)] for r in rows_done])
            ppar = prefill_parity(torch, par_sel[ix], timed_out_rows[ix], ref_sel, ref_out)
            parity = {"prefill": ppar, "decode": dpar,
                      "bar": "selection bit-exact; max-abs <= 2e-2, rel-L2 <= 5e-3 vs the float64 oracle",
                      "what": "outputs of the timed calls themselves (no selection / lse output, reused workspace)"}
            res["parity"] = parity
    print(json.dumps(res), flush=True)
    if parity is not None and not (parity["prefill"]["ok"] and parity["decode"]["ok"]):
        print("parity check of the timed calls failed", file=sys.stderr)
        sys.exit(3)
    if args.calibration_copy:
        src = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
        dst = torch.neg(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy done: 1 GiB read, 1 GiB written (neg kernel)")


if __name__ == "__main__":
    main()
