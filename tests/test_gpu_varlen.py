"""GPU parity of the variable-length / chunked prefill entry point
(msa_prefill_varlen) against the float64 oracle.

A chunk's rows are the same rows of the whole sequence (row i depends only on
positions <= i), so the oracle of the whole sequence is the reference for every
chunk. Cache positions past a chunk's end hold NaN: a kernel that read a future
position would poison the output. When every chunk starts at a multiple of 16
the 16-row units are those of a one-call prefill, so the outputs must be
identical bit for bit to that call's.

Bar as in the other parity tests: selection bit-exact, outputs max-abs 2e-2 and
relative L2 5e-3, lse 4e-3.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_07_amd as msa
import msa_synth as syn
from tests._parity import compare_lse, compare_out, log, oracle_prefill, prefill_device_inputs, timed

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    msa.load()  # raises if the HIP library is missing: no fallback exists
    yield
    torch.cuda.empty_cache()


def dims(G, topk):
    return syn.Dims(num_q_heads=16 * G, num_kv_heads=G, head_dim=128, index_dim=64, block_size=128, topk=topk)


def cache_upto(rows: torch.Tensor, valid: int, max_ctx: int) -> torch.Tensor:
    """[max_ctx, ...] copy of the first `valid` rows; every later position NaN."""
    t = torch.empty((max_ctx,) + tuple(rows.shape[1:]), dtype=torch.bfloat16, device=rows.device)
    t.view(torch.int16).fill_(BF16_NAN)
    t[:valid] = rows[:valid]
    return t


def check_rows(out, sel, lse, ref, lo, hi, label):
    """out [R,Hq,d], sel [G,R,k], lse [R,Hq] of rows lo..hi-1 vs the oracle's
    rows (ref holds rows 0.. of the sequence)."""
    got_sel = sel.permute(1, 0, 2).cpu().numpy()
    mism = np.argwhere(got_sel != ref["sel"][lo:hi])
    assert mism.size == 0, f"{label}: selection mismatch at {mism[:5].tolist()}"
    compare_out(out, ref["out"][lo:hi], f"{label} out")
    compare_lse(lse, ref["lse"][lo:hi], label)


@pytest.mark.parametrize("G,topk,recipe,bounds", [
    (2, 8, "planted", [0, 5, 21, 700, 1030, 1031, 2048, 3000]),
    (4, 16, "planted", [0, 1999, 2000, 2013, 4096]),
    (1, 4, "tiny", [0, 127, 129, 255, 2047, 2048]),
])
def test_chunked_prefill_vs_oracle(G, topk, recipe, bounds):
    n = bounds[-1]
    inp = syn.PrefillInputs(n, dims(G, topk), 31, recipe, n_planted=4)
    q, k, v, qi, ki = (x[0] for x in prefill_device_inputs(inp))
    log(f"case chunked N={n} G={G} k={topk} bounds={bounds}")
    with timed("oracle"):
        ref = oracle_prefill(inp, np.arange(n), topk)
    for a, b in zip(bounds[:-1], bounds[1:]):
        log(f"  chunk [{a}, {b})")
        kc, vc, kic = (cache_upto(t, b, n)[None] for t in (k, v, ki))
        out, sel, lse = msa.prefill_varlen(q[a:b].contiguous(), qi[a:b].contiguous(), kc, vc, kic, [a], [b - a],
                                           topk=topk, want_sel=True, want_lse=True)
        torch.cuda.synchronize()
        check_rows(out, sel, lse, ref, a, b, f"chunk [{a},{b})")


def test_chunks_at_multiples_of_16_equal_one_call():
    n, G, topk = 5000, 4, 16
    inp = syn.PrefillInputs(n, dims(G, topk), 41, "planted")
    q, k, v, qi, ki = prefill_device_inputs(inp)
    full_out, full_sel, full_lse = msa.prefill(q, k, v, qi, ki, topk=topk, want_sel=True, want_lse=True)
    q, k, v, qi, ki = q[0], k[0], v[0], qi[0], ki[0]
    bounds = [0, 16, 528, 2048, 2064, 4112, 5000]
    log(f"case aligned chunks N={n} bounds={bounds}")
    for a, b in zip(bounds[:-1], bounds[1:]):
        kc, vc, kic = (cache_upto(t, b, n)[None] for t in (k, v, ki))
        out, sel, lse = msa.prefill_varlen(q[a:b].contiguous(), qi[a:b].contiguous(), kc, vc, kic, [a], [b - a],
                                           topk=topk, want_sel=True, want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(sel, full_sel[0][:, a:b]), f"chunk [{a},{b}) selection"
        assert torch.equal(out.view(torch.int16), full_out[0][a:b].view(torch.int16)), f"chunk [{a},{b}) out"
        assert torch.equal(lse, full_lse[0][a:b]), f"chunk [{a},{b}) lse"


@pytest.mark.parametrize("bk", [128, 32])
def test_varlen_batch_vs_oracle(bk):
    G, topk = 4, 16
    # (q_start, q_len): fresh prompts, continuations of a cache, one token,
    # an empty entry, an unaligned start with a ragged length
    specs = [(0, 1500), (777, 1300), (2000, 1), (3, 0), (1040, 37), (0, 2100)]
    max_ctx = 2100
    B = len(specs)
    d = syn.Dims(num_q_heads=16 * G, num_kv_heads=G, head_dim=128, index_dim=64, block_size=bk, topk=topk)
    inps = [syn.PrefillInputs(max(s + l, 1), d, 50 + b, "planted", n_planted=3)
            for b, (s, l) in enumerate(specs)]
    kc = torch.empty((B, max_ctx, G, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    kic = torch.empty((B, max_ctx, 64), dtype=torch.bfloat16, device="cuda")
    qs, qis = [], []
    for b, ((s, l), inp) in enumerate(zip(specs, inps)):
        ctx = s + l
        kc[b] = cache_upto(inp.k(device="cuda"), ctx, max_ctx)
        vc[b] = cache_upto(inp.v(device="cuda"), ctx, max_ctx)
        kic[b] = cache_upto(inp.k_idx(device="cuda"), ctx, max_ctx)
        rows = np.arange(s, s + l)
        if l:
            qs.append(inp.q(rows, device="cuda"))
            qis.append(inp.q_idx(rows, device="cuda"))
    q = torch.cat(qs).contiguous()
    qi = torch.cat(qis).contiguous()
    log(f"case varlen batch B_k={bk} specs={specs}")
    out, sel, lse = msa.prefill_varlen(q, qi, kc, vc, kic, [s for s, _ in specs], [l for _, l in specs],
                                       topk=topk, block_size=bk, want_sel=True, want_lse=True)
    torch.cuda.synchronize()
    r = 0
    for b, ((s, l), inp) in enumerate(zip(specs, inps)):
        if l:
            ref = oracle_prefill(inp, np.arange(s, s + l), topk)
            got = (out[r:r + l], sel[:, r:r + l], lse[r:r + l])
            check_rows(*got, ref, 0, l, f"seq{b} [{s},{s + l})")
        r += l


def test_varlen_nothing_to_do():
    kc = torch.zeros((2, 256, 4, 128), dtype=torch.bfloat16, device="cuda")
    ki = torch.zeros((2, 256, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((0, 64, 128), dtype=torch.bfloat16, device="cuda")
    qi = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    out, sel, lse = msa.prefill_varlen(q, qi, kc, kc, ki, [0, 100], [0, 0], want_sel=True, want_lse=True)
    assert out.shape == (0, 64, 128) and sel.shape == (4, 0, 16) and lse.shape == (0, 64)
