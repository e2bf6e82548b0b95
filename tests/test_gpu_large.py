"""GPU parity at the large configurations, on seeded sampled rows:
skewed 128K prefill (hot blocks shared by every group), 1M-token prefill (16
query windows), and decode of 8 sequences with 1M-token caches.

Device inputs come from the same counter-based generator the oracle uses; for
these sizes the oracle reads the big key/value tensors through row-wise copies
of the device tensors (the generator's CPU/GPU equality is checked in
test_gpu_parity.py), and regenerates the sampled query rows on the CPU.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_07_amd as msa
import msa_synth as syn
from oracle import msa_oracle as mo
from tests._parity import compare_lse, compare_out, log, timed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    msa.load()
    yield
    torch.cuda.empty_cache()


class RowsF64:
    """Row-indexed float64 view of a device bf16 tensor."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, idx):
        if isinstance(idx, tuple):
            idx = tuple(torch.as_tensor(np.asarray(i), device=self.t.device) if not isinstance(i, (int, slice))
                        else i for i in idx)
        elif not isinstance(idx, (int, slice)):
            idx = torch.as_tensor(np.asarray(idx), device=self.t.device)
        return mo.to_f64(self.t[idx])


def oracle_rows_threaded(rows, q_rows, qi_rows, ki, k, v, topk, threads=16, block_size=128):
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    parts = np.array_split(np.arange(len(rows)), max(1, min(64, len(rows) // 16)))
    done = [0]

    def run(ix):
        r = mo.prefill_rows(rows[ix], q_rows[ix], qi_rows[ix], ki, k, v, block_size=block_size, topk=topk)
        done[0] += len(ix)
        if done[0] % 512 < len(ix):
            log(f"    oracle rows {done[0]}/{len(rows)}")
        return r

    with threadpool_limits(1):
        with ThreadPoolExecutor(threads) as ex:
            res = list(ex.map(run, parts))
    return {key: np.concatenate([r[key] for r in res]) for key in ("sel", "out", "lse")}


def prefill_sampled(inp, topk, rows, label):
    bk = inp.dims.block_size
    dev = "cuda"
    log(f"case {label}: N={inp.n} rows={len(rows)}")
    with timed("inputs"):
        q = inp.q(device=dev)[None]
        k = inp.k(device=dev)[None]
        v = inp.v(device=dev)[None]
        qi = inp.q_idx(device=dev)[None]
        ki = inp.k_idx(device=dev)[None]
        torch.cuda.synchronize()
    with timed("gpu"):
        out, sel, lse = msa.prefill(q, k, v, qi, ki, topk=topk, block_size=bk, want_sel=True, want_lse=True)
        torch.cuda.synchronize()
    rows = np.asarray(rows, dtype=np.int64)
    rt = torch.as_tensor(rows, device=dev)
    got_sel = sel[0][:, rt].permute(1, 0, 2).cpu().numpy()
    got_out = out[0][rt].cpu()
    got_lse = lse[0][rt].cpu()
    del out, lse, q
    with timed("oracle"):
        ref = oracle_rows_threaded(rows, mo.to_f64(inp.q(rows)), mo.to_f64(inp.q_idx(rows)),
                                   mo.to_f64(ki[0]), RowsF64(k[0]), RowsF64(v[0]), topk, block_size=bk)
    mism = np.argwhere(got_sel != ref["sel"])
    assert mism.size == 0, f"selection mismatch at {mism[:5].tolist()}"
    compare_out(got_out, ref["out"], f"{label} out")
    compare_lse(got_lse, ref["lse"], label)


@pytest.mark.timeout(1200)
def test_prefill_128k_skewed_sampled():
    n, topk = 131072, 16
    inp = syn.PrefillInputs(n, syn.Dims(), 3, "skewed", n_planted=4, n_hot=4)
    extra = sorted(set(inp.hot) | {b for g in inp.planted.values() for b in g})
    rows = syn.stratified_rows(n, 4096, 128, 3, topk, extra=extra)
    prefill_sampled(inp, topk, rows, "prefill 128K skewed")


@pytest.mark.timeout(1800)
def test_prefill_1m_sampled():
    n, topk = 1 << 20, 16
    inp = syn.PrefillInputs(n, syn.Dims(), 4, "planted", n_planted=8)
    extra = sorted({b for g in inp.planted.values() for b in g})
    # rows at every window boundary (65536-row windows) and the ragged tail
    bounds = [w * 65536 + o for w in range(16) for o in (0, 1, 127, 128, 65535) if w * 65536 + o < n]
    rows = np.union1d(syn.stratified_rows(n, 4096, 128, 4, topk, extra=extra), bounds)
    prefill_sampled(inp, topk, rows, "prefill 1M")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("bk", [64, 32])
def test_prefill_longest_at_small_blocks_sampled(bk):
    """The longest sequence a smaller block size takes (2^20 * B_k / 128
    positions: 8192 blocks, as at B_k = 128 and 1M), over several windows."""
    n, topk = (1 << 20) * bk // 128, 16
    dims = syn.Dims(block_size=bk)
    inp = syn.PrefillInputs(n, dims, 9, "planted", n_planted=8)
    extra = sorted({b for g in inp.planted.values() for b in g})
    bounds = [w * 65536 + o for w in range(n // 65536 + 1) for o in (0, 1, bk - 1, bk, 65535)
              if w * 65536 + o < n] + [n - 1]
    rows = np.union1d(syn.stratified_rows(n, 2048, bk, 7, topk, extra=extra), bounds)
    prefill_sampled(inp, topk, rows, f"prefill {n} at B_k={bk}")


@pytest.mark.timeout(1200)
def test_decode_1m_eight_sequences():
    B, L, topk, G = 8, 1 << 20, 16, 4
    dims = syn.Dims()
    lens = [L, L - 1, L - 127, L - 128, 65537, 1000000, 700001, L]
    dec = syn.DecodeInputs(B, L, dims, 5, ctx_lens=lens)
    log(f"case decode 8x1M")
    with timed("inputs"):
        q = torch.stack([dec.q(b, "cuda") for b in range(B)]).contiguous()
        qi = torch.stack([dec.q_idx(b, "cuda") for b in range(B)]).contiguous()
        kc = torch.empty((B, L, G, 128), dtype=torch.bfloat16, device="cuda")
        vc = torch.empty_like(kc)
        kic = torch.empty((B, L, 64), dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            kc[b] = dec.k_cache(b, device="cuda")
            vc[b] = dec.v_cache(b, device="cuda")
            kic[b] = dec.k_idx_cache(b, device="cuda")
        ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    with timed("gpu"):
        out, sel, lse = msa.decode(q, qi, kc, vc, kic, ctx, topk=topk, want_sel=True, want_lse=True)
        torch.cuda.synchronize()
    with timed("oracle"):
        for b in range(B):
            Lb = lens[b]
            ref = mo.decode_seq(mo.to_f64(dec.q(b)), mo.to_f64(dec.q_idx(b)), mo.to_f64(kic[b, :Lb]),
                                RowsF64(kc[b]), RowsF64(vc[b]), Lb, block_size=128, topk=topk)
            assert np.array_equal(sel[b].cpu().numpy(), ref["sel"]), f"seq {b}"
            compare_out(out[b], ref["out"], f"decode 1M seq{b}")
            compare_lse(lse[b], ref["lse"], f"decode 1M seq{b}")


@pytest.mark.timeout(1200)
def test_chunk_across_windows_sampled():
    """A 69995-row chunk continuing a 5-token cache: an unaligned 11-row head
    window, a full 65536-row window and a ragged tail window."""
    n, a, topk, max_ctx = 70000, 5, 16, 70400
    inp = syn.PrefillInputs(n, syn.Dims(), 6, "planted", n_planted=8)
    dev = "cuda"
    log(f"case chunk [{a},{n}) of a {max_ctx}-position cache")
    with timed("inputs"):
        chunk = np.arange(a, n)
        q = inp.q(chunk, device=dev)
        qi = inp.q_idx(chunk, device=dev)
        caches = []
        for t in (inp.k(device=dev), inp.v(device=dev), inp.k_idx(device=dev)):
            c = torch.empty((1, max_ctx) + tuple(t.shape[1:]), dtype=torch.bfloat16, device=dev)
            c.view(torch.int16).fill_(0x7FC0)  # NaN past the chunk's end
            c[0, :n] = t
            caches.append(c)
            del t
        torch.cuda.synchronize()
    with timed("gpu"):
        out, sel, lse = msa.prefill_varlen(q, qi, *caches, [a], [n - a], topk=topk, want_sel=True, want_lse=True)
        torch.cuda.synchronize()
    extra = sorted({b for g in inp.planted.values() for b in g})
    edges = [5, 6, 15, 16, 17, 127, 128, 65551, 65552, 65553, 69999]
    rows = np.union1d(syn.stratified_rows(n, 1536, 128, 6, topk, extra=extra), edges)
    rows = rows[rows >= a]
    rt = torch.as_tensor(rows - a, device=dev)
    got_sel = sel[:, rt].permute(1, 0, 2).cpu().numpy()
    got_out, got_lse = out[rt].cpu(), lse[rt].cpu()
    k0, v0, ki0 = caches
    with timed("oracle"):
        ref = oracle_rows_threaded(rows, mo.to_f64(inp.q(rows)), mo.to_f64(inp.q_idx(rows)),
                                   mo.to_f64(ki0[0, :n]), RowsF64(k0[0]), RowsF64(v0[0]), topk)
    mism = np.argwhere(got_sel != ref["sel"])
    assert mism.size == 0, f"selection mismatch at {mism[:5].tolist()}"
    compare_out(got_out, ref["out"], "chunk out")
    compare_lse(got_lse, ref["lse"], "chunk")
