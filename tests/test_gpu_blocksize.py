"""GPU parity of the smaller key blocks, B_k = 64 and 32, against the float64
oracle (which takes B_k as a parameter): pooled scores and selections bit for
bit, outputs and lse to the bar of the B_k = 128 tests (tests/_parity.py).
Covers whole-sequence prefill (every row, ragged tails, one to several
windows' worth of blocks), chunked prefill over a cache with unaligned chunk
starts, and decode with ragged context lengths."""
import numpy as np
import pytest
import torch

import block_sparse_long_07_amd as msa
import msa_synth as syn
from oracle import msa_oracle as mo
from tests._parity import compare_lse, compare_out, log, oracle_prefill, prefill_device_inputs, timed

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    msa.load()
    yield
    torch.cuda.empty_cache()


def dims(G, topk, bk):
    return syn.Dims(num_q_heads=16 * G, num_kv_heads=G, head_dim=128, index_dim=64, block_size=bk, topk=topk)


def check_sel_out_lse(out, sel, lse, ref, rows, label):
    rt = torch.as_tensor(rows, device=sel.device)
    got_sel = sel[:, rt].permute(1, 0, 2).cpu().numpy()
    mism = np.argwhere(got_sel != ref["sel"])
    assert mism.size == 0, f"{label}: selection mismatch at {mism[:5].tolist()}"
    compare_out(out[rt], ref["out"], f"{label} out")
    compare_lse(lse[rt], ref["lse"], label)


@pytest.mark.parametrize("bk", [64, 32])
@pytest.mark.parametrize("G,n,recipe,topk", [(1, 2048, "tiny", 4), (4, 3001, "planted", 16), (2, 700, "tiny", 3)])
def test_index_scores_exact(bk, G, n, recipe, topk):
    inp = syn.PrefillInputs(n, dims(G, topk, bk), 3, recipe)
    qi = inp.q_idx(device="cuda").contiguous()
    ki = inp.k_idx(device="cuda").contiguous()
    sc = msa.index_scores(qi, ki, topk=topk, block_size=bk)
    torch.cuda.synchronize()
    assert sc.shape[-1] == (n + bk - 1) // bk
    rows = [r for r in syn.stratified_rows(n, 256, bk, 3, topk) if r // bk >= topk]
    ref = oracle_prefill(inp, rows, topk, want_scores=True)
    got = sc.cpu().numpy()
    for r, i in enumerate(rows):
        b_loc = i // bk
        assert np.array_equal(got[i, :, :b_loc], ref["scores"][r]), f"row {i}"


@pytest.mark.parametrize("bk", [64, 32])
@pytest.mark.parametrize("n", [5000, 600])   # thread-per-row and wave-per-row kernels
@pytest.mark.parametrize("topk", [1, 4, 16])
def test_select_exact_with_ties(bk, topk, n):
    G = 2
    nb = (n + bk - 1) // bk
    g = torch.Generator().manual_seed(100 + topk)
    scores = torch.randint(-2, 3, (n, G, nb), generator=g).float()
    sel = msa.select_blocks(scores.cuda().contiguous(), topk=topk, block_size=bk)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    s = scores.numpy().astype(np.float64)
    for i in range(0, n, 5 if n > 2000 else 1):
        b_loc = i // bk
        for gg in range(G):
            want = mo.select_blocks(s[i, gg, :b_loc], b_loc, topk)
            assert got[gg, i].tolist() == want.tolist(), (i, gg)


@pytest.mark.parametrize("bk", [64, 32])
@pytest.mark.parametrize("n,G,topk,recipe", [
    (1, 1, 4, "tiny"), (33, 1, 2, "tiny"), (129, 1, 4, "tiny"), (1000, 2, 4, "planted"),
    (2500, 4, 16, "planted"), (1920, 1, 1, "tiny"), (4321, 3, 7, "tiny"), (1500, 8, 16, "planted"),
])
def test_prefill_all_rows(bk, n, G, topk, recipe):
    inp = syn.PrefillInputs(n, dims(G, topk, bk), 5, recipe, n_planted=2)
    log(f"case B_k={bk} N={n} G={G} k={topk} recipe={recipe}")
    q, k, v, qi, ki = prefill_device_inputs(inp)
    with timed("gpu"):
        out, sel, lse = msa.prefill(q, k, v, qi, ki, topk=topk, block_size=bk, want_sel=True, want_lse=True)
        torch.cuda.synchronize()
    rows = np.arange(n)
    with timed("oracle"):
        ref = oracle_prefill(inp, rows, topk)
    check_sel_out_lse(out[0], sel[0], lse[0], ref, rows, f"B_k={bk} N={n}")


@pytest.mark.parametrize("bk", [64, 32])
def test_prefill_16k_sampled(bk):
    """Many blocks per row (512 at B_k = 32): the selection then differs from
    the forced ones for most rows."""
    n, G, topk = 16384, 4, 16
    inp = syn.PrefillInputs(n, dims(G, topk, bk), 8, "planted", n_planted=6)
    q, k, v, qi, ki = prefill_device_inputs(inp)
    log(f"case B_k={bk} N={n} sampled")
    out, sel, lse = msa.prefill(q, k, v, qi, ki, topk=topk, block_size=bk, want_sel=True, want_lse=True)
    torch.cuda.synchronize()
    rows = syn.stratified_rows(n, 512, bk, 2, topk, extra=sorted({b for g in inp.planted.values() for b in g}))
    with timed("oracle"):
        ref = oracle_prefill(inp, rows, topk)
    check_sel_out_lse(out[0], sel[0], lse[0], ref, rows, f"B_k={bk} 16K")


def cache_upto(rows: torch.Tensor, valid: int, max_ctx: int) -> torch.Tensor:
    """[max_ctx, ...] copy of the first `valid` rows; every later position NaN."""
    t = torch.empty((max_ctx,) + tuple(rows.shape[1:]), dtype=torch.bfloat16, device=rows.device)
    t.view(torch.int16).fill_(BF16_NAN)
    t[:valid] = rows[:valid]
    return t


@pytest.mark.parametrize("bk,bounds", [(64, [0, 5, 63, 64, 700, 1031, 2048, 2600]),
                                       (32, [0, 31, 33, 500, 1030, 2013, 2600])])
def test_chunked_prefill_vs_oracle(bk, bounds):
    n, G, topk = bounds[-1], 2, 8
    inp = syn.PrefillInputs(n, dims(G, topk, bk), 31, "planted", n_planted=4)
    q, k, v, qi, ki = (x[0] for x in prefill_device_inputs(inp))
    log(f"case B_k={bk} chunked bounds={bounds}")
    with timed("oracle"):
        ref = oracle_prefill(inp, np.arange(n), topk)
    for a, b in zip(bounds[:-1], bounds[1:]):
        kc, vc, kic = (cache_upto(t, b, n)[None] for t in (k, v, ki))
        out, sel, lse = msa.prefill_varlen(q[a:b].contiguous(), qi[a:b].contiguous(), kc, vc, kic, [a], [b - a],
                                           topk=topk, block_size=bk, want_sel=True, want_lse=True)
        torch.cuda.synchronize()
        got_sel = sel.permute(1, 0, 2).cpu().numpy()
        assert np.array_equal(got_sel, ref["sel"][a:b]), f"chunk [{a},{b}) selection"
        compare_out(out, ref["out"][a:b], f"chunk [{a},{b}) out")
        compare_lse(lse, ref["lse"][a:b], f"chunk [{a},{b})")


@pytest.mark.parametrize("bk,G", [(64, 4), (32, 4), (64, 1), (32, 8)])
def test_decode_ragged(bk, G):
    topk, B, max_ctx = 16, 7, 3000
    lens = [1, bk, bk + 1, 1500, 2048, 2999, 3000]
    dec = syn.DecodeInputs(B, max_ctx, dims(G, topk, bk), 4, ctx_lens=lens)
    log(f"case decode B_k={bk} G={G}")
    q = torch.stack([dec.q(b, "cuda") for b in range(B)]).contiguous()
    qi = torch.stack([dec.q_idx(b, "cuda") for b in range(B)]).contiguous()
    kc = torch.stack([dec.k_cache(b, device="cuda") for b in range(B)]).contiguous()
    vc = torch.stack([dec.v_cache(b, device="cuda") for b in range(B)]).contiguous()
    kic = torch.stack([dec.k_idx_cache(b, device="cuda") for b in range(B)]).contiguous()
    # positions past each context are NaN: nothing may read them
    for b, L in enumerate(lens):
        for t in (kc, vc, kic):
            t[b, L:].view(torch.int16).fill_(BF16_NAN)
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, sel, lse = msa.decode(q, qi, kc, vc, kic, lt, topk=topk, block_size=bk, want_sel=True, want_lse=True)
    torch.cuda.synchronize()
    f = mo.to_f64
    for b, L in enumerate(lens):
        ref = mo.decode_seq(f(dec.q(b)), f(dec.q_idx(b)), f(dec.k_idx_cache(b))[:L], f(dec.k_cache(b))[:L],
                            f(dec.v_cache(b))[:L], L, block_size=bk, topk=topk)
        assert np.array_equal(sel[b].cpu().numpy(), ref["sel"]), f"seq {b}"
        compare_out(out[b], ref["out"], f"decode B_k={bk} seq{b}")
        compare_lse(lse[b], ref["lse"], f"decode B_k={bk} seq{b}")


def test_block_size_64_matches_128_when_pairs_merge():
    """Consistency across block sizes: with k = all blocks (no choice left),
    B_k = 64 and 128 both attend to every earlier key, so outputs agree."""
    n, G = 1024, 1
    inp128 = syn.PrefillInputs(n, dims(G, 8, 128), 13, "tiny")
    q, k, v, qi, ki = prefill_device_inputs(inp128)
    o128, _, l128 = msa.prefill(q, k, v, qi, ki, topk=8, block_size=128, want_lse=True)
    o64, _, l64 = msa.prefill(q, k, v, qi, ki, topk=16, block_size=64, want_lse=True)
    torch.cuda.synchronize()
    assert (o128.float() - o64.float()).abs().max().item() <= 2e-2
    assert (l128 - l64).abs().max().item() <= 4e-3
