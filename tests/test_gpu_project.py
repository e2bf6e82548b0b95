"""GPU parity of the Index Branch projections (msa_index_project,
msa_index_project_decode) against the float64 oracle (oracle/proj_oracle.py).

Bar: with small-integer inputs every product and sum is exact in fp32, so the
outputs equal the oracle's result rounded to bf16 bit for bit (both round to
nearest even). With real-valued inputs each output is within
2^-8 |ref| (bf16 output rounding) + d_model 2^-24 sum_k |x_k w_k| (fp32
accumulation, any order) of the float64 result. Both the single-pass path
(many tokens) and the split-d_model path with its ordered reduce (few tokens,
as in decode) are covered, as is the decode key append.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_07_amd as msa
import msa_synth as syn
from oracle import msa_oracle as mo
from oracle import proj_oracle as po
from tests._parity import log, timed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    msa.load()
    yield
    torch.cuda.empty_cache()


def int_inputs(seed, n, dm, G, lo=-3, hi=3):
    g = torch.Generator().manual_seed(seed)
    x = torch.randint(lo, hi + 1, (n, dm), generator=g).to(torch.bfloat16)
    wq = torch.randint(lo, hi + 1, (G, 64, dm), generator=g).to(torch.bfloat16)
    wk = torch.randint(lo, hi + 1, (64, dm), generator=g).to(torch.bfloat16)
    return x, wq, wk


def normal_inputs(seed, n, dm, G):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((n, dm), generator=g).to(torch.bfloat16)
    s = dm ** -0.5
    wq = (torch.randn((G, 64, dm), generator=g) * s).to(torch.bfloat16)
    wk = (torch.randn((64, dm), generator=g) * s).to(torch.bfloat16)
    return x, wq, wk


def f64(t):
    return t.to(torch.float64).cpu().numpy()


def run(x, wq, wk):
    q, k = msa.index_project(x.cuda(), wq.cuda(), wk.cuda())
    torch.cuda.synchronize()
    return f64(q), f64(k)


# few tokens (one column unit per workgroup, with and without a d_model split)
# and many (all columns, or two parts of them, per workgroup), every G
@pytest.mark.parametrize("G,n,dm", [(4, 1, 64), (4, 129, 320), (1, 1000, 256), (8, 127, 1024), (5, 300, 128),
                                    (6, 64, 8192), (4, 33000, 128), (2, 40000, 192), (1, 9000, 64),
                                    (3, 8200, 128), (7, 8200, 128), (8, 8200, 64), (5, 8300, 64), (6, 8200, 64),
                                    # many tokens and d_model a multiple of 256: the warp-specialised
                                    # kernel (all units, or two parts with the last unit clamped)
                                    (4, 8300, 256), (1, 9000, 512), (8, 8200, 256), (6, 16500, 256),
                                    (3, 33000, 256), (4, 8192, 768)])
def test_integer_inputs_bit_exact(G, n, dm):
    x, wq, wk = int_inputs(G * 1000 + n, n, dm, G)
    log(f"case project int G={G} n={n} d_model={dm}")
    gq, gk = run(x, wq, wk)
    q, k = po.index_project(f64(x), f64(wq), f64(wk))
    assert np.abs(q).max() < 2 ** 24 and np.abs(k).max() < 2 ** 24
    rq, rk = po.round_bf16(q), po.round_bf16(k)
    bad = np.argwhere(gq != rq)
    assert bad.size == 0, f"q_idx differs at {bad[:5].tolist()}"
    bad = np.argwhere(gk != rk)
    assert bad.size == 0, f"k_idx differs at {bad[:5].tolist()}"


@pytest.mark.parametrize("G,n,dm", [(4, 64, 8192), (4, 33024, 2048), (3, 500, 6144), (8, 8200, 1024), (1, 16500, 512)])
def test_normal_inputs_within_bound(G, n, dm):
    x, wq, wk = normal_inputs(7 + n, n, dm, G)
    log(f"case project normal G={G} n={n} d_model={dm}")
    with timed("gpu"):
        gq, gk = run(x, wq, wk)
    with timed("oracle"):
        X, WQ, WK = f64(x), f64(wq), f64(wk)
        q, k = po.index_project(X, WQ, WK)
        bq, bk = po.fp32_error_bound(X, WQ, WK)
    for got, ref, b, name in ((gq, q, bq, "q_idx"), (gk, k, bk, "k_idx")):
        err = np.abs(got - ref)
        lim = 2.0 ** -8 * np.abs(ref) + b
        worst = float((err / np.maximum(lim, 1e-30)).max())
        log(f"  {name}: max err {err.max():.3e}, worst err/bound {worst:.3f}")
        assert (err <= lim).all(), f"{name}: error above bound at {np.argwhere(err > lim)[:5].tolist()}"


def test_split_and_single_pass_agree_to_the_bound():
    """The same rows through both paths: 64 tokens (split d_model, ordered
    reduce) and the same 64 tokens inside a 40000-token call (one pass)."""
    G, dm = 4, 4096
    x, wq, wk = normal_inputs(99, 40000, dm, G)
    xs = x[:64].contiguous()
    q1, k1 = run(xs, wq, wk)
    q2, k2 = run(x, wq, wk)
    X, WQ, WK = f64(xs), f64(wq), f64(wk)
    q, k = po.index_project(X, WQ, WK)
    bq, bk = po.fp32_error_bound(X, WQ, WK)
    for a, b_, ref, bnd in ((q1, q2[:64], q, bq), (k1, k2[:64], k, bk)):
        assert (np.abs(a - b_) <= 2 * (2.0 ** -8 * np.abs(ref) + bnd)).all()


def test_decode_appends_key_at_context_end():
    G, B, max_ctx, dm = 4, 5, 300, 1024
    lens = [1, 2, 150, 299, 300]
    x, wq, wk = int_inputs(5, B, dm, G, -2, 2)
    cache = torch.full((B, max_ctx, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qi = msa.index_project_decode(x.cuda(), wq.cuda(), wk.cuda(), cache, lt)
    torch.cuda.synchronize()
    q, k = po.index_project(f64(x), f64(wq), f64(wk))
    assert np.array_equal(f64(qi), po.round_bf16(q))
    c = f64(cache)
    for b, L in enumerate(lens):
        assert np.array_equal(c[b, L - 1], po.round_bf16(k[b])), f"seq {b}"
        rest = np.delete(c[b], L - 1, axis=0)
        assert (rest == 7.0).all(), f"seq {b}: a row other than {L - 1} changed"


def test_decode_append_many_sequences():
    """A decode step of 8200 sequences (enough for the many-token kernel, with
    d_model a multiple of 256): each key lands in its own sequence's row
    ctx_lens[b] - 1 and no other cache row changes."""
    G, B, max_ctx, dm = 4, 8200, 3, 256
    x, wq, wk = int_inputs(17, B, dm, G, -2, 2)
    g = torch.Generator().manual_seed(3)
    lt_h = torch.randint(1, max_ctx + 1, (B,), generator=g, dtype=torch.int32)
    cache = torch.full((B, max_ctx, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    log(f"case project decode B={B} d_model={dm}")
    qi = msa.index_project_decode(x.cuda(), wq.cuda(), wk.cuda(), cache, lt_h.cuda())
    torch.cuda.synchronize()
    q, k = po.index_project(f64(x), f64(wq), f64(wk))
    assert np.array_equal(f64(qi), po.round_bf16(q))
    c = f64(cache)
    lens = lt_h.numpy().astype(np.int64)
    rows = np.arange(B)
    assert np.array_equal(c[rows, lens - 1], po.round_bf16(k))
    untouched = np.ones((B, max_ctx), dtype=bool)
    untouched[rows, lens - 1] = False
    assert (c[untouched] == 7.0).all(), "a row other than ctx_lens - 1 changed"


def test_projection_feeds_prefill_selection_exactly():
    """Hidden states -> projections -> prefill: with {-1, 0, 1} inputs and
    d_model 64 the projected heads are small integers (exact in bf16), so the
    block selection must equal the oracle's on the oracle's projections."""
    n, G, topk, dm = 3000, 4, 16, 64
    x, wq, wk = int_inputs(11, n, dm, G, -1, 1)
    qi, ki = msa.index_project(x.cuda(), wq.cuda(), wk.cuda())
    dims = syn.Dims(num_q_heads=16 * G, num_kv_heads=G, head_dim=128, index_dim=64, block_size=128, topk=topk)
    inp = syn.PrefillInputs(n, dims, 3, "tiny")
    q, k, v = (t(device="cuda")[None].contiguous() for t in (inp.q, inp.k, inp.v))
    out, sel, lse = msa.prefill(q, k, v, qi[None].contiguous(), ki[None].contiguous(), topk=topk, want_sel=True,
                                want_lse=True)
    torch.cuda.synchronize()
    Q, K = po.index_project(f64(x), f64(wq), f64(wk))
    rows = syn.stratified_rows(n, 384, 128, 5, topk)
    ref = mo.prefill_rows(rows, mo.to_f64(inp.q(rows)), Q[rows], K, mo.to_f64(inp.k()), mo.to_f64(inp.v()),
                          block_size=128, topk=topk)
    rt = torch.as_tensor(rows, device="cuda")
    assert np.array_equal(sel[0][:, rt].permute(1, 0, 2).cpu().numpy(), ref["sel"])
    err = np.abs(out[0][rt].double().cpu().numpy() - ref["out"]).max()
    assert err <= 2e-2


def test_split_reduce_is_deterministic():
    """The split plan sums its partials in a fixed order: two calls agree bit
    for bit."""
    x, wq, wk = normal_inputs(3, 64, 8192, 4)
    xc, wqc, wkc = x.cuda(), wq.cuda(), wk.cuda()
    a = [t.clone() for t in msa.index_project(xc, wqc, wkc)]
    b = msa.index_project(xc, wqc, wkc)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))
