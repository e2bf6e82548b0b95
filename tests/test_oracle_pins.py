"""Pins of the float64 oracle against facts fixed outside the oracle itself:
a hand-derived worked case, textbook dense attention, torch's SDPA, brute-force
subset enumeration, closed forms of the planted recipe, special cases and
metamorphic relations. CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import msa_synth as syn
from oracle import dense_ref, msa_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers that are NOT the oracle: brute force by subset enumeration
# ---------------------------------------------------------------------------

def brute_force_top(scores, count):
    """The unique subset C of size `count` such that every member beats every
    non-member (higher score, or equal score and lower index). Found by
    enumerating all subsets; returns it sorted."""
    n = len(scores)
    if count >= n:
        return list(range(n))
    found = []
    for subset in itertools.combinations(range(n), count):
        inside = set(subset)
        ok = all((scores[a] > scores[b]) or (scores[a] == scores[b] and a < b)
                 for a in inside for b in range(n) if b not in inside)
        if ok:
            found.append(sorted(subset))
    assert len(found) == 1, "the tie-break must make the selection unique"
    return found[0]


def sdpa_masked(q, k, v, mask_gnn, scale=None):
    """torch SDPA in float64 on CPU with heads expanded to the query heads."""
    N, Hq, d = q.shape
    G = k.shape[1]
    hpg = Hq // G
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]            # [1, Hq, N, d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hpg, 0)[None].contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hpg, 0)[None].contiguous()
    causal = torch.tril(torch.ones(N, N, dtype=torch.bool))
    m = torch.from_numpy(mask_gnn).repeat_interleave(hpg, 0) & causal   # [Hq, N, N]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m[None], scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def make_case(n, G, hpg, d, di, bk, seed, recipe="tiny", **kw):
    dims = syn.Dims(num_q_heads=G * hpg, num_kv_heads=G, head_dim=d, index_dim=di, block_size=bk, topk=4)
    inp = syn.PrefillInputs(n, dims, seed, recipe, **kw)
    f = mo.to_f64
    return inp, f(inp.q()), f(inp.k()), f(inp.v()), f(inp.q_idx()), f(inp.k_idx())


def run_oracle(q, k, v, qi, ki, bk, topk, rows=None, **kw):
    n = q.shape[0]
    rows = list(range(n)) if rows is None else list(rows)
    return mo.prefill_rows(rows, q[rows], qi[rows], ki, k, v, block_size=bk, topk=topk, **kw)


# ---------------------------------------------------------------------------
# 1. hand-derived worked case
# ---------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "worked_selection.json")) as f:
        return json.load(f)


def test_golden_selection_and_pooling():
    gd = _golden()
    ki = np.array(gd["k_idx"], dtype=np.float64)
    qi = np.array(gd["q_idx"], dtype=np.float64)[:, None, :]
    n, d = ki.shape[0], 8
    q = np.zeros((n, 1, d))
    k = np.eye(d)[:n, None, :]
    v = np.eye(d)[:n, None, :]
    res = run_oracle(q, k, v, qi, ki, gd["block_size"], gd["topk"], want_scores=True)
    assert res["sel"][:, 0, :].tolist() == gd["expected_sel"]
    for i_str, exp in gd["expected_pooled_scores"].items():
        i = int(i_str)
        assert res["scores"][i][0].tolist() == exp
    # uniform weights: out = indicator(T) / |T|, lse = ln |T|
    for i, T in enumerate(gd["expected_token_sets"]):
        want = np.zeros(d)
        want[T] = 1.0 / len(T)
        np.testing.assert_allclose(res["out"][i, 0], want, rtol=0, atol=1e-15)
        assert abs(res["lse"][i, 0] - math.log(len(T))) < 1e-14


def test_golden_weighted_scale():
    gd = _golden()
    ki = np.array(gd["k_idx"], dtype=np.float64)
    qi = np.array(gd["q_idx"], dtype=np.float64)[:, None, :]
    n, d = ki.shape[0], 8
    q = np.zeros((n, 1, d))
    q[:, 0, 0] = math.sqrt(8.0)
    k = np.zeros((n, 1, d))
    k[:, 0, 0] = np.log(np.arange(n) + 1.0)
    v = np.eye(d)[:n, None, :]
    res = run_oracle(q, k, v, qi, ki, gd["block_size"], gd["topk"])
    for i, T in enumerate(gd["expected_token_sets"]):
        tot = gd["case_weighted"]["expected_weight_sums"][i]
        assert tot == sum(j + 1 for j in T)
        want = np.zeros(d)
        for j in T:
            want[j] = (j + 1) / tot
        np.testing.assert_allclose(res["out"][i, 0], want, rtol=0, atol=1e-13)
        assert abs(res["lse"][i, 0] - math.log(tot)) < 1e-13


# ---------------------------------------------------------------------------
# 2. k covering every block == dense causal GQA attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1])
def test_dense_equivalence(seed):
    n, G, hpg, d, di, bk = 256, 2, 3, 16, 8, 32
    nb = n // bk
    _, q, k, v, qi, ki = make_case(n, G, hpg, d, di, bk, seed)
    res = run_oracle(q, k, v, qi, ki, bk, topk=nb)
    out_ref, lse_ref = dense_ref.masked_gqa_attention(q, k, v)
    np.testing.assert_allclose(res["out"], out_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["lse"], lse_ref, rtol=0, atol=1e-12)
    # torch SDPA (float64, CPU), plain causal GQA
    o_sdpa = sdpa_masked(q, k, v, np.ones((G, n, n), dtype=bool))
    np.testing.assert_allclose(res["out"], o_sdpa, rtol=0, atol=1e-12)
    # every row selected every block up to its own
    for i in range(n):
        for g in range(G):
            s = res["sel"][i, g]
            assert s[s >= 0].tolist() == list(range(i // bk + 1))


# ---------------------------------------------------------------------------
# 3. selection == brute-force subset enumeration on tiny tied inputs
# ---------------------------------------------------------------------------

def test_selection_bruteforce():
    rng = np.random.default_rng(123)
    checked = 0
    for _ in range(400):
        b_loc = int(rng.integers(0, 10))
        k = int(rng.integers(1, 7))
        S = rng.integers(-1, 2, size=b_loc).astype(np.float64)  # many ties
        got = mo.select_blocks(S, b_loc, k)
        want = sorted(brute_force_top(S.tolist(), min(k - 1, b_loc)) + [b_loc])
        assert got[got >= 0].tolist() == want
        assert (got[len(want):] == -1).all()
        checked += 1
    assert checked == 400


def test_scores_bruteforce_tiny():
    """Pooled scores against a plain triple loop on a tiny case."""
    inp, q, k, v, qi, ki = make_case(64, 2, 2, 8, 4, 8, seed=5)
    res = run_oracle(q, k, v, qi, ki, 8, topk=3, want_scores=True)
    for i in range(64):
        S = res["scores"][i]
        b_loc = i // 8
        assert S.shape == (2, b_loc)
        for g in range(2):
            for b in range(b_loc):
                best = -np.inf
                for j in range(b * 8, b * 8 + 8):
                    best = max(best, sum(qi[i, g, c] * ki[j, c] for c in range(4)))
                assert S[g, b] == best


# ---------------------------------------------------------------------------
# 4. invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("recipe", ["tiny", "planted"])
def test_invariants(recipe):
    n, bk, topk = 2048, 128, 4
    G = 1 if recipe == "tiny" else 4
    dims = syn.Dims(num_q_heads=16 * G, num_kv_heads=G, head_dim=128, index_dim=64, block_size=bk, topk=topk)
    inp = syn.PrefillInputs(n, dims, 3, recipe, n_planted=2)
    rows = syn.stratified_rows(n, 96, bk, 3, topk)
    f = mo.to_f64
    ki = f(inp.k_idx())
    qi = f(inp.q_idx(rows))
    # attention outputs are not needed here: zero-size heads keep it fast
    q = np.zeros((len(rows), G, 1))
    kv = np.zeros((n, G, 1))
    res = mo.prefill_rows(rows, q, qi, ki, kv, kv, block_size=bk, topk=topk)
    for r, i in enumerate(rows):
        b_loc = i // bk
        for g in range(G):
            s = res["sel"][r, g]
            valid = s[s >= 0]
            assert b_loc in valid
            assert valid.size == min(topk, b_loc + 1)
            assert (np.diff(valid) > 0).all()
            assert valid.min() >= 0 and valid.max() <= b_loc
            assert (s[valid.size:] == -1).all()


# ---------------------------------------------------------------------------
# 5. planted recipe: closed form of the needle margin
# ---------------------------------------------------------------------------

def test_planted_recall_and_margin():
    n, bk, topk = 8192, 128, 16
    dims = syn.Dims(block_size=bk, topk=topk)
    inp = syn.PrefillInputs(n, dims, 11, "planted", n_planted=8)
    rows = syn.stratified_rows(n, 64, bk, 11, topk)
    f = mo.to_f64
    ki = f(inp.k_idx())
    qi = f(inp.q_idx(rows))
    q = np.zeros((len(rows), 4, 1))
    kv = np.zeros((n, 4, 1))
    res = mo.prefill_rows(rows, q, qi, ki, kv, kv, block_size=bk, topk=topk, want_scores=True)
    for r, i in enumerate(rows):
        b_loc = i // bk
        for g in range(4):
            S = res["scores"][r][g]
            for b in range(b_loc):
                if b in inp.planted[g]:
                    assert S[b] == 144.0          # 3 * 3 * 16
                else:
                    assert S[b] <= 96.0           # 3 * 16 + 48
            for p in inp.planted[g]:
                if p < b_loc:
                    assert p in res["sel"][r, g]


def test_skewed_hot_blocks_selected():
    n, bk, topk = 8192, 128, 16
    dims = syn.Dims(block_size=bk, topk=topk)
    inp = syn.PrefillInputs(n, dims, 2, "skewed", n_planted=4, n_hot=4)
    assert inp.hot[0] == 0 and len(inp.hot) == 4
    rows = [n - 1, n // 2, 3000]
    f = mo.to_f64
    res = mo.prefill_rows(rows, np.zeros((3, 4, 1)), f(inp.q_idx(rows)), f(inp.k_idx()),
                          np.zeros((n, 4, 1)), np.zeros((n, 4, 1)), block_size=bk, topk=topk,
                          want_scores=True)
    for r, i in enumerate(rows):
        for g in range(4):
            for b in inp.hot:
                if b < i // bk:
                    assert b in res["sel"][r, g]
                    assert res["scores"][r][g][b] >= 144.0


# ---------------------------------------------------------------------------
# 6. metamorphic relations
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m", [-1, 1, 3])
def test_power_of_two_scaling_keeps_selection(m):
    n, bk = 1024, 64
    _, q, k, v, qi, ki = make_case(n, 2, 2, 8, 8, bk, seed=9)
    a = run_oracle(q, k, v, qi, ki, bk, topk=4)
    b = run_oracle(q, k, v, qi * (2.0 ** m), ki, bk, topk=4)
    assert (a["sel"] == b["sel"]).all()
    np.testing.assert_array_equal(a["out"], b["out"])


def test_group_permutation_permutes_selection():
    n, bk, G, hpg = 512, 32, 3, 2
    _, q, k, v, qi, ki = make_case(n, G, hpg, 8, 6, bk, seed=4)
    perm = [2, 0, 1]
    head_perm = [g * hpg + t for g in perm for t in range(hpg)]
    a = run_oracle(q, k, v, qi, ki, bk, topk=4)
    b = run_oracle(q[:, head_perm], k[:, perm], v[:, perm], qi[:, perm], ki, bk, topk=4)
    assert (b["sel"] == a["sel"][:, perm]).all()
    np.testing.assert_allclose(b["out"], a["out"][:, head_perm], rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# 7. special cases that reduce to textbook attention
# ---------------------------------------------------------------------------

def test_k1_is_block_local_causal():
    n, bk, G = 256, 32, 2
    _, q, k, v, qi, ki = make_case(n, G, 2, 16, 8, bk, seed=6)
    res = run_oracle(q, k, v, qi, ki, bk, topk=1)
    blk = np.arange(n) // bk
    local = (blk[:, None] == blk[None, :])
    out_ref, lse_ref = dense_ref.masked_gqa_attention(q, k, v, mask=np.stack([local] * G))
    np.testing.assert_allclose(res["out"], out_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["lse"], lse_ref, rtol=0, atol=1e-12)


def test_block_size_one_is_token_topk():
    """B_k = 1: the selection is the query token plus its top k-1 earlier tokens
    by raw index score (brute-forced), attention over exactly those tokens."""
    n, G, topk = 40, 2, 4
    _, q, k, v, qi, ki = make_case(n, G, 2, 8, 4, 1, seed=8)
    res = run_oracle(q, k, v, qi, ki, 1, topk=topk)
    mask = np.zeros((G, n, n), dtype=bool)
    for i in range(n):
        for g in range(G):
            raw = [float(qi[i, g] @ ki[j]) for j in range(i)]
            chosen = brute_force_top(raw, min(topk - 1, i)) + [i]
            s = res["sel"][i, g]
            assert s[s >= 0].tolist() == sorted(chosen)
            mask[g, i, chosen] = True
    out_ref, _ = dense_ref.masked_gqa_attention(q, k, v, mask=mask)
    np.testing.assert_allclose(res["out"], out_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 2])
def test_general_case_equals_masked_sdpa(seed):
    n, bk, G, hpg, topk = 512, 32, 2, 4, 4
    _, q, k, v, qi, ki = make_case(n, G, hpg, 16, 8, bk, seed)
    res = run_oracle(q, k, v, qi, ki, bk, topk)
    mask = dense_ref.block_mask_from_selection(res["sel"], n, bk)
    o_sdpa = sdpa_masked(q, k, v, mask)
    np.testing.assert_allclose(res["out"], o_sdpa, rtol=0, atol=1e-12)
    out_ref, lse_ref = dense_ref.masked_gqa_attention(q, k, v, mask=mask)
    np.testing.assert_allclose(res["out"], out_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["lse"], lse_ref, rtol=0, atol=1e-12)


def test_decode_equals_last_prefill_row():
    n, bk = 640, 64
    _, q, k, v, qi, ki = make_case(n, 2, 2, 8, 8, bk, seed=12)
    for L in (1, 63, 64, 65, 640):
        a = mo.decode_seq(q[L - 1], qi[L - 1], ki, k, v, L, block_size=bk, topk=3)
        b = run_oracle(q, k, v, qi, ki, bk, 3, rows=[L - 1])
        assert (a["sel"] == b["sel"][0]).all()
        np.testing.assert_array_equal(a["out"], b["out"][0])


# ---------------------------------------------------------------------------
# 8. the two-phase combine identity used by the GPU design
# ---------------------------------------------------------------------------

def test_lse_merge_identity():
    """Softmax over a union of blocks == log-sum-exp merge of per-block partials
    (m, l, o): o = sum_u l_u e^{m_u - M} o_u / sum_u l_u e^{m_u - M}."""
    rng = np.random.default_rng(0)
    d, H = 16, 3
    blocks = [rng.normal(size=(n, d)) * 3 for n in (5, 17, 1, 9)]
    vals = [rng.normal(size=(b.shape[0], d)) for b in blocks]
    q = rng.normal(size=(H, d))
    direct_o, direct_lse = mo.attend(q, np.concatenate(blocks), np.concatenate(vals), 0.7)
    ms, ls, os_ = [], [], []
    for kb, vb in zip(blocks, vals):
        z = 0.7 * q @ kb.T
        m = z.max(axis=1)
        p = np.exp(z - m[:, None])
        ms.append(m)
        ls.append(p.sum(axis=1))
        os_.append((p @ vb) / p.sum(axis=1)[:, None])   # normalised partial
    M = np.max(ms, axis=0)
    w = [l * np.exp(m - M) for m, l in zip(ms, ls)]
    tot = np.sum(w, axis=0)
    merged = sum(wu[:, None] * ou for wu, ou in zip(w, os_)) / tot[:, None]
    np.testing.assert_allclose(merged, direct_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(M + np.log(tot), direct_lse, rtol=0, atol=1e-13)
