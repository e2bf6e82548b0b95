"""Pins of the index-projection oracle (oracle/proj_oracle.py) to things other
than itself: brute force on tiny inputs, selector weights whose outputs are
known slices of the input (a transposed or mis-indexed operand fails them), the
bilinear form the index score becomes, and bf16 rounding at known ties. CPU
only."""
import numpy as np
import pytest

from oracle import proj_oracle as po


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    n, dm, G, di = 3, 5, 2, 3
    x = rng.normal(size=(n, dm))
    wq = rng.normal(size=(G, di, dm))
    wk = rng.normal(size=(di, dm))
    q, k = po.index_project(x, wq, wk)
    for t in range(n):
        for g in range(G):
            for c in range(di):
                s = 0.0
                for m in range(dm):
                    s += wq[g][c][m] * x[t][m]
                assert abs(q[t, g, c] - s) < 1e-12
        for c in range(di):
            s = 0.0
            for m in range(dm):
                s += wk[c][m] * x[t][m]
            assert abs(k[t, c] - s) < 1e-12


def test_selector_weights_return_input_slices():
    """W_qi[g] picks input dims [g*d_idx, (g+1)*d_idx) and W_ki the last d_idx
    dims, reversed; the outputs are those slices of x exactly."""
    rng = np.random.default_rng(1)
    n, G, di = 7, 3, 4
    dm = (G + 1) * di + 2
    x = rng.normal(size=(n, dm))
    wq = np.zeros((G, di, dm))
    for g in range(G):
        for c in range(di):
            wq[g, c, g * di + c] = 1.0
    wk = np.zeros((di, dm))
    for c in range(di):
        wk[c, dm - 1 - c] = 1.0
    q, k = po.index_project(x, wq, wk)
    for g in range(G):
        assert np.array_equal(q[:, g, :], x[:, g * di:(g + 1) * di])
    assert np.array_equal(k, x[:, ::-1][:, :di])


def test_index_score_is_a_bilinear_form():
    """q_idx[i,g] . k_idx[j] = x_i^T (W_qi[g]^T W_ki) x_j: the projected score
    equals the bilinear form taken in the other association order."""
    rng = np.random.default_rng(2)
    n, dm, G, di = 6, 9, 2, 4
    x = rng.normal(size=(n, dm))
    wq = rng.normal(size=(G, di, dm))
    wk = rng.normal(size=(di, dm))
    q, k = po.index_project(x, wq, wk)
    for g in range(G):
        M = wq[g].T @ wk                       # d_model x d_model
        want = x @ M @ x.T                     # [i, j]
        got = q[:, g, :] @ k.T
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("v,want", [
    (1.0 + 2.0 ** -8, 1.0),                    # tie: mantissa 0 is even
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),    # tie between odd 1 and even 2
    (257.0, 256.0), (259.0, 260.0), (-259.0, -260.0),
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0 + 2.0 ** -7),   # just above the tie
    (255.0, 255.0), (3.0, 3.0),
])
def test_round_bf16_ties_to_even(v, want):
    assert po.round_bf16(np.array([v]))[0] == want


def test_fp32_error_bound_covers_sequential_fp32_sums():
    rng = np.random.default_rng(3)
    n, dm, G, di = 4, 4096, 1, 8
    x = rng.normal(size=(n, dm)).astype(np.float32).astype(np.float64)
    wq = rng.normal(size=(G, di, dm)).astype(np.float32).astype(np.float64)
    wk = rng.normal(size=(di, dm)).astype(np.float32).astype(np.float64)
    q, k = po.index_project(x, wq, wk)
    bq, bk = po.fp32_error_bound(x, wq, wk)
    # a left-to-right fp32 accumulation, the worst ordering for error growth
    for t in range(n):
        for c in range(di):
            acc = np.float32(0.0)
            prods = (x[t] * wk[c]).astype(np.float32)
            for p in prods:
                acc = np.float32(acc + p)
            assert abs(float(acc) - k[t, c]) <= bk[t, c]
