"""Pins of the KL-alignment oracle (oracle/kl_oracle.py) to things other than
itself: finite differences of the loss, closed forms, special cases and sum
identities. CPU only."""
import math

import numpy as np
import pytest

from oracle import kl_oracle as ko


def rand_inputs(seed, N=40, G=2, hpg=2, d=8, d_idx=4):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(N, G * hpg, d)), rng.normal(size=(N, G, d)),
            rng.normal(size=(N, G, d_idx)), rng.normal(size=(N, d_idx)))


def total_loss(q, k, qi, ki, sel, bk, topk):
    return ko.index_kl(q, k, qi, ki, block_size=bk, topk=topk, sel=sel)["loss"].sum()


@pytest.mark.parametrize("seed", [0, 1])
def test_gradients_match_finite_differences(seed):
    """Central differences of the summed loss with the selection held fixed
    (top-k is not differentiable; the loss lives on the selected support)."""
    bk, topk = 4, 3
    q, k, qi, ki = rand_inputs(seed)
    ref = ko.index_kl(q, k, qi, ki, block_size=bk, topk=topk)
    sel = ref["sel"]
    rng = np.random.default_rng(100 + seed)
    h = 1e-6
    for _ in range(12):
        i, g, c = rng.integers(qi.shape[0]), rng.integers(qi.shape[1]), rng.integers(qi.shape[2])
        qp, qm = qi.copy(), qi.copy()
        qp[i, g, c] += h
        qm[i, g, c] -= h
        fd = (total_loss(q, k, qp, ki, sel, bk, topk) - total_loss(q, k, qm, ki, sel, bk, topk)) / (2 * h)
        assert abs(fd - ref["dq_idx"][i, g, c]) <= 1e-6 * max(1.0, abs(fd)), (i, g, c, fd, ref["dq_idx"][i, g, c])
    for _ in range(12):
        j, c = rng.integers(ki.shape[0]), rng.integers(ki.shape[1])
        kp, km = ki.copy(), ki.copy()
        kp[j, c] += h
        km[j, c] -= h
        fd = (total_loss(q, k, qi, kp, sel, bk, topk) - total_loss(q, k, qi, km, sel, bk, topk)) / (2 * h)
        assert abs(fd - ref["dk_idx"][j, c]) <= 1e-6 * max(1.0, abs(fd)), (j, c, fd, ref["dk_idx"][j, c])


def test_student_equal_to_teacher_gives_zero():
    """One head per group and index projections equal to the scaled main ones:
    the two distributions coincide, so the divergence and its gradients vanish."""
    rng = np.random.default_rng(3)
    N, d = 48, 8
    q = rng.normal(size=(N, 1, d))
    k = rng.normal(size=(N, 1, d))
    scale = 1.0 / math.sqrt(d)
    res = ko.index_kl(q, k, scale * q[:, :, :], k[:, 0, :], block_size=4, topk=3)
    assert np.abs(res["loss"]).max() < 1e-12
    assert np.abs(res["dq_idx"]).max() < 1e-12
    assert np.abs(res["dk_idx"]).max() < 1e-12


def test_uniform_teacher_closed_form():
    """q = 0 makes the teacher uniform on T, so the loss is
    KL(U || P_idx) = -log|T| - mean_T log P_idx (teacher first)."""
    rng = np.random.default_rng(4)
    N, G, d, di, bk, topk = 30, 1, 4, 3, 4, 2
    q = np.zeros((N, 2, d))
    k = rng.normal(size=(N, G, d))
    qi = rng.normal(size=(N, G, di))
    ki = rng.normal(size=(N, di))
    res = ko.index_kl(q, k, qi, ki, block_size=bk, topk=topk)
    for i in (0, 5, 17, 29):
        T = np.nonzero([(j <= i) and (j // bk in res["sel"][i, 0]) for j in range(N)])[0]
        s = ki[T] @ qi[i, 0]
        logp = s - np.log(np.exp(s).sum())
        assert abs(res["loss"][0, i] - (-math.log(len(T)) - logp.mean())) < 1e-12


def test_teacher_is_mean_of_head_probabilities():
    """Support {0, 1} (B_k = 2, k = 1, row 1). Head 0 puts all weight on key 0,
    head 1 is uniform: the teacher is (3/4, 1/4); a student with logits
    (log 3, 0) matches it exactly, so the loss is 0."""
    big = 200.0
    q = np.zeros((2, 2, 2))
    k = np.zeros((2, 1, 2))
    k[0, 0] = [1.0, 0.0]
    q[1, 0] = [big, 0.0]       # head 0: logits (big, 0) -> (1, 0)
    q[1, 1] = [0.0, 0.0]       # head 1: logits (0, 0)   -> (1/2, 1/2)
    qi = np.zeros((2, 1, 1))
    qi[1, 0, 0] = math.log(3.0)
    ki = np.array([[1.0], [0.0]])
    res = ko.index_kl(q, k, qi, ki, block_size=2, topk=1, scale=1.0)
    assert abs(res["loss"][0, 1]) < 1e-12
    assert np.abs(res["dq_idx"][1]).max() < 1e-12


@pytest.mark.parametrize("seed", [5, 6])
def test_divergence_nonnegative_and_gradient_sums(seed):
    """KL >= 0; the gradient of each (row, group) w.r.t. its scores sums to 0,
    so sum_j dk_idx[j] = 0 and sum q_idx . dq_idx = sum k_idx . dk_idx."""
    q, k, qi, ki = rand_inputs(seed, N=64, G=3, hpg=2, d=8, d_idx=5)
    res = ko.index_kl(q, k, qi, ki, block_size=8, topk=3)
    assert res["loss"].min() >= -1e-12
    assert np.abs(res["dk_idx"].sum(axis=0)).max() < 1e-10
    lhs = float(np.sum(qi * res["dq_idx"]))
    rhs = float(np.sum(ki * res["dk_idx"]))
    assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(lhs))


def test_rows_entry_point_matches_whole_sequence():
    q, k, qi, ki = rand_inputs(7, N=50, G=2)
    full = ko.index_kl(q, k, qi, ki, block_size=4, topk=3)
    rows = np.array([0, 3, 4, 17, 49])
    part = ko.index_kl_rows(rows, q[rows], qi[rows], k, ki, block_size=4, topk=3)
    assert np.allclose(part["loss"], full["loss"][:, rows].T, atol=1e-14)
    assert np.allclose(part["dq_idx"], full["dq_idx"][rows], atol=1e-14)
