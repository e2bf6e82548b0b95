"""GPU parity of the Index Branch KL-alignment backward (msa_index_kl_backward)
against the float64 oracle (oracle/kl_oracle.py).

The GPU teacher uses the forward pass's lse (as a training step would), which
carries the forward's bf16 rounding of P: |d lse| <= 4e-3, i.e. P_main off by
a relative 4e-3 at most, and the gradients, sums of gs = P_idx - P_main
terms, by as much relative to P_main. The bars follow from that: gradients
within relative L2 5e-3 and max-abs 5e-3 * max|reference|; the loss, whose
log terms amplify that error, within 1e-2 * (1 + |loss|).
Selections are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_07_amd as msa
import msa_synth as syn
from oracle import kl_oracle as ko
from oracle import msa_oracle as mo
from tests._parity import log, prefill_device_inputs, timed

pytestmark = pytest.mark.gpu

REL_L2 = 5e-3
MAX_REL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    msa.load()
    yield
    torch.cuda.empty_cache()


def dims(G, topk):
    return syn.Dims(num_q_heads=16 * G, num_kv_heads=G, head_dim=128, index_dim=64, block_size=128, topk=topk)


def run_gpu(inp, topk):
    q, k, v, qi, ki = prefill_device_inputs(inp)
    _, sel, lse = msa.prefill(q, k, v, qi, ki, topk=topk, want_sel=True, want_lse=True)
    loss, dq, dk = msa.index_kl_backward(q[0], k[0], qi[0], ki[0], sel[0].contiguous(), lse[0].contiguous(),
                                         topk=topk)
    torch.cuda.synchronize()
    return sel[0], loss, dq, dk, (q[0], k[0], qi[0], ki[0])


def compare_grad(got, want, what):
    g = got.detach().cpu().double().numpy()
    diff = g - want
    scale = max(np.abs(want).max(), 1e-30)
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-30))
    mx = float(np.abs(diff).max())
    log(f"  {what}: max_abs={mx:.3e} (ref max {scale:.3e}) rel_l2={rel:.3e}")
    assert rel <= REL_L2, f"{what}: rel L2 {rel}"
    assert mx <= MAX_REL * scale, f"{what}: max abs {mx}"


def compare_loss(got, want, what):
    g = got.detach().cpu().double().numpy()
    err = np.abs(g - want) / (1.0 + np.abs(want))
    log(f"  {what}: max scaled err {err.max():.3e} (loss range {want.min():.3e} .. {want.max():.3e})")
    assert err.max() <= 1e-2, f"{what}: loss err {err.max()}"


@pytest.mark.parametrize("n,G,topk,recipe", [(2048, 1, 4, "tiny"), (1500, 2, 8, "planted"), (2048, 4, 16, "planted"),
                                             (300, 1, 16, "tiny")])
def test_kl_backward_all_rows(n, G, topk, recipe):
    inp = syn.PrefillInputs(n, dims(G, topk), 11, recipe, n_planted=3)
    log(f"case kl N={n} G={G} k={topk} recipe={recipe}")
    with timed("gpu"):
        sel, loss, dq, dk, _ = run_gpu(inp, topk)
    with timed("oracle"):
        ref = ko.index_kl(mo.to_f64(inp.q()), mo.to_f64(inp.k()), mo.to_f64(inp.q_idx()), mo.to_f64(inp.k_idx()),
                          block_size=128, topk=topk)
    assert np.array_equal(sel.permute(1, 0, 2).cpu().numpy(), ref["sel"]), "selection"
    compare_loss(loss, ref["loss"], "loss")
    compare_grad(dq, ref["dq_idx"], "dq_idx")
    compare_grad(dk, ref["dk_idx"], "dk_idx")


@pytest.mark.timeout(900)
def test_kl_backward_32k_sampled_and_identities():
    n, G, topk = 32768, 4, 16
    inp = syn.PrefillInputs(n, dims(G, topk), 0, "planted", n_planted=8)
    log(f"case kl 32K")
    with timed("gpu"):
        sel, loss, dq, dk, (q, k, qi, ki) = run_gpu(inp, topk)
    # identities at full size: sum_j dk[j] = 0; sum q_idx . dq = sum k_idx . dk
    dk64 = dk.double()
    col = dk64.sum(dim=0).abs().max().item()
    scale = dk64.abs().sum(dim=0).max().item()
    lhs = (qi.double() * dq.double()).sum().item()
    rhs = (ki.double() * dk64).sum().item()
    log(f"  identities: |sum dk| {col:.3e} of {scale:.3e}; q.dq {lhs:.6e} vs k.dk {rhs:.6e}")
    assert col <= 1e-4 * scale
    assert abs(lhs - rhs) <= 1e-4 * max(abs(lhs), (qi.double().abs() * dq.double().abs()).sum().item())
    rows = syn.stratified_rows(n, 768, 128, 1, topk, extra=sorted({b for g in inp.planted.values() for b in g}))
    with timed("oracle"):
        ref = ko.index_kl_rows(rows, mo.to_f64(inp.q(rows)), mo.to_f64(inp.q_idx(rows)), mo.to_f64(k.cpu()),
                               mo.to_f64(ki.cpu()), block_size=128, topk=topk)
    rt = torch.as_tensor(rows, device="cuda")
    compare_loss(loss[:, rt].T, ref["loss"], "loss (sampled)")
    compare_grad(dq[rt], ref["dq_idx"], "dq_idx (sampled)")


def test_kl_backward_deterministic():
    """Every sum is taken in a fixed order (no atomics): two calls agree bit for bit."""
    inp = syn.PrefillInputs(3000, dims(4, 16), 12, "planted", n_planted=3)
    q, k, v, qi, ki = prefill_device_inputs(inp)
    _, sel, lse = msa.prefill(q, k, v, qi, ki, topk=16, want_sel=True, want_lse=True)
    a = msa.index_kl_backward(q[0], k[0], qi[0], ki[0], sel[0].contiguous(), lse[0].contiguous(), topk=16)
    a = [x.clone() for x in a]
    b = msa.index_kl_backward(q[0], k[0], qi[0], ki[0], sel[0].contiguous(), lse[0].contiguous(), topk=16)
    torch.cuda.synchronize()
    for x, y, name in zip(a, b, ("loss", "dq_idx", "dk_idx")):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), name
