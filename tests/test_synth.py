"""The seeded generator: determinism, row addressability and recipe shape."""
import numpy as np
import torch

import msa_synth as syn


def test_hash_reference_values():
    # fmix32 of small integers, computed with plain Python ints
    idx = torch.arange(4, dtype=torch.int64)
    h = syn.hash32(0, 1, idx)
    k1, k2 = syn._keys(0, 1)
    want = [syn._fmix32_int(syn._fmix32_int(i ^ k1) ^ 0 ^ k2) for i in range(4)]
    assert h.tolist() == want


def test_mul32_exact():
    rng = np.random.default_rng(0)
    x = rng.integers(0, 2 ** 32, size=1000, dtype=np.uint64)
    c = 0xC2B2AE35
    got = syn._mul32(torch.from_numpy(x.astype(np.int64)), c).numpy().astype(np.uint64)
    want = np.array([(int(a) * c) & 0xFFFFFFFF for a in x], dtype=np.uint64)
    assert (got == want).all()


def test_rows_regenerate_identically():
    dims = syn.Dims(num_q_heads=8, num_kv_heads=2, head_dim=16, index_dim=8, block_size=16, topk=4)
    inp = syn.PrefillInputs(300, dims, 5, "planted", n_planted=3)
    rows = [0, 7, 150, 299]
    for fn in (inp.q, inp.k, inp.v, inp.q_idx, inp.k_idx):
        full = fn()
        part = fn(rows)
        assert torch.equal(full[rows], part)


def test_normal_moments():
    x = syn.normal_bf16(1, 2, torch.arange(200000, dtype=torch.int64)).float()
    assert abs(x.mean().item()) < 0.01
    assert abs(x.std().item() - 1.0) < 0.01
    assert x.abs().max().item() <= 6.0


def test_index_values_are_small_integers():
    dims = syn.Dims()
    inp = syn.PrefillInputs(4096, dims, 0, "planted")
    ki = inp.k_idx().float()
    qi = inp.q_idx().float()
    assert set(torch.unique(ki).tolist()) <= {-1.0, 0.0, 1.0, 3.0}
    assert set(torch.unique(qi).tolist()) <= {-1.0, 0.0, 1.0, 3.0}
    assert (qi[:, 2, 32:48] == 3).all()
    tiny = syn.PrefillInputs(2048, syn.Dims(num_q_heads=16, num_kv_heads=1, topk=4), 0, "tiny")
    assert set(torch.unique(tiny.k_idx().float()).tolist()) <= set(float(v) for v in range(-3, 4))


def test_decode_inputs_follow_prefill_recipe():
    dims = syn.Dims()
    dec = syn.DecodeInputs(2, 2048, dims, 3, ctx_lens=[2048, 1000])
    assert torch.equal(dec.q_idx(1), dec.seqs[1].q_idx([999])[0])
    assert dec.seqs[0].seed == 3000 and dec.seqs[1].seed == 3001
