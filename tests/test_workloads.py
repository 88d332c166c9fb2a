"""Seeded generators: determinism, bf16 exactness, slice independence (CPU)."""
import numpy as np
import torch

import workloads as WL


def test_bf16_rounding_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 7
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0]   # exact ties both ways
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(WL.round_bf16(x), ref)


def test_slices_equal_full_tensor_and_deterministic():
    full = WL.make_inputs("C2")
    part = WL.make_inputs("C2", heads=[5, 2])
    for key in ("q", "k", "v", "g_c", "g_f"):
        np.testing.assert_array_equal(part[key][0, 0], full[key][0, 5])
        np.testing.assert_array_equal(part[key][0, 1], full[key][0, 2])
        bf = torch.from_numpy(full[key]).to(torch.bfloat16).float().numpy()
        np.testing.assert_array_equal(bf, full[key])


def test_spike_recipe():
    w = WL.get("C2")
    x = WL.make_inputs("C2", heads=[0])
    k = x["k"][0, 0].reshape(w.N, w.head_dim)
    # spiked rows have mean about 3, the others about 0
    n_spk = int((k.mean(1) > 1.5).sum())
    assert abs(n_spk - 164) <= 2


def test_lowrank_recipe_shares_structure_across_tensors():
    x = WL.make_inputs("C3", heads=[0], gates=False)
    w = WL.get("C3")
    # per-channel variance near 2 (unit noise + unit low-rank signal)
    assert 1.8 < x["q"].var() < 2.2
    # the cube-constant component survives pooling: pooled variance >> 1/64
    qc = x["q"][0, 0].reshape(w.T // 4, 4, w.H // 4, 4, w.W // 4, 4, -1).mean(axis=(1, 3, 5))
    assert qc.var() > 0.5


def test_variable_lists():
    x = WL.make_inputs("C5", heads=[3], batches=[1], gates=False)
    idx, lens = x["idx"][0, 0], x["len"][0, 0]
    assert lens.min() >= 8 and lens.max() <= 64
    for i in range(idx.shape[0]):
        row = idx[i, :lens[i]]
        assert np.all(np.diff(row) > 0) and row.min() >= 0 and row.max() < 256
        assert np.all(idx[i, lens[i]:] == -1)
