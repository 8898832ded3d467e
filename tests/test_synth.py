"""The seeded input generator: encodings and the varlen length recipe."""
import numpy as np
import torch

from gdr_synth import bf16_bits_from_f32, generate, varlen_lengths, workload


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 0.0, 1e-40],
                                 dtype=np.float32)])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_varlen_lengths_recipe():
    for seed in range(20):
        rng = np.random.Generator(np.random.PCG64(seed))
        lens = varlen_lengths(rng, 8, 32768, 16384)
        assert lens.sum() == 32768 and lens.min() >= 1 and lens.max() <= 16384


def test_workload_shapes_and_determinism():
    a = workload(0)
    b = workload(0)
    for key in ("q", "k", "v", "g", "beta"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].dtype == np.float32 and a["q"].shape == (64, 2, 64)
    assert np.all(a["g"] < 0) and np.all((a["beta"] > 0) & (a["beta"] < 1))
    assert a["state0"] is None
    nrm = np.linalg.norm(a["k"].astype(np.float64), axis=-1)
    assert np.allclose(nrm, 1.0, atol=1e-6)
    c3 = workload(3, H=1)
    assert c3["T"] == 32768 and c3["N"] == 8 and c3["cu_seqlens"][-1] == 32768


def test_orthonormal_keys_option():
    d = generate([16, 5], 2, 16, 8, dtype="f32", keys="orthonormal", seed=3)
    k = d["k"].astype(np.float64)
    for n, (a, b) in enumerate(((0, 16), (16, 21))):
        for h in range(2):
            G = k[a:b, h] @ k[a:b, h].T
            assert np.allclose(G, np.eye(b - a), atol=1e-6)
