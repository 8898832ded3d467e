"""Seeded random multi-token decode configurations against the oracle.

Twelve fixed seeds each draw N, H, d in {64, 128}, bf16 or fp32 inputs and a
gate variant; even seeds take 2 <= T <= 40 tokens without per-token states (the
chunked kernel, one to five chunks of 8), odd seeds T in 1..16 with or without
them (the token-by-token kernel with them or for T = 1, else the chunked one),
and compare outputs, final states and per-token states with the token-by-token
recurrence (1e-3 for bf16 inputs, 1e-5 for fp32)."""
import numpy as np
import pytest

import oracle
from gpu_util import host64, rel_err, say, tol_for
from test_gpu_mtp import mtp_inputs, run_mtp

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", list(range(500, 512)))
def test_mtp_random_config(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 6))
    chunked = seed % 2 == 0  # half the seeds take the chunked kernel
    T = int(rng.integers(2, 41)) if chunked else int(rng.integers(1, 17))
    H = int(rng.choice([1, 2, 3, 4]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    gate = str(rng.choice(["std", "slow", "steep", "unit"]))
    inter = False if chunked else bool(rng.integers(0, 2))
    say(f"random mtp seed {seed}: N={N} T={T} H={H} d={d} {dtype} gate={gate} inter={inter}")
    data, _, x = mtp_inputs(N, T, H, d, dtype, seed=seed, gate=gate)
    o, so, I = run_mtp(x, inter=inter)
    o_ref, s_ref, cs_ref = oracle.recurrent(data["q"], data["k"], data["v"], data["g"],
                                            data["beta"], data["cu_seqlens"], data["state0"],
                                            chunk=1 if inter else 0)
    tol = tol_for(data)
    errs = {"o": rel_err(host64(o).reshape(o_ref.shape), o_ref),
            "state_out": rel_err(host64(so), s_ref)}
    if inter:
        errs["inter"] = rel_err(host64(I).reshape(cs_ref.shape), cs_ref)
    say(f"  errors: {errs}")
    for key, e in errs.items():
        assert e <= tol, (key, e)
