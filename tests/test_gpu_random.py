"""Seeded random prefill configurations against the oracle.

Twenty fixed seeds each draw a packed batch (1-12 sequences with empty,
length-1, ragged and chunk-multiple lengths), a head count, d in {64, 128},
a gate variant (std, slow, steep, unit), an initial state or none, and what
the caller asks for (L and M -- the chunk-parallel form --, the chunk-end
states, or nothing).  Every output is compared element by element with the
token-by-token recurrence of the oracle (max|gpu - ref| / max|ref| <= 1e-3,
bf16 inputs, fp32 outputs), so the schedule choices (sequential scan in its
whole-tile and column-split forms, chunk-parallel form) and the ragged-chunk
handling are crossed with each other."""
import numpy as np
import pytest

from gdr_synth import workload
from gpu_util import say
from test_gpu_prefill import check_against_oracle, run_prefill

pytestmark = pytest.mark.gpu


def random_case(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 13))
    kinds = rng.integers(0, 5, size=N)
    lens = []
    for kind in kinds:
        if kind == 0:
            lens.append(int(rng.choice([0, 1])))
        elif kind == 1:
            lens.append(int(rng.integers(2, 64)))
        elif kind == 2:
            lens.append(64 * int(rng.integers(1, 5)))
        else:
            lens.append(int(rng.integers(65, 500)))
    H = int(rng.choice([1, 2, 3, 4, 8]))
    d = int(rng.choice([64, 128]))
    gate = str(rng.choice(["std", "slow", "steep", "unit"]))
    state0 = bool(rng.integers(0, 2))
    schedule = str(rng.choice(["cp", "scan", "none"]))
    return dict(lens=lens, H=H, d=d, gate=gate, state0=state0, schedule=schedule)


@pytest.mark.parametrize("seed", list(range(400, 420)))
def test_prefill_random_config(seed):
    c = random_case(seed)
    if sum(c["lens"]) == 0:
        c["lens"][0] = 1
    d = workload(2, seed=seed, seqlens=c["lens"], H=c["H"], dk=c["d"], dv=c["d"],
                 gate=c["gate"], state0=c["state0"])
    say(f"random prefill seed {seed}: lens={c['lens']} H={c['H']} d={c['d']} gate={c['gate']} "
        f"state0={c['state0']} ask={c['schedule']}")
    res = run_prefill(d, schedule=c["schedule"], state_in="given" if c["state0"] else None)
    check_against_oracle(d, res, d["chunk"])


@pytest.mark.parametrize("seed", list(range(430, 440)))
def test_prefill_random_config_f32(seed):
    """The same draws with fp32 inputs (chunk 64, the chunk-parallel form on
    three bf16 planes per operand), compared at 1e-5."""
    c = random_case(seed)
    if sum(c["lens"]) == 0:
        c["lens"][0] = 1
    d = workload(2, seed=seed, seqlens=c["lens"], H=c["H"], dk=c["d"], dv=c["d"],
                 gate=c["gate"], state0=c["state0"], dtype="f32")
    say(f"random fp32 prefill seed {seed}: lens={c['lens']} H={c['H']} d={c['d']} "
        f"gate={c['gate']} state0={c['state0']} ask={c['schedule']}")
    res = run_prefill(d, schedule=c["schedule"], state_in="given" if c["state0"] else None)
    check_against_oracle(d, res, d["chunk"])
