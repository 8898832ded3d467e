"""GPU parity of gdr_decode_step against the oracle's recurrence (T = 1)."""
import numpy as np
import pytest
import torch

import oracle
from gdr_synth import generate, workload
from gpu_util import (dev_inputs, host64, rel_err, say, tol_for)

pytestmark = pytest.mark.gpu


def run_decode(di, out_dtype, state):
    import gated_delta_rule_100_amd as gdr
    N, H, _ = di["q"].shape
    dv = di["v"].shape[2]
    o = torch.empty(N, H, dv, dtype=out_dtype, device="cuda")
    gdr.gdr_decode_step(di["q"], di["k"], di["v"], di["g"], di["beta"], state, o)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("case", ["decode-N64-H32-d128-bf16", "d64-bf16", "d128-f32", "d64-f32"])
def test_decode_matches_oracle(case):
    if case == "decode-N64-H32-d128-bf16":
        d = workload(1)
    else:
        dd = 64 if "d64" in case else 128
        d = generate([1] * 9, 3, dd, dd, dtype="bf16" if "bf16" in case else "f32",
                     state0=True, seed=101)
    say(f"decode {case}: N={d['N']} H={d['H']} dk={d['dk']}")
    di = dev_inputs(d)
    s32 = di["state0"].clone()
    o32 = run_decode(di, torch.float32, s32)
    o_ref, s_ref, _ = oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       d["cu_seqlens"], d["state0"])
    tol = tol_for(d)
    assert rel_err(host64(o32), o_ref) <= tol
    assert rel_err(host64(s32), s_ref) <= tol
    # bf16 output is the RNE of the fp32 output, and the state update is deterministic
    s16 = di["state0"].clone()
    o16 = run_decode(di, torch.bfloat16, s16)
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(s16, s32)


def test_decode_chain_equals_recurrence_tiny_fp32():
    # the tiny workload token by token: 64 decode calls (fp32, dk = dv = 64)
    d = workload(0)
    say("decode chain tiny-gdr-T64-H2-d64-f32")
    di = dev_inputs(d)
    T, H, dk = d["q"].shape
    state = torch.zeros(1, H, dk, dk, dtype=torch.float32, device="cuda")
    outs = []
    for t in range(T):
        sl = slice(t, t + 1)
        # fresh (16-byte aligned) copies of the one-token slices
        sub = {key: di[key][sl].clone() for key in ("q", "k", "v", "g", "beta")}
        outs.append(run_decode(sub, torch.float32, state)[0])
    o = torch.stack(outs)
    o_ref, s_ref, _ = oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       d["cu_seqlens"], None)
    assert rel_err(host64(o), o_ref) <= 1e-5
    assert rel_err(host64(state), s_ref) <= 1e-5


def test_decode_leaves_guard_bands_untouched():
    import gated_delta_rule_100_amd as gdr
    d = generate([1] * 5, 2, 128, 128, dtype="bf16", state0=True, seed=102)
    say("decode guard bands")
    di = dev_inputs(d)
    G = 256
    n_state = 5 * 2 * 128 * 128
    sbuf = torch.full((n_state + 2 * G,), float("nan"), device="cuda")
    state = sbuf[G:G + n_state].view(5, 2, 128, 128)
    state.copy_(di["state0"])
    obuf = torch.full((5 * 2 * 128 + 2 * G,), float("nan"), device="cuda")
    o = obuf[G:G + 5 * 2 * 128].view(5, 2, 128)
    gdr.gdr_decode_step(di["q"], di["k"], di["v"], di["g"], di["beta"], state, o)
    torch.cuda.synchronize()
    for buf, n in ((sbuf, n_state), (obuf, 5 * 2 * 128)):
        assert torch.isnan(buf[:G]).all() and torch.isnan(buf[G + n:]).all()
        assert torch.isfinite(buf[G:G + n]).all()
