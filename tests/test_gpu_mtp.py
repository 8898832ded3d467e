"""GPU parity of gdr_decode_mtp (T decode tokens per sequence) against the
oracle: outputs, final states and the state after every token, compared with
the token-by-token recurrence (max|gpu - ref| / max|ref| <= 1e-3 for bf16
inputs, 1e-5 for fp32 inputs, fp32 outputs).  T = 1 must equal
gdr_decode_step bit for bit; the result must agree with gdr_chunk_prefill over
the same tokens packed as N sequences of T tokens."""
import numpy as np
import pytest
import torch

import oracle
from gdr_synth import generate
from gpu_util import dev_inputs, host64, rel_err, say, tol_for

pytestmark = pytest.mark.gpu


def mtp_inputs(N, T, H, d, dtype, seed, gate="std"):
    data = generate([T] * N, H, d, d, dtype=dtype, state0=True, seed=seed, gate=gate)
    di = dev_inputs(data)
    shaped = {key: di[key].view(N, T, H, -1) for key in ("q", "k", "v")}
    shaped["g"] = di["g"].view(N, T, H)
    shaped["beta"] = di["beta"].view(N, T, H)
    shaped["state0"] = di["state0"]
    return data, di, shaped


def run_mtp(x, out_dtype=torch.float32, state_out="new", inter=True):
    import gated_delta_rule_100_amd as gdr
    N, T, H, dk = x["q"].shape
    dv = x["v"].shape[3]
    o = torch.full((N, T, H, dv), float("nan"), dtype=out_dtype, device="cuda")
    I = torch.full((N, T, H, dv, dk), float("nan"), device="cuda") if inter else None
    if state_out == "new":
        so = torch.full_like(x["state0"], float("nan"))
    elif state_out == "inplace":
        so = x["state0"]
    else:
        so = None
    gdr.gdr_decode_mtp(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"], so, o, I)
    torch.cuda.synchronize()
    return o, so, I


CASES = {
    "N3-T4-H2-d128-bf16": (3, 4, 2, 128, "bf16"),
    "N2-T8-H3-d64-f32": (2, 8, 3, 64, "f32"),
    "N4-T2-H2-d128-f32": (4, 2, 2, 128, "f32"),
    "N5-T1-H2-d64-bf16": (5, 1, 2, 64, "bf16"),
    "N2-T16-H1-d128-bf16-slow": (2, 16, 1, 128, "bf16"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_mtp_matches_oracle(name):
    N, T, H, d, dtype = CASES[name]
    gate = "slow" if name.endswith("slow") else "std"
    say(f"mtp {name}")
    data, _, x = mtp_inputs(N, T, H, d, dtype, seed=300 + T, gate=gate)
    o, so, I = run_mtp(x)
    o_ref, s_ref, cs_ref = oracle.recurrent(data["q"], data["k"], data["v"], data["g"],
                                            data["beta"], data["cu_seqlens"], data["state0"],
                                            chunk=1)
    tol = tol_for(data)
    errs = {"o": rel_err(host64(o).reshape(o_ref.shape), o_ref),
            "state_out": rel_err(host64(so), s_ref),
            "inter": rel_err(host64(I).reshape(cs_ref.shape), cs_ref)}
    say(f"  errors: {errs}")
    for key, e in errs.items():
        assert e <= tol, (key, e)


def test_mtp_T1_equals_decode_step_bitwise():
    import gated_delta_rule_100_amd as gdr
    N, H, d = 6, 3, 128
    say("mtp T=1 vs decode step")
    _, di, x = mtp_inputs(N, 1, H, d, "bf16", seed=310)
    for out_dtype in (torch.float32, torch.bfloat16):
        o1, s1, _ = run_mtp(x, out_dtype, inter=False)
        s2 = di["state0"].clone()
        o2 = torch.empty(N, H, d, dtype=out_dtype, device="cuda")
        gdr.gdr_decode_step(di["q"], di["k"], di["v"], di["g"], di["beta"], s2, o2)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(N, H, d), o2)
        assert torch.equal(s1, s2)


# Without per-token states, T >= 2 tokens take the chunked kernel (every 8
# tokens one chunk of the chunked form on the matrix cores, the state kept in
# registers across the chunks; T > 8 ends on a shorter chunk unless T is a
# multiple of 8); T = 1 takes the token-by-token kernel (the decode step,
# tested below).
CHUNKED_CASES = {
    "N3-T6-H2-d128-bf16": (3, 6, 2, 128, "bf16", "std"),
    "N2-T8-H3-d64-f32": (2, 8, 3, 64, "f32", "std"),
    "N4-T7-H2-d128-f32": (4, 7, 2, 128, "f32", "std"),
    "N3-T7-H2-d128-bf16-slow": (3, 7, 2, 128, "bf16", "slow"),
    "N2-T5-H2-d64-bf16-steep": (2, 5, 2, 64, "bf16", "steep"),
    "N2-T8-H2-d128-f32-unit": (2, 8, 2, 128, "f32", "unit"),
    "N2-T12-H2-d64-bf16-slow": (2, 12, 2, 64, "bf16", "slow"),
    "N3-T16-H2-d128-bf16": (3, 16, 2, 128, "bf16", "std"),
    "N2-T17-H2-d128-f32": (2, 17, 2, 128, "f32", "std"),
    "N2-T33-H1-d64-f32-steep": (2, 33, 1, 64, "f32", "steep"),
    "N2-T64-H2-d128-bf16-unit": (2, 64, 2, 128, "bf16", "unit"),
    "N1-T64-H3-d128-f32-slow": (1, 64, 3, 128, "f32", "slow"),
    "N3-T3-H2-d128-bf16": (3, 3, 2, 128, "bf16", "std"),
    "N4-T2-H2-d64-f32-slow": (4, 2, 2, 64, "f32", "slow"),
}


@pytest.mark.parametrize("name", list(CHUNKED_CASES))
def test_mtp_chunked_matches_oracle(name):
    N, T, H, d, dtype, gate = CHUNKED_CASES[name]
    say(f"mtp chunked {name}")
    data, _, x = mtp_inputs(N, T, H, d, dtype, seed=320 + T, gate=gate)
    o, so, _ = run_mtp(x, inter=False)
    o_ref, s_ref, _ = oracle.recurrent(data["q"], data["k"], data["v"], data["g"], data["beta"],
                                       data["cu_seqlens"], data["state0"])
    tol = tol_for(data)
    errs = {"o": rel_err(host64(o).reshape(o_ref.shape), o_ref),
            "state_out": rel_err(host64(so), s_ref)}
    say(f"  errors: {errs}")
    for key, e in errs.items():
        assert e <= tol, (key, e)


def test_mtp_in_place_and_uncommitted():
    N, T, H, d = 3, 6, 2, 128
    say("mtp in place / no final state")
    _, _, x = mtp_inputs(N, T, H, d, "bf16", seed=311)
    ref_o, ref_s, ref_i = run_mtp(x)
    # no final state: the input state is untouched, the last intermediate is the final state
    before = x["state0"].clone()
    o, so, I = run_mtp(x, state_out=None)
    assert so is None and torch.equal(x["state0"], before)
    assert torch.equal(o, ref_o) and torch.equal(I, ref_i)
    assert torch.equal(I[:, -1], ref_s)
    # without intermediates (T >= 2: the chunked kernel): a new final state
    # and in place give the same bits, and both agree with the token-by-token
    # kernel to rounding
    o2, so2, _ = run_mtp(x, inter=False)
    o, so, _ = run_mtp(x, state_out="inplace", inter=False)
    assert torch.equal(o, o2) and torch.equal(x["state0"], so2)
    assert rel_err(host64(o), host64(ref_o)) <= 1e-5
    assert rel_err(host64(so2), host64(ref_s)) <= 1e-5


def test_mtp_bf16_output_is_rne_and_deterministic():
    N, T, H, d = 4, 3, 2, 64
    say("mtp bf16 output and determinism")
    _, _, x = mtp_inputs(N, T, H, d, "bf16", seed=312)
    o32, s32, i32 = run_mtp(x)
    o32b, s32b, i32b = run_mtp(x)
    o16, s16, _ = run_mtp(x, torch.bfloat16)
    assert torch.equal(o32, o32b) and torch.equal(s32, s32b) and torch.equal(i32, i32b)
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(s16, s32)


def test_mtp_agrees_with_prefill():
    import gated_delta_rule_100_amd as gdr
    N, T, H, d = 4, 6, 2, 128
    say("mtp vs prefill of N sequences of T tokens")
    data, di, x = mtp_inputs(N, T, H, d, "bf16", seed=313)
    o, so, _ = run_mtp(x, inter=False)
    op = torch.empty(N * T, H, d, device="cuda")
    sp = torch.empty_like(di["state0"])
    gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"], di["state0"],
                          sp, op, chunk=64)
    torch.cuda.synchronize()
    assert rel_err(host64(o).reshape(N * T, H, d), host64(op)) <= 1e-3
    assert rel_err(host64(so), host64(sp)) <= 1e-3


def test_mtp_full_size_sampled():
    # the decode workload's shape with 4 draft tokens: 64 sequences x 32 heads, d = 128
    N, T, H, d = 64, 4, 32, 128
    say("mtp full size N=64 T=4 H=32 d=128 bf16")
    data, _, x = mtp_inputs(N, T, H, d, "bf16", seed=314)
    o, so, I = run_mtp(x)
    pairs = [(0, 0), (17, 5), (63, 31), (40, 16)]
    o_ref, s_ref, cs_ref = oracle.recurrent(data["q"], data["k"], data["v"], data["g"],
                                            data["beta"], data["cu_seqlens"], data["state0"],
                                            pairs=pairs, chunk=1)
    oh = host64(o).reshape(N * T, H, d)
    Ih = host64(I).reshape(N * T, H, d, d)
    sh = host64(so)
    for n, h in pairs:
        rows = slice(n * T, (n + 1) * T)
        e = (rel_err(oh[rows, h], o_ref[rows, h]), rel_err(sh[n, h], s_ref[n, h]),
             rel_err(Ih[rows, h], cs_ref[rows, h]))
        say(f"  pair ({n},{h}): o {e[0]:.2e} state {e[1]:.2e} inter {e[2]:.2e}")
        assert max(e) <= 1e-3


@pytest.mark.parametrize("T", [8, 32])
def test_mtp_chunked_full_size_sampled(T):
    # the decode workload's shape with 8 (one chunk) or 32 (four chunks) draft
    # tokens, without per-token states
    N, H, d = 64, 32, 128
    say(f"mtp chunked full size N=64 T={T} H=32 d=128 bf16")
    data, _, x = mtp_inputs(N, T, H, d, "bf16", seed=315 + T)
    o, so, _ = run_mtp(x, torch.bfloat16, inter=False)
    o32, so32, _ = run_mtp(x, inter=False)
    assert torch.equal(o, o32.to(torch.bfloat16)) and torch.equal(so, so32)
    pairs = [(0, 0), (17, 5), (63, 31), (40, 16)]
    o_ref, s_ref, _ = oracle.recurrent(data["q"], data["k"], data["v"], data["g"], data["beta"],
                                       data["cu_seqlens"], data["state0"], pairs=pairs)
    oh = host64(o32).reshape(N * T, H, d)
    sh = host64(so32)
    for n, h in pairs:
        rows = slice(n * T, (n + 1) * T)
        e = (rel_err(oh[rows, h], o_ref[rows, h]), rel_err(sh[n, h], s_ref[n, h]))
        say(f"  pair ({n},{h}): o {e[0]:.2e} state {e[1]:.2e}")
        assert max(e) <= 1e-3
