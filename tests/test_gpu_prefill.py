"""GPU parity of gdr_chunk_prefill against the oracle.

Reduced-size versions of every prefill workload (several chunks, ragged
tails, empty and length-1 sequences) are compared element by element with the
token-by-token recurrence (o, final states, chunk-end states) and with the
chunked form's L and M; slow and unit gates make M far from zero so the fixup
is exercised.  Tolerance: max|gpu - ref| / max|ref| <= 1e-3 for bf16 inputs,
1e-5 for fp32 inputs, on fp32 outputs; bf16 outputs must equal the
round-to-nearest-even of the fp32 outputs bit for bit.

Two schedules are covered: the chunk-parallel form (fp32 inputs, chunk 16)
and the sequential chunk scan (bf16 inputs at chunk 64; segmented when the
sequences are long and few), which also writes L and M through the
chunk-local kernel when they are requested.  Each parity case runs with
"cp": L, M and the chunk-end states requested, "scan": the chunk-end states
only, and some with "none": nothing optional."""
import numpy as np
import pytest
import torch

import oracle
from gdr_synth import generate, workload
from gpu_util import dev_inputs, host64, rel_err, say, tol_for

pytestmark = pytest.mark.gpu


def run_prefill(d, out_dtype=torch.float32, chunk=None, schedule="cp", state_in="given"):
    import gated_delta_rule_100_amd as gdr
    chunk = chunk or d["chunk"]
    di = dev_inputs(d)
    T, H, dk = d["q"].shape
    dv = d["v"].shape[2]
    N = d["N"]
    mc = gdr.gdr_max_chunks(T, N, chunk)
    o = torch.full((T, H, dv), float("nan"), dtype=out_dtype, device="cuda")
    sout = torch.full((N, H, dv, dk), float("nan"), device="cuda")
    L = M = F = None
    if schedule == "cp":
        L = torch.full((mc, H, dv, dk), float("nan"), device="cuda")
        M = torch.full((mc, H, dk, dk), float("nan"), device="cuda")
    if schedule in ("cp", "scan"):
        F = torch.full((mc, H, dv, dk), float("nan"), device="cuda")
    sin = di["state0"] if state_in == "given" else None
    gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"], sin, sout, o,
                          chunk=chunk, L_out=L, M_out=M, fixed_out=F)
    torch.cuda.synchronize()
    return dict(o=o, state_out=sout, L=L, M=M, fixed=F)


def check_against_oracle(d, res, chunk, check_locals=True):
    tol = tol_for(d)
    o_ref, s_ref, cs_ref = oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                            d["cu_seqlens"], d["state0"], chunk=chunk)
    errs = {"o": rel_err(host64(res["o"]), o_ref),
            "state_out": rel_err(host64(res["state_out"]), s_ref)}
    if res["fixed"] is not None:
        n = cs_ref.shape[0]
        errs["fixed"] = rel_err(host64(res["fixed"][:n]), cs_ref)
    if check_locals and res["L"] is not None:
        r2 = oracle.chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk,
                            d["state0"])
        n = r2["L"].shape[0]
        errs["L"] = rel_err(host64(res["L"][:n]), r2["L"])
        errs["M"] = rel_err(host64(res["M"][:n]), r2["M"])
    say(f"  errors: {errs}")
    for key, e in errs.items():
        assert e <= tol, (key, e)


CASES = {
    # name: (workload index, overrides)
    "tiny-gdr-T64-H2-d64-C16-f32": (0, {}),
    "tiny-f32-state": (0, dict(state0=True, seqlens=[50, 0, 14, 1], H=2)),
    "prefill-B4-T256-H4-d128-C64-bf16": (2, dict(seqlens=[256] * 4, H=4)),
    "prefill-B4-T256-H4-slow-gates": (2, dict(seqlens=[256] * 4, H=4, gate="slow")),
    "prefill-B2-T200-H2-unit-gates": (2, dict(seqlens=[200, 72], H=2, gate="unit")),
    "varlen-ragged-H2-d128-C64": (3, dict(seqlens=[1, 63, 64, 65, 0, 200, 130, 7], H=2)),
    "varlen-ragged-slow": (3, dict(seqlens=[129, 0, 1, 77], H=2, gate="slow")),
    "long-T8192-H4-slow-gates": (4, dict(seqlens=[8192], H=4, gate="slow")),
    # skewed lengths with enough (sequence, head) pairs to fill the GPU: more
    # scan workgroups than compute units, whole-tile form
    "varlen-skewed-H32": (3, dict(seqlens=[4000, 50, 300, 64, 1, 0, 700, 129], H=32)),
    "varlen-skewed-H32-slow": (3, dict(seqlens=[70, 3100, 0, 1100, 64, 640, 1, 9], H=32,
                                       gate="slow")),
    # 64 sequences (the most whose chunk layout the scan kernels form
    # themselves) and 65 (the layout kernel runs first), with empty ones
    "varlen-64-sequences": (3, dict(seqlens=[(37 * i) % 150 for i in range(64)], H=2)),
    "varlen-65-sequences": (3, dict(seqlens=[(41 * i) % 170 for i in range(65)], H=2)),
    # in-chunk decays far below e^-87: decay factors and gamma underflow
    "steep-gates-ragged": (2, dict(seqlens=[200, 130, 64, 5], H=2, gate="steep")),
    "d64-C64-bf16": (2, dict(seqlens=[150, 64, 3], H=3, dk=64, dv=64, gate="slow")),
    "d128-C16-bf16": (2, dict(seqlens=[70, 33], H=2, chunk=16, gate="slow")),
    "d128-C16-f32": (0, dict(seqlens=[40, 17, 0], H=2, dk=128, dv=128, gate="slow", state0=True)),
    # many (sequence, head) pairs: the fixup takes 32 and 64 state rows per workgroup
    "many-heads-H64-rows32": (2, dict(seqlens=[150, 70], H=64, gate="slow")),
    "many-heads-H128-rows64": (2, dict(seqlens=[100], H=128, gate="slow")),
    # fp32 inputs at chunk 64 (the chunk-parallel form on three bf16 planes per
    # operand), reduced versions of the prefill, varlen and long workloads:
    # ragged, empty and length-1 sequences; every gate variant; with and
    # without an initial state; L and M checked against the chunked oracle
    "f32-C64-prefill-ragged": (2, dict(seqlens=[256, 130, 1, 0, 64], H=2, dtype="f32")),
    "f32-C64-prefill-slow-no-state": (2, dict(seqlens=[200, 65], H=2, dtype="f32", gate="slow",
                                              state0=False)),
    "f32-C64-varlen-steep": (3, dict(seqlens=[1, 63, 64, 65, 0, 129], H=2, dtype="f32",
                                     gate="steep")),
    "f32-C64-varlen-unit": (3, dict(seqlens=[100, 0, 1, 77], H=2, dtype="f32", gate="unit")),
    "f32-C64-long-slow": (4, dict(seqlens=[4096], H=2, dtype="f32", gate="slow")),
    "f32-C64-d64": (2, dict(seqlens=[150, 64, 3], H=3, dk=64, dv=64, dtype="f32", gate="slow")),
}


SCHEDULES = ["cp", "scan"]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle(name, schedule):
    idx, ov = CASES[name]
    d = workload(idx, seed=100 + idx, **ov)
    say(f"prefill {name} [{schedule}]: T={d['T']} N={d['N']} H={d['H']} d={d['dk']} "
        f"C={d['chunk']} {d['dtype']}")
    res = run_prefill(d, schedule=schedule)
    check_against_oracle(d, res, d["chunk"], check_locals=d["T"] <= 20000)


@pytest.mark.parametrize("seqlens", [[256, 130, 1], [16384]])
def test_prefill_large_values(seqlens):
    # v and the initial state 4096 times the recipe's (exact in bf16 and fp32):
    # the scan's fp16 operand planes of R / 16 in U = T R then reach several
    # hundred, and the errors stay within the tolerance relative to max|ref|;
    # [16384] takes the segmented scan
    from gdr_synth import bf16_bits_from_f32
    d = workload(2, seed=120, seqlens=seqlens, H=2, gate="slow")
    d["v"] = bf16_bits_from_f32((oracle.bf16_to_f64(d["v"]) * 4096.0).astype(np.float32))
    d["state0"] = (d["state0"] * np.float32(4096.0)).astype(np.float32)
    say(f"prefill with 4096-fold v and state: T={d['T']} N={d['N']} H={d['H']}")
    res = run_prefill(d, schedule="scan")
    check_against_oracle(d, res, d["chunk"], check_locals=False)


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_prefill_without_initial_state(schedule):
    d = workload(2, seed=110, seqlens=[130, 64, 0, 5], H=2, gate="slow")
    say(f"prefill without initial state [{schedule}]")
    res = run_prefill(d, schedule=schedule, state_in=None)
    d0 = dict(d)
    d0["state0"] = None
    check_against_oracle(d0, res, d["chunk"])


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_prefill_bf16_output_is_rne_of_fp32_and_deterministic(schedule):
    d = workload(3, seed=111, seqlens=[300, 1, 64, 129], H=2)
    say(f"prefill bf16-vs-fp32 output and determinism [{schedule}]")
    r32 = run_prefill(d, torch.float32, schedule=schedule)
    r32b = run_prefill(d, torch.float32, schedule=schedule)
    r16 = run_prefill(d, torch.bfloat16, schedule=schedule)
    n_chunks = int(oracle.layout(d["cu_seqlens"], d["chunk"])[0][-1])
    for key in ("o", "state_out"):
        assert torch.equal(r32[key], r32b[key]), key
    for key in ("L", "M", "fixed"):  # slots past the real chunk count are never written
        if r32[key] is not None:
            assert torch.equal(r32[key][:n_chunks], r32b[key][:n_chunks]), key
    assert torch.equal(r16["o"], r32["o"].to(torch.bfloat16))
    assert torch.equal(r16["state_out"], r32["state_out"])


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_prefill_packing_invariance(schedule):
    # a packed varlen batch gives bit-identical results to separate calls
    lens = [77, 0, 130, 64, 1]
    d = workload(3, seed=112, seqlens=lens, H=2)
    say(f"prefill packing invariance [{schedule}]")
    packed = run_prefill(d, schedule=schedule)
    cu = d["cu_seqlens"]
    for n, ln in enumerate(lens):
        a, b = int(cu[n]), int(cu[n + 1])
        sub = dict(d)
        for key in ("q", "k", "v", "g", "beta"):
            sub[key] = np.ascontiguousarray(d[key][a:b])
        sub["state0"] = np.ascontiguousarray(d["state0"][n:n + 1])
        sub["cu_seqlens"] = np.array([0, b - a], dtype=np.int32)
        sub["N"], sub["T"] = 1, b - a
        single = run_prefill(sub, schedule=schedule)
        assert torch.equal(single["o"], packed["o"][a:b])
        assert torch.equal(single["state_out"][0], packed["state_out"][n])


def test_prefill_scan_forms_agree_bitwise():
    # The sequential scan splits each 16-row state tile over two SIMDs when the
    # workgroups of a batch fit the GPU at once (few (sequence, head) pairs)
    # and keeps whole tiles per wave otherwise; both add the two column
    # halves' contractions in the same order, so a packed batch of many pairs
    # (whole tiles) and its sequences run alone (split tiles) agree bit for bit.
    rng = np.random.default_rng(113)
    lens = [int(x) for x in rng.integers(1, 200, size=33)]
    lens[3], lens[10] = 0, 64
    d = workload(3, seed=113, seqlens=lens, H=8)
    say(f"prefill scan forms: N={len(lens)} H=8 T={d['T']} (packed: whole tiles; alone: split)")
    packed = run_prefill(d, schedule="scan")
    check_against_oracle(d, packed, d["chunk"], check_locals=False)
    cu = d["cu_seqlens"]
    for n in (0, 3, 10, 32):
        a, b = int(cu[n]), int(cu[n + 1])
        sub = dict(d)
        for key in ("q", "k", "v", "g", "beta"):
            sub[key] = np.ascontiguousarray(d[key][a:b])
        sub["state0"] = np.ascontiguousarray(d["state0"][n:n + 1])
        sub["cu_seqlens"] = np.array([0, b - a], dtype=np.int32)
        sub["N"], sub["T"] = 1, b - a
        single = run_prefill(sub, schedule="scan")
        assert torch.equal(single["o"], packed["o"][a:b])
        assert torch.equal(single["state_out"][0], packed["state_out"][n])
        c0 = int(np.sum((np.array(lens[:n]) + 63) // 64))
        nc = (b - a + 63) // 64
        assert torch.equal(single["fixed"][:nc], packed["fixed"][c0:c0 + nc])


@pytest.mark.parametrize("dk,H", [(128, 32), (64, 32), (128, 12)])
def test_prefill_mixed_scan_agrees_bitwise(dk, H):
    # A batch whose column-split workgroups do not all fit the GPU at once but
    # whose longest sequence dominates: the scan runs that sequence in the
    # split form and the others in whole tiles, in one launch (also with L and
    # M requested, when the chunk-local kernel runs first).  Each sequence run
    # alone takes the split form; all agree bit for bit, wherever the long
    # sequence sits in the batch.
    lens = [37, 0, 64, 5, 1, 650, 20, 129]
    d = workload(3, seed=131, seqlens=lens, H=H, dk=dk, dv=dk)
    say(f"prefill mixed scan: N={len(lens)} H={H} d={dk} T={d['T']} (long sequence 5)")
    packed = run_prefill(d, schedule="scan")
    check_against_oracle(d, packed, d["chunk"], check_locals=False)
    with_lm = run_prefill(d, schedule="cp")  # L and M requested
    nc = int(np.sum((np.array(lens) + 63) // 64))  # chunk slots written
    assert torch.equal(with_lm["o"], packed["o"])
    assert torch.equal(with_lm["state_out"], packed["state_out"])
    assert torch.equal(with_lm["fixed"][:nc], packed["fixed"][:nc])
    cu = d["cu_seqlens"]
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        sub = dict(d)
        for key in ("q", "k", "v", "g", "beta"):
            sub[key] = np.ascontiguousarray(d[key][a:b])
        sub["state0"] = np.ascontiguousarray(d["state0"][n:n + 1])
        sub["cu_seqlens"] = np.array([0, b - a], dtype=np.int32)
        sub["N"], sub["T"] = 1, b - a
        single = run_prefill(sub, schedule="scan")
        assert torch.equal(single["o"], packed["o"][a:b])
        assert torch.equal(single["state_out"][0], packed["state_out"][n])
        c0 = int(np.sum((np.array(lens[:n]) + 63) // 64))
        nc = (b - a + 63) // 64
        assert torch.equal(single["fixed"][:nc], packed["fixed"][c0:c0 + nc])


def test_prefill_mixed_scan_eligibility_boundary():
    # Up to 63 sequences a batch whose split form does not fit may take the
    # mixed launch (here: one long sequence among short ones); with a 64th,
    # empty sequence the same batch runs in whole tiles.  Same bits.
    rng = np.random.default_rng(143)
    lens = [int(x) for x in rng.integers(1, 100, size=63)]
    lens[17], lens[40] = 1200, 0
    d = workload(3, seed=143, seqlens=lens, H=2)
    say(f"prefill mixed/whole boundary: N=63 and 64, H=2, T={d['T']}")
    mixed = run_prefill(d, schedule="scan")
    check_against_oracle(d, mixed, d["chunk"], check_locals=False)
    d64 = dict(d)
    d64["cu_seqlens"] = np.concatenate([d["cu_seqlens"], d["cu_seqlens"][-1:]]).astype(np.int32)
    d64["state0"] = np.concatenate([d["state0"], d["state0"][:1]], axis=0)
    d64["N"] = 64
    whole = run_prefill(d64, schedule="scan")
    nc = int(np.sum((np.array(lens) + 63) // 64))
    assert torch.equal(mixed["o"], whole["o"])
    assert torch.equal(mixed["state_out"], whole["state_out"][:63])
    assert torch.equal(mixed["fixed"][:nc], whole["fixed"][:nc])


def test_prefill_workspace_on_side_stream():
    """With no workspace given, the binding allocates one on the launch stream:
    a prefill on a side stream followed at once by allocations and writes on
    the current stream gives the same bits as a prefill on the current stream."""
    d = workload(3, seed=119, seqlens=[300, 1, 64, 129], H=4)
    say("prefill on a side stream with the binding's own workspace")
    import gated_delta_rule_100_amd as gdr
    ref = run_prefill(d, schedule="none")
    di = dev_inputs(d)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o = torch.empty_like(ref["o"])
    sout = torch.empty_like(ref["state_out"])
    gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"], di["state0"],
                          sout, o, chunk=64, stream=side)
    junk = [torch.full((1 << 22,), float(i), device="cuda") for i in range(8)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o, ref["o"])
    assert torch.equal(sout, ref["state_out"])


def test_prefill_all_sequences_empty():
    import gated_delta_rule_100_amd as gdr
    say("prefill with T_total = 0")
    H, dk = 2, 128
    s0 = torch.randn(3, H, dk, dk, device="cuda")
    sout = torch.full_like(s0, float("nan"))
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    e = torch.empty(0, H, dk, dtype=torch.bfloat16, device="cuda")
    ge = torch.empty(0, H, dtype=torch.float32, device="cuda")
    gdr.gdr_chunk_prefill(e, e, e, ge, ge, cu, s0, sout, e.clone(), chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(sout, s0)
    gdr.gdr_chunk_prefill(e, e, e, ge, ge, cu, None, sout, e.clone(), chunk=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(sout) == 0


def test_prefill_in_place_state():
    d = workload(2, seed=113, seqlens=[100, 0, 64], H=2, gate="slow")
    say("prefill in-place state")
    import gated_delta_rule_100_amd as gdr
    di = dev_inputs(d)
    ref = run_prefill(d, schedule="none")
    st = di["state0"].clone()
    o = torch.empty_like(ref["o"])
    gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"], st, st, o,
                          chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o, ref["o"])
    assert torch.equal(st, ref["state_out"])


def test_prefill_mixed_scan_repeated():
    """The mixed scan (the long sequence in the split form beside the others in
    whole tiles) gives the same bits on every call, with and without L and M
    requested."""
    lens = [4000, 50, 300, 64, 1, 0, 700, 129]
    d = workload(3, seed=141, seqlens=lens, H=32)
    say(f"prefill mixed scan x8 against the same call with L and M, T={d['T']}")
    ref = run_prefill(d, schedule="cp")
    nc = int(np.sum((np.array(lens) + 63) // 64))  # chunk slots written
    for _ in range(8):
        got = run_prefill(d, schedule="scan")
        assert torch.equal(got["o"], ref["o"])
        assert torch.equal(got["state_out"], ref["state_out"])
        assert torch.equal(got["fixed"][:nc], ref["fixed"][:nc])


def test_prefill_in_place_state_mixed():
    """The mixed scan in place gives the same bits as with a separate output,
    and without initial states it matches the oracle from zero states."""
    lens = [300, 1, 900, 0, 64, 70, 5, 200]
    d = workload(3, seed=139, seqlens=lens, H=32, gate="slow")
    say(f"prefill in-place state, mixed scan, T={d['T']}")
    import gated_delta_rule_100_amd as gdr
    di = dev_inputs(d)
    ref = run_prefill(d, schedule="none")
    st = di["state0"].clone()
    o = torch.empty_like(ref["o"])
    gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"], st, st, o,
                          chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o, ref["o"])
    assert torch.equal(st, ref["state_out"])
    zero = run_prefill(d, schedule="none", state_in="none")
    d0 = dict(d)
    d0["state0"] = np.zeros_like(d["state0"])
    check_against_oracle(d0, zero, d["chunk"], check_locals=False)


def test_prefill_in_place_state_segmented():
    """The segmented scan reads the initial state for the segment fixup and the
    segment starts, and writes the final state last: in place gives the same
    bits as a separate output."""
    d = workload(4, seed=118, seqlens=[30000, 0, 19500], H=1, gate="slow", state0=True)
    say("prefill in-place state, segmented scan")
    import gated_delta_rule_100_amd as gdr
    di = dev_inputs(d)
    ref = run_prefill(d, schedule="none")
    st = di["state0"].clone()
    o = torch.empty_like(ref["o"])
    gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"], st, st, o,
                          chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o, ref["o"])
    assert torch.equal(st, ref["state_out"])


def test_prefill_guard_bands():
    import gated_delta_rule_100_amd as gdr
    d = workload(3, seed=114, seqlens=[65, 1, 130], H=2)
    say("prefill guard bands")
    di = dev_inputs(d)
    T, H, dv = d["T"], d["H"], d["dv"]
    G = 512
    n_o = T * H * dv
    obuf = torch.full((n_o + 2 * G,), float("nan"), device="cuda")
    o = obuf[G:G + n_o].view(T, H, dv)
    n_s = d["N"] * H * dv * d["dk"]
    sbuf = torch.full((n_s + 2 * G,), float("nan"), device="cuda")
    sout = sbuf[G:G + n_s].view(d["N"], H, dv, d["dk"])
    gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"], di["state0"],
                          sout, o, chunk=64)
    torch.cuda.synchronize()
    for buf, n in ((obuf, n_o), (sbuf, n_s)):
        assert torch.isnan(buf[:G]).all() and torch.isnan(buf[G + n:]).all()
        assert torch.isfinite(buf[G:G + n]).all()


def test_decode_steps_equal_prefill():
    import gated_delta_rule_100_amd as gdr
    d = workload(2, seed=115, seqlens=[40], H=2, gate="slow")
    say("decode chain vs prefill")
    di = dev_inputs(d)
    res = run_prefill(d, schedule="none")
    st = di["state0"].clone()
    outs = []
    for t in range(d["T"]):
        o = torch.empty(1, 2, 128, device="cuda")
        one = [di[key][t:t + 1].clone() for key in ("q", "k", "v", "g", "beta")]
        gdr.gdr_decode_step(*one, st, o)
        outs.append(o[0])
    torch.cuda.synchronize()
    assert rel_err(host64(torch.stack(outs)), host64(res["o"])) <= 1e-3
    assert rel_err(host64(st), host64(res["state_out"])) <= 1e-3


def test_split_prefill_resumes():
    d = workload(2, seed=116, seqlens=[300], H=2, gate="slow")
    say("split prefill resume")
    full = run_prefill(d, schedule="none")
    T1 = 130
    parts = []
    state = d["state0"]
    for a, b in ((0, T1), (T1, 300)):
        sub = dict(d)
        for key in ("q", "k", "v", "g", "beta"):
            sub[key] = np.ascontiguousarray(d[key][a:b])
        sub["state0"] = state
        sub["cu_seqlens"] = np.array([0, b - a], dtype=np.int32)
        sub["T"] = b - a
        r = run_prefill(sub, schedule="none")
        parts.append(r["o"])
        state = r["state_out"].cpu().numpy()
    assert rel_err(host64(torch.cat(parts)), host64(full["o"])) <= 1e-3
    assert rel_err(state.astype(np.float64), host64(full["state_out"])) <= 1e-3


# Long sequences with few heads: bf16 inputs take the segmented scan (local
# segment states, segment transfer matrices, segment fixup, final pass from the
# true starts), with L and M from the chunk-local kernel when requested ("cp");
# fp32 inputs take the two-level fixup of the chunk-parallel form (fold
# segments of chunks, scan the segments, apply the scanned starts).
LONG_CASES = {
    "long-T32768-H1-slow": (4, dict(seqlens=[32768], H=1, gate="slow")),
    # fp32 inputs always take the chunk-parallel form: here its two-level fixup
    "long-T32768-H1-f32-state": (4, dict(seqlens=[32768], H=1, gate="slow", dtype="f32",
                                         state0=True)),
    "long-T32768-H1-unit-state": (4, dict(seqlens=[32768], H=1, gate="unit", state0=True)),
    "long-T32768-H1-std-state": (4, dict(seqlens=[32768], H=1, state0=True)),
    "long-varlen-ragged-empty-H1": (4, dict(seqlens=[30000, 0, 19500], H=1, gate="slow",
                                            state0=True)),
}


@pytest.mark.parametrize("schedule", ["cp", "scan", "none"])
@pytest.mark.parametrize("name", list(LONG_CASES))
def test_prefill_long_two_level(name, schedule):
    idx, ov = LONG_CASES[name]
    d = workload(idx, seed=120, **ov)
    say(f"prefill long {name} ({schedule}): T={d['T']} N={d['N']} H={d['H']}")
    res = run_prefill(d, schedule=schedule)
    check_against_oracle(d, res, d["chunk"], check_locals=False)
