"""Full-size prefill workloads, in the launch configuration the benchmark
uses, checked on EVERY (sequence, head) pair against the token-by-token
recurrence of the oracle: outputs, final states and every chunk-end state,
element by element, max|gpu - ref| / max|ref| per tensor <= 1e-3 for bf16
inputs and <= 1e-5 for fp32 inputs (fp32 outputs).

bf16 inputs take the scan schedules (sequential scan; segmented for the long
sequence), with L and M from the chunk-local kernel when they are requested
(checked on sampled chunks against the chunked oracle).  fp32 inputs of the
same shapes take the chunk-parallel form (chunk-local L and M, the dense
fixup -- two-level for the long sequence -- and the chunk outputs)."""
import numpy as np
import pytest
import torch

import oracle
from gdr_synth import workload
from gpu_util import BF16_TOL, FP32_TOL, dev_inputs, host64, rel_err, say

pytestmark = pytest.mark.gpu


def run_full(d, keep_fixed=True, keep_lm=False):
    import gated_delta_rule_100_amd as gdr
    di = dev_inputs(d)
    T, H, D, N, C = d["T"], d["H"], d["dk"], d["N"], d["chunk"]
    o = torch.full((T, H, D), float("nan"), dtype=torch.float32, device="cuda")
    sout = torch.full((N, H, D, D), float("nan"), device="cuda")
    F = L = M = None
    mc = gdr.gdr_max_chunks(T, N, C)
    if keep_fixed:
        F = torch.full((mc, H, D, D), float("nan"), device="cuda")
    if keep_lm:
        L = torch.full((mc, H, D, D), float("nan"), device="cuda")
        M = torch.full((mc, H, D, D), float("nan"), device="cuda")
    gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"], di["state0"],
                          sout, o, chunk=C, L_out=L, M_out=M, fixed_out=F)
    torch.cuda.synchronize()
    del di
    return dict(o=o, state_out=sout, fixed=F, L=L, M=M)


def check_all_pairs(d, res, tol):
    """Every pair: o, final states and (when kept) every chunk-end state."""
    keep_fixed = res["fixed"] is not None
    o_ref, s_ref, cs_ref = oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                            d["cu_seqlens"], d["state0"],
                                            chunk=d["chunk"] if keep_fixed else 0)
    errs = {"o": rel_err(host64(res["o"]), o_ref),
            "state_out": rel_err(host64(res["state_out"]), s_ref)}
    del o_ref, s_ref
    if keep_fixed:
        n = cs_ref.shape[0]
        # per block of chunk slots, so that the fp64 copies stay small
        scale = float(np.max(np.abs(cs_ref)))
        worst = 0.0
        for a in range(0, n, 64):
            b = min(a + 64, n)
            got = host64(res["fixed"][a:b])
            if not np.all(np.isfinite(got)):
                worst = float("inf")
                break
            worst = max(worst, float(np.max(np.abs(got - cs_ref[a:b]))))
        errs["fixed"] = worst / scale
        del cs_ref
    say(f"  all pairs: {errs}")
    for key, e in errs.items():
        assert e <= tol, (key, e)
    return errs


def check_lm_samples(d, res, tol, chunks):
    """L and M of sampled chunk slots (all heads) against the chunked oracle."""
    K, V = oracle.as_f64(d["k"]), oracle.as_f64(d["v"])
    g, b = d["g"].astype(np.float64), d["beta"].astype(np.float64)
    cu = d["cu_seqlens"]
    _, idx = oracle.layout(cu, d["chunk"])
    eL = eM = 0.0
    for c in chunks:
        n, j = idx[c]
        lo, hi = oracle.chunk_token_range(cu, d["chunk"], n, j)
        for h in range(d["H"]):
            loc = oracle.chunk_local(K[lo:hi, h], V[lo:hi, h], g[lo:hi, h], b[lo:hi, h])
            eL = max(eL, rel_err(host64(res["L"][c, h]), loc["L"]))
            eM = max(eM, rel_err(host64(res["M"][c, h]), loc["M"]))
    say(f"  L/M on chunk slots {list(chunks)}: L {eL:.2e} M {eM:.2e}")
    assert eL <= tol and eM <= tol, (eL, eM)


def test_full_prefill_B4_T4096_H16():
    d = workload(2)
    say("full prefill B=4 T=4096 H=16 d=128 C=64 bf16 (scan), every pair")
    res = run_full(d)
    check_all_pairs(d, res, BF16_TOL)


def test_full_prefill_B4_T4096_H16_with_L_and_M():
    d = workload(2)
    say("full prefill B=4 T=4096 H=16 bf16, L and M requested, every pair")
    res = run_full(d, keep_lm=True)
    check_all_pairs(d, res, BF16_TOL)
    check_lm_samples(d, res, BF16_TOL, [0, 63, 64, 200, 255])


def test_full_prefill_B4_T4096_H16_f32_chunk_parallel():
    d = workload(2, dtype="f32")
    say("full prefill B=4 T=4096 H=16 fp32 inputs (chunk-parallel form), every pair")
    res = run_full(d, keep_lm=True)
    check_all_pairs(d, res, FP32_TOL)
    check_lm_samples(d, res, FP32_TOL, [0, 100, 255])


def test_full_varlen_32768_tokens_H32():
    d = workload(3)
    say(f"full varlen lengths={list(d['seqlens'])} H=32 bf16 (scan), every pair")
    res = run_full(d)
    check_all_pairs(d, res, BF16_TOL)


def test_full_varlen_32768_tokens_H32_f32_chunk_parallel():
    d = workload(3, dtype="f32")
    say(f"full varlen lengths={list(d['seqlens'])} H=32 fp32 inputs (chunk-parallel form), "
        "every pair")
    res = run_full(d)
    check_all_pairs(d, res, FP32_TOL)


def test_full_long_T131072_H4():
    d = workload(4)
    say("full long sequence B=1 T=131072 H=4 bf16 (segmented scan), every head")
    res = run_full(d)
    check_all_pairs(d, res, BF16_TOL)


def test_full_long_T131072_H4_with_L_and_M():
    d = workload(4)
    say("full long sequence B=1 T=131072 H=4 bf16, L and M requested, every head")
    res = run_full(d, keep_lm=True)
    check_all_pairs(d, res, BF16_TOL)
    check_lm_samples(d, res, BF16_TOL, [0, 1024, 2047])


def test_full_long_T131072_H4_f32_two_level():
    d = workload(4, dtype="f32")
    say("full long sequence B=1 T=131072 H=4 fp32 inputs (chunk-parallel form, two-level "
        "fixup), every head")
    res = run_full(d)
    check_all_pairs(d, res, FP32_TOL)
