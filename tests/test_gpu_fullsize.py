"""Full-size prefill workloads, in the launch configuration the benchmark
uses, checked on sampled (sequence, head) pairs that the oracle computes one
by one: outputs, final states and (for the long sequence) every chunk-end
state of the sampled head.  bf16 inputs: max|gpu - ref| / max|ref| <= 1e-3 per
tensor, fp32 outputs."""
import numpy as np
import pytest
import torch

import oracle
from gdr_synth import workload
from gpu_util import dev_inputs, host64, rel_err, say

pytestmark = pytest.mark.gpu


def run_full(d, keep_fixed=False, keep_lm=False):
    import gated_delta_rule_100_amd as gdr
    di = dev_inputs(d)
    T, H, D, N, C = d["T"], d["H"], d["dk"], d["N"], d["chunk"]
    o = torch.empty(T, H, D, dtype=torch.float32, device="cuda")
    sout = torch.empty(N, H, D, D, device="cuda")
    F = L = M = None
    mc = gdr.gdr_max_chunks(T, N, C)
    if keep_fixed:
        F = torch.empty(mc, H, D, D, device="cuda")
    if keep_lm:  # asking for L and M selects the chunk-parallel schedule
        L = torch.empty(mc, H, D, D, device="cuda")
        M = torch.empty(mc, H, D, D, device="cuda")
    gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"], di["state0"],
                          sout, o, chunk=C, L_out=L, M_out=M, fixed_out=F)
    torch.cuda.synchronize()
    return o, sout, F


def check_pairs(d, o, sout, pairs, fixed=None):
    o_ref, s_ref, cs_ref = oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                            d["cu_seqlens"], d["state0"], pairs=pairs,
                                            chunk=d["chunk"] if fixed is not None else 0)
    cu = d["cu_seqlens"]
    offs, _ = oracle.layout(cu, d["chunk"])
    for n, h in pairs:
        a, b = int(cu[n]), int(cu[n + 1])
        e_o = rel_err(host64(o[a:b, h]), o_ref[a:b, h])
        e_s = rel_err(host64(sout[n, h]), s_ref[n, h])
        msg = f"  pair ({n},{h}): o {e_o:.2e} state {e_s:.2e}"
        assert e_o <= 1e-3 and e_s <= 1e-3, msg
        if fixed is not None:
            c0, c1 = int(offs[n]), int(offs[n + 1])
            e_f = rel_err(host64(fixed[c0:c1, h]), cs_ref[c0:c1, h])
            msg += f" fixed {e_f:.2e}"
            assert e_f <= 1e-3, msg
        say(msg)


def test_full_prefill_B4_T4096_H16():
    d = workload(2)
    say("full prefill B=4 T=4096 H=16 d=128 C=64")
    o, sout, _ = run_full(d)
    check_pairs(d, o, sout, [(0, 0), (1, 7), (2, 15), (3, 3)])


def test_full_prefill_B4_T4096_H16_chunk_parallel():
    d = workload(2)
    say("full prefill B=4 T=4096 H=16 d=128 C=64, chunk-parallel schedule")
    o, sout, F = run_full(d, keep_fixed=True, keep_lm=True)
    check_pairs(d, o, sout, [(0, 1), (3, 14)], fixed=F)


def test_full_varlen_32768_tokens_H32():
    d = workload(3)
    say(f"full varlen lengths={list(d['seqlens'])} H=32")
    o, sout, F = run_full(d, keep_fixed=True)
    longest = int(np.argmax(d["seqlens"]))
    check_pairs(d, o, sout, [(longest, 5), (0, 31), (d["N"] - 1, 0)], fixed=F)


def test_full_long_T131072_H4():
    d = workload(4)
    say("full long sequence B=1 T=131072 H=4 (segmented scan)")
    o, sout, F = run_full(d, keep_fixed=True)
    check_pairs(d, o, sout, [(0, 2)], fixed=F)


def test_full_long_T131072_H4_chunk_parallel():
    d = workload(4)
    say("full long sequence B=1 T=131072 H=4 (chunk-parallel form, two-level fixup)")
    o, sout, F = run_full(d, keep_fixed=True, keep_lm=True)
    check_pairs(d, o, sout, [(0, 1)], fixed=F)
