"""gdr_chunk_prefill_noalloc -- the chunked prefill on the library's static
device scratch -- against gdr_chunk_prefill with a caller workspace, through
the C ABI: two calls in a row on one device, the second on a smaller batch
(the scratch keeps the first call's contents), under each schedule the
scratch serves (sequential scan, segmented scan, chunk-parallel form).  The
two entry points run the same kernels, so the results must agree bit for bit.
The workspace of the reference call is filled with NaN first: neither entry
point may depend on the contents of its scratch."""
import numpy as np
import pytest
import torch

from gdr_synth import workload
from gpu_util import dev_inputs, say

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 128 << 20


def run(d, noalloc, keep_lm=False, keep_fixed=True):
    """One prefill through either entry point; fp32 outputs and states."""
    import gated_delta_rule_100_amd as gdr
    di = dev_inputs(d)
    T, H, D, N, C = d["T"], d["H"], d["dk"], d["N"], d["chunk"]
    mc = gdr.gdr_max_chunks(T, N, C)
    o = torch.full((T, H, D), float("nan"), device="cuda")
    sout = torch.full((N, H, D, D), float("nan"), device="cuda")
    F = torch.full((mc, H, D, D), float("nan"), device="cuda") if keep_fixed else None
    L = M = None
    if keep_lm:
        L = torch.full((mc, H, D, D), float("nan"), device="cuda")
        M = torch.full((mc, H, D, D), float("nan"), device="cuda")
    kw = dict(chunk=C, L_out=L, M_out=M, fixed_out=F)
    if noalloc:
        gdr.gdr_chunk_prefill_noalloc(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"],
                                      di["state0"], sout, o, **kw)
    else:
        need = gdr.gdr_chunk_prefill_workspace_bytes(T, N, H, D, D, C, di["q"].dtype)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        ws.view(torch.float16)[: ws.numel() // 2].fill_(float("nan"))
        gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"],
                              di["state0"], sout, o, workspace=ws, **kw)
    torch.cuda.synchronize()
    n = int(sum((np.asarray(d["seqlens"]) + C - 1) // C))
    out = dict(o=o, state_out=sout)
    if F is not None:
        out["fixed"] = F[:n]
    if L is not None:
        out["L"], out["M"] = L[:n], M[:n]
    return out


def same(a, b, what):
    for key in a:
        assert torch.equal(a[key], b[key]), (what, key)


# pairs of calls: (first, second), each (workload index, overrides, ask for L
# and M, ask for the chunk-end states)
SEQUENCES = {
    "scan-then-smaller-scan": ((2, dict(seqlens=[700, 64, 1, 0, 300], H=8), False, True),
                               (3, dict(seqlens=[130, 5], H=2), True, True)),
    # fp32 inputs take the chunk-parallel form; without fixed_out its chunk-end
    # states live in the scratch
    "segmented-then-smaller-chunk-parallel": (
        (4, dict(seqlens=[32768], H=1, state0=True), False, True),
        (2, dict(seqlens=[200, 0, 65], H=2, dtype="f32"), False, False)),
}


@pytest.mark.parametrize("name", list(SEQUENCES))
def test_noalloc_matches_workspace_entry_point(name):
    for i, (idx, ov, lm, fx) in enumerate(SEQUENCES[name]):
        d = workload(idx, seed=900 + i, **ov)
        say(f"noalloc {name} call {i}: T={d['T']} N={d['N']} H={d['H']} {d['dtype']} L/M={lm} "
            f"fixed={fx}")
        ref = run(d, noalloc=False, keep_lm=lm, keep_fixed=fx)
        got = run(d, noalloc=True, keep_lm=lm, keep_fixed=fx)
        same(got, ref, f"{name} call {i}")


def test_noalloc_full_prefill_workload():
    # the benchmark's prefill workload (4 x 4096 tokens, 16 heads) fits the scratch
    d = workload(2)
    say("noalloc full prefill B=4 T=4096 H=16")
    ref = run(d, noalloc=False, keep_fixed=False)
    got = run(d, noalloc=True, keep_fixed=False)
    same(got, ref, "full prefill")


def test_noalloc_refuses_calls_beyond_its_scratch():
    import gated_delta_rule_100_amd as gdr
    # 8 x 4096 tokens, 32 heads: about 220 MB of chunk factors
    T, H, D, N = 32768, 32, 128, 8
    need = gdr.gdr_chunk_prefill_workspace_bytes(T, N, H, D, D, 64, gdr.GDR_BF16)
    assert need > SCRATCH_BYTES
    say(f"noalloc refusal: needs {need} bytes")
    x = torch.zeros(T, H, D, dtype=torch.bfloat16, device="cuda")
    gb = torch.zeros(T, H, device="cuda")
    cu = torch.arange(0, T + 1, T // N, dtype=torch.int32, device="cuda")
    s = torch.zeros(N, H, D, D, device="cuda")
    o = torch.full((T, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdr.GdrError, match="scratch"):
        gdr.gdr_chunk_prefill_noalloc(x, x, x, gb, gb, cu, None, s, o, chunk=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(s) == 0 and bool((o == 7.0).all()), "a refused call writes nothing"
