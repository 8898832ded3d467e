"""Calls on different streams at once.

The library keeps no state between calls except per-device caches filled
before any launch, so calls with their own buffers may run concurrently on
different streams.  Two prefills (each with its own workspace, one of them
with L and M requested) and a decode step are launched on three streams
without synchronising in between, and every result must equal, bit for bit,
the same call run alone."""
import pytest
import torch

from gdr_synth import workload
from gpu_util import dev_inputs, say

pytestmark = pytest.mark.gpu


def _prefill(gdr, d, di, lm, stream=None):
    T, H, D, N, C = d["T"], d["H"], d["dk"], d["N"], d["chunk"]
    o = torch.empty(T, H, D, device="cuda")
    so = torch.empty(N, H, D, D, device="cuda")
    mc = gdr.gdr_max_chunks(T, N, C)
    # zero-filled: chunk slots past the batch's chunks are not written
    L = torch.zeros(mc, H, D, D, device="cuda") if lm else None
    M = torch.zeros(mc, H, D, D, device="cuda") if lm else None
    ws = torch.empty(gdr.gdr_chunk_prefill_workspace_bytes(T, N, H, D, D, C, gdr.GDR_BF16),
                     dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def call():
        gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"],
                              di["state0"], so, o, chunk=C, L_out=L, M_out=M, workspace=ws,
                              stream=stream)
    return call, [x for x in (o, so, L, M) if x is not None]


def test_prefills_and_decode_on_three_streams():
    import gated_delta_rule_100_amd as gdr
    da = workload(2, seed=960, seqlens=[700, 64, 1, 300], H=8, gate="slow")
    db = workload(3, seed=961, seqlens=[4000, 90, 0, 1500], H=4)
    dd = workload(1, seed=962, seqlens=[1] * 32, H=8)
    dia, dib, did = dev_inputs(da), dev_inputs(db), dev_inputs(dd)
    streams = [torch.cuda.Stream() for _ in range(3)]
    say("two prefills and a decode step on three streams at once")

    # alone, in turn
    ca, outa = _prefill(gdr, da, dia, lm=False)
    cb, outb = _prefill(gdr, db, dib, lm=True)
    s0 = did["state0"].clone()
    od = torch.empty(32, 8, 128, dtype=torch.bfloat16, device="cuda")
    ca()
    torch.cuda.synchronize()
    cb()
    torch.cuda.synchronize()
    gdr.gdr_decode_step(did["q"], did["k"], did["v"], did["g"], did["beta"], did["state0"], od)
    torch.cuda.synchronize()
    ref = [x.clone() for x in outa + outb] + [od.clone(), did["state0"].clone()]

    # at once
    for x in outa + outb + [od]:
        x.fill_(float("nan"))
    did["state0"].copy_(s0)
    ca2, outa2 = _prefill(gdr, da, dia, lm=False, stream=streams[0])
    cb2, outb2 = _prefill(gdr, db, dib, lm=True, stream=streams[1])
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    ca2()
    cb2()
    gdr.gdr_decode_step(did["q"], did["k"], did["v"], did["g"], did["beta"], did["state0"], od,
                        stream=streams[2])
    torch.cuda.synchronize()
    got = outa2 + outb2 + [od, did["state0"]]
    for i, (x, y) in enumerate(zip(got, ref)):
        assert torch.equal(x, y), i
