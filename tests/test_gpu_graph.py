"""The entry points captured in a HIP graph and replayed.

The library allocates, frees and synchronises nothing and records no memory
set, so its calls can be captured.  Each test runs the calls eagerly once
(which also fills the per-device caches: device properties, the static
scratch's address), captures the same calls into a graph with torch's capture
API, then replays the graph several times with eager work and synchronisation
between the replays, and checks every replay bit for bit against the eager
result (the kernels are deterministic).  The inputs are refilled between
replays, so a replay that silently reused the previous result would fail."""
import pytest
import torch

from gdr_synth import workload
from gpu_util import dev_inputs, say

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _prefill_case():
    d = workload(3, seed=950, seqlens=[300, 1, 64, 129, 0, 77], H=4, gate="slow")
    return d, dev_inputs(d)


def _check_replays(graph, refill, outputs, expected):
    for r in range(REPLAYS):
        refill(r)
        torch.cuda.synchronize()
        # eager work on the same stream between replays
        junk = torch.full((1 << 20,), float(r), device="cuda") * 2.0
        graph.replay()
        torch.cuda.synchronize()
        del junk
        for name, (got, ref) in enumerate(zip(outputs, expected[r % 2])):
            assert torch.equal(got, ref), (r, name)


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_prefill_in_graph(entry):
    import gated_delta_rule_100_amd as gdr
    d, di = _prefill_case()
    say(f"prefill captured in a graph ({entry}), {REPLAYS} replays")
    T, H, D, N, C = d["T"], d["H"], d["dk"], d["N"], d["chunk"]
    o = torch.empty(T, H, D, device="cuda")
    sout = torch.empty(N, H, D, D, device="cuda")
    mc = gdr.gdr_max_chunks(T, N, C)
    F = torch.zeros(mc, H, D, D, device="cuda")  # slots past the batch's chunks stay zero
    ws = torch.empty(gdr.gdr_chunk_prefill_workspace_bytes(T, N, H, D, D, C, gdr.GDR_BF16),
                     dtype=torch.uint8, device="cuda")
    q0, v0 = di["q"].clone(), di["v"].clone()
    v1 = (di["v"].float() * -0.5).to(torch.bfloat16)  # the second input set

    def call(stream=None):
        if entry == "workspace":
            gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"],
                                  di["state0"], sout, o, chunk=C, fixed_out=F, workspace=ws,
                                  stream=stream)
        else:
            gdr.gdr_chunk_prefill_noalloc(di["q"], di["k"], di["v"], di["g"], di["beta"],
                                          di["cu"], di["state0"], sout, o, chunk=C, fixed_out=F,
                                          stream=stream)

    expected = []
    for vv in (v0, v1):  # eager results for both input sets
        di["v"].copy_(vv)
        call()
        torch.cuda.synchronize()
        expected.append((o.clone(), sout.clone(), F.clone()))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        call(stream=s)
    torch.cuda.synchronize()

    def refill(r):
        di["v"].copy_(v0 if r % 2 == 0 else v1)
        di["q"].copy_(q0)

    _check_replays(g, refill, (o, sout, F), expected)


def test_decode_in_graph():
    import gated_delta_rule_100_amd as gdr
    d = workload(1, seed=951, seqlens=[1] * 16, H=8)
    di = dev_inputs(d)
    say(f"decode step captured in a graph, {REPLAYS} replays")
    s0 = di["state0"].clone()
    st = s0.clone()
    o = torch.empty(16, 8, 128, device="cuda")
    expected = []
    gb = di["g"].clone()
    for gg in (gb, gb * 0.5):
        st.copy_(s0)
        di["g"].copy_(gg)
        gdr.gdr_decode_step(di["q"], di["k"], di["v"], di["g"], di["beta"], st, o)
        torch.cuda.synchronize()
        expected.append((o.clone(), st.clone()))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        gdr.gdr_decode_step(di["q"], di["k"], di["v"], di["g"], di["beta"], st, o, stream=s)
    torch.cuda.synchronize()

    def refill(r):
        st.copy_(s0)  # the state is updated in place: restart it
        di["g"].copy_(gb if r % 2 == 0 else gb * 0.5)

    _check_replays(g, refill, (o, st), expected)


@pytest.mark.parametrize("T, inter", [(8, False), (20, False), (3, True)])
def test_decode_mtp_in_graph(T, inter):
    # without per-token states the chunked kernel (T = 20: three chunks, the
    # next chunk's rows copied in while one is applied), with them (T = 3) the
    # token-by-token one
    import gated_delta_rule_100_amd as gdr
    from gdr_synth import generate
    N, H, D = 8, 4, 128
    data = generate([T] * N, H, D, D, dtype="bf16", state0=True, seed=952, gate="slow")
    di = dev_inputs(data)
    q, k, v = (di[x].view(N, T, H, D) for x in ("q", "k", "v"))
    g, b = di["g"].view(N, T, H), di["beta"].view(N, T, H)
    say(f"multi-token decode T={T} captured in a graph, {REPLAYS} replays")
    s0 = di["state0"].clone()
    st = s0.clone()
    o = torch.empty(N, T, H, D, device="cuda")
    I = torch.empty(N, T, H, D, D, device="cuda") if inter else None
    gb = g.clone()
    expected = []
    for gg in (gb, gb * 0.5):
        st.copy_(s0)
        g.copy_(gg)
        gdr.gdr_decode_mtp(q, k, v, g, b, st, st, o, I)
        torch.cuda.synchronize()
        expected.append((o.clone(), st.clone()) + ((I.clone(),) if inter else ()))
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=s):
        gdr.gdr_decode_mtp(q, k, v, g, b, st, st, o, I, stream=s)
    torch.cuda.synchronize()

    def refill(r):
        st.copy_(s0)  # updated in place: restart it
        g.copy_(gb if r % 2 == 0 else gb * 0.5)

    _check_replays(graph, refill, (o, st) + ((I,) if inter else ()), expected)
