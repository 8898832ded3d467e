"""Batches with tensors of more than 2^31 elements, so that offsets past the
boundary need 64-bit arithmetic:
  - a state of more than 131072 (sequence, head) pairs at d = 128 (9.1 GB of
    fp32 state) under decode, chunked multi-token decode and prefill;
  - a prefill whose q, k, v and o hold more than 2^31 elements (token rows past
    524288 at 32 heads).
Sampled pairs on both sides of the boundary are checked against the oracle,
run on that pair alone (bf16 inputs: max|gpu - ref| / max|ref| <= 1e-3).
The large tensors are drawn on the device from seeded generators; the host
keeps copies of the sampled pairs only."""
import numpy as np
import pytest
import torch

import oracle
from gdr_synth import generate
from gpu_util import BF16_TOL, FP32_TOL, dev_inputs, host64, rel_err, say

pytestmark = pytest.mark.gpu

N, H, D = 4352, 32, 128          # 139264 pairs: 2.28e9 state elements
PAIRS = [(0, 0), (2048, 17), (4095, 31), (4096, 1), (4200, 9), (N - 1, H - 1)]


def big_state(seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    s = torch.randn(N, H, D, D, generator=gen, device="cuda", dtype=torch.float32)
    return s.mul_(0.02)


def pair_problem(d, n, h, tokens, s0):
    """The inputs of one (sequence, head) pair as a one-sequence, one-head batch."""
    a, b = int(d["cu_seqlens"][n]), int(d["cu_seqlens"][n + 1])
    assert b - a == tokens
    sub = {key: np.ascontiguousarray(d[key][a:b, h:h + 1]) for key in ("q", "k", "v", "g", "beta")}
    return oracle.recurrent(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"],
                            np.array([0, tokens]), s0[None, None])


def check(d, tokens, s0_host, o, s_new, label):
    for (n, h) in PAIRS:
        o_ref, s_ref, _ = pair_problem(d, n, h, tokens, s0_host[(n, h)])
        a = int(d["cu_seqlens"][n])
        e_o = rel_err(host64(o[a:a + tokens, h]), o_ref[:, 0])
        e_s = rel_err(host64(s_new[n, h]), s_ref[0, 0])
        say(f"  {label} pair ({n},{h}) offset {(n * H + h) * D * D:.3e}: o {e_o:.2e} state {e_s:.2e}")
        assert e_o <= BF16_TOL and e_s <= BF16_TOL, (label, n, h, e_o, e_s)


def test_decode_state_past_2_31_elements():
    import gated_delta_rule_100_amd as gdr
    say(f"decode N={N} H={H} d={D}: state of {N * H * D * D:.3e} elements")
    d = generate([1] * N, H, D, D, dtype="bf16", state0=False, seed=700)
    di = dev_inputs(d)
    state = big_state(701)
    s0 = {p: host64(state[p[0], p[1]]) for p in PAIRS}
    o = torch.empty(N, H, D, dtype=torch.float32, device="cuda")
    gdr.gdr_decode_step(di["q"], di["k"], di["v"], di["g"], di["beta"], state, o)
    torch.cuda.synchronize()
    check(d, 1, s0, o, state, "decode")
    del state
    torch.cuda.empty_cache()


def test_mtp_chunked_state_past_2_31_elements():
    import gated_delta_rule_100_amd as gdr
    T = 5
    say(f"multi-token decode (chunked) N={N} T={T} H={H} d={D}, in place")
    d = generate([T] * N, H, D, D, dtype="bf16", state0=False, seed=710)
    di = dev_inputs(d)
    x = {key: di[key].view(N, T, H, -1) for key in ("q", "k", "v")}
    state = big_state(711)
    s0 = {p: host64(state[p[0], p[1]]) for p in PAIRS}
    o = torch.empty(N, T, H, D, dtype=torch.float32, device="cuda")
    gdr.gdr_decode_mtp(x["q"], x["k"], x["v"], di["g"].view(N, T, H), di["beta"].view(N, T, H),
                       state, state, o, None)
    torch.cuda.synchronize()
    check(d, T, s0, o.view(N * T, H, D), state, "mtp")
    del state
    torch.cuda.empty_cache()


def test_prefill_state_past_2_31_elements():
    import gated_delta_rule_100_amd as gdr
    T = 2
    say(f"prefill N={N} sequences of {T} tokens, H={H} d={D}: states of {N * H * D * D:.3e} elements")
    d = generate([T] * N, H, D, D, dtype="bf16", state0=False, seed=720)
    di = dev_inputs(d)
    state_in = big_state(721)
    s0 = {p: host64(state_in[p[0], p[1]]) for p in PAIRS}
    state_out = torch.empty_like(state_in)
    o = torch.empty(N * T, H, D, dtype=torch.float32, device="cuda")
    gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"], state_in,
                          state_out, o, chunk=64)
    torch.cuda.synchronize()
    check(d, T, s0, o, state_out, "prefill")
    del state_in, state_out
    torch.cuda.empty_cache()


def test_prefill_tokens_past_2_31_elements():
    # 560 sequences of 1000 tokens, 32 heads: q, k, v and o hold 2.29e9 elements,
    # so token rows past 524288 sit beyond 2^31 elements.  Inputs are drawn on
    # the device from a seeded generator (q, k L2-normalised per token, v
    # N(0,1), g = -softplus(N(0,1)), beta = sigmoid(N(0,1)), S0 = 0); the host
    # copies the sampled pairs' tokens only.
    import gated_delta_rule_100_amd as gdr
    Nn, L, Hh = 560, 1000, 32
    T = Nn * L
    say(f"prefill {Nn} sequences of {L} tokens, H={Hh} d={D}: q/k/v/o of {T * Hh * D:.3e} elements")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(730)

    def unit_rows():
        x = torch.randn(T, Hh, D, generator=gen, device="cuda")
        x /= x.norm(dim=-1, keepdim=True)
        return x.to(torch.bfloat16)

    q, k = unit_rows(), unit_rows()
    v = torch.randn(T, Hh, D, generator=gen, device="cuda").to(torch.bfloat16)
    g = -torch.nn.functional.softplus(torch.randn(T, Hh, generator=gen, device="cuda"))
    beta = torch.sigmoid(torch.randn(T, Hh, generator=gen, device="cuda"))
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device="cuda")
    state_out = torch.empty(Nn, Hh, D, D, device="cuda")
    o = torch.empty(T, Hh, D, dtype=torch.float32, device="cuda")
    gdr.gdr_chunk_prefill(q, k, v, g, beta, cu, None, state_out, o, chunk=64)
    torch.cuda.synchronize()

    def bits(t):
        return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    for n, h in [(0, 0), (300, 5), (524, 31), (540, 16), (Nn - 1, Hh - 1)]:
        a, b = n * L, (n + 1) * L
        sl = (slice(a, b), slice(h, h + 1))
        o_ref, s_ref, _ = oracle.recurrent(
            bits(q[sl]), bits(k[sl]), bits(v[sl]), g[sl].contiguous().cpu().numpy(),
            beta[sl].contiguous().cpu().numpy(), np.array([0, L]))
        e_o = rel_err(host64(o[a:b, h]), o_ref[:, 0])
        e_s = rel_err(host64(state_out[n, h]), s_ref[0, 0])
        say(f"  pair ({n},{h}) last token offset {((b - 1) * Hh + h) * D:.3e}: o {e_o:.2e} state {e_s:.2e}")
        assert e_o <= BF16_TOL and e_s <= BF16_TOL, (n, h, e_o, e_s)
    del q, k, v, o, state_out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_chunk_states_past_2_31_elements(dt):
    # L and M requested on 4 sequences of 67200 tokens at 32 heads: L, M and
    # the fixed states hold 4204 chunk slots x 32 heads x 128 x 128 = 2.2e9
    # elements each, so the chunks past slot 4096 sit beyond 2^31.  bf16
    # inputs take the scan (L and M from the chunk-local kernel); fp32 inputs
    # the chunk-parallel form (chunk-local, dense fixup, chunk outputs).
    # Inputs drawn on the device from a seeded generator (the recipe of the
    # token test above, S0 = 0).  The last sequence is checked against the
    # oracle run on two of its heads: outputs, final state and the fixed
    # states of its last chunks (slots past 4096), and L and M of its last
    # chunk against the chunked oracle.
    import gated_delta_rule_100_amd as gdr
    Nn, L, Hh, C = 4, 67200, 32, 64
    T = Nn * L
    mc = gdr.gdr_max_chunks(T, Nn, C)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    tol = BF16_TOL if dt == "bf16" else FP32_TOL
    say(f"prefill {Nn} x {L} tokens, H={Hh}, {dt}: L/M/fixed of {mc * Hh * D * D:.3e} elements")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(740)

    def unit_rows():
        x = torch.randn(T, Hh, D, generator=gen, device="cuda")
        x /= x.norm(dim=-1, keepdim=True)
        return x.to(tdt)

    q, k = unit_rows(), unit_rows()
    v = torch.randn(T, Hh, D, generator=gen, device="cuda").to(tdt)
    g = -torch.nn.functional.softplus(torch.randn(T, Hh, generator=gen, device="cuda"))
    beta = torch.sigmoid(torch.randn(T, Hh, generator=gen, device="cuda"))
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device="cuda")
    state_out = torch.empty(Nn, Hh, D, D, device="cuda")
    o = torch.empty(T, Hh, D, dtype=torch.float32, device="cuda")
    Lo = torch.empty(mc, Hh, D, D, device="cuda")
    Mo = torch.empty(mc, Hh, D, D, device="cuda")
    F = torch.empty(mc, Hh, D, D, device="cuda")
    gdr.gdr_chunk_prefill(q, k, v, g, beta, cu, None, state_out, o, chunk=C, L_out=Lo, M_out=Mo,
                          fixed_out=F)
    torch.cuda.synchronize()

    def host(t):
        t = t.contiguous().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    n = Nn - 1
    a, b = n * L, (n + 1) * L
    c0 = n * (L // C)                     # the sequence's first chunk slot
    nch = L // C
    for h in (0, Hh - 1):
        sl = (slice(a, b), slice(h, h + 1))
        o_ref, s_ref, cs_ref = oracle.recurrent(
            host(q[sl]), host(k[sl]), host(v[sl]), g[sl].contiguous().cpu().numpy(),
            beta[sl].contiguous().cpu().numpy(), np.array([0, L]), chunk=C)
        e_o = rel_err(host64(o[a:b, h]), o_ref[:, 0])
        e_s = rel_err(host64(state_out[n, h]), s_ref[0, 0])
        last = slice(c0 + nch - 8, c0 + nch)
        e_f = rel_err(host64(F[last, h]), cs_ref[nch - 8:nch, 0])
        lo = b - C
        loc = oracle.chunk_local(oracle.as_f64(host(k[lo:b, h])), oracle.as_f64(host(v[lo:b, h])),
                                 g[lo:b, h].double().cpu().numpy(),
                                 beta[lo:b, h].double().cpu().numpy())
        e_l = rel_err(host64(Lo[c0 + nch - 1, h]), loc["L"])
        e_m = rel_err(host64(Mo[c0 + nch - 1, h]), loc["M"])
        say(f"  pair ({n},{h}) last slot offset {((c0 + nch - 1) * Hh + h) * D * D:.3e}: "
            f"o {e_o:.2e} state {e_s:.2e} fixed {e_f:.2e} L {e_l:.2e} M {e_m:.2e}")
        assert max(e_o, e_s, e_f, e_l, e_m) <= tol, (h, e_o, e_s, e_f, e_l, e_m)
    del q, k, v, o, state_out, F, Lo, Mo
    torch.cuda.empty_cache()
