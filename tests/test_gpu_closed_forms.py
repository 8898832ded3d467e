"""GPU results against closed forms of the recurrence, computed here in fp64
from the inputs (not by the oracle):
  - beta = 0 and alpha = 1 (g = 0): every step is the identity, so the state
    must come back unchanged bit for bit, and o_t = S_0 q_t;
  - S_0 = 0 and mutually orthogonal keys (a sequence no longer than dk): the
    erase term S_{t-1} k_t vanishes, so with G the running sum of g
        S_T = sum_s beta_s e^{G_T - G_s} v_s k_s^T,
        o_t = sum_{s<=t} beta_s e^{G_t - G_s} (k_s . q_t) v_s.
  - beta = 0 with any gates (pure decay): S_t = e^{G_t} S_0 and
    o_t = e^{G_t} S_0 q_t.
Keys for the orthogonal case are signed one-hot rows under a random permutation
per (sequence, head): orthonormal and exact in bf16.  Every entry point runs
both cases: decode (token by token), multi-token decode (chunked and token by
token), and prefill under both schedules; the fixup scan on its own is checked
with scaled-identity transfer matrices.  Outputs are fp32;
max|gpu - ref| / max|ref| <= 1e-3 (bf16 inputs) or 1e-5 (fp32 inputs)."""
import numpy as np
import pytest
import torch

from gdr_synth import bf16_bits_from_f32, generate
from gpu_util import dev_inputs, host64, rel_err, say, tol_for

pytestmark = pytest.mark.gpu


def f64(x):
    """Input array as fp64 (bf16 bits widen exactly)."""
    if x.dtype == np.uint16:
        return np.left_shift(x.astype(np.uint32), 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def onehot_keys(d, seed):
    """Replace k by signed one-hot rows, a fresh permutation per (sequence, head)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, H, dk = d["T"], d["H"], d["dk"]
    k = np.zeros((T, H, dk), dtype=np.float32)
    cu = d["cu_seqlens"]
    for n in range(d["N"]):
        a, b = int(cu[n]), int(cu[n + 1])
        assert b - a <= dk
        for h in range(H):
            cols = rng.permutation(dk)[:b - a]
            k[np.arange(a, b), h, cols] = rng.choice([-1.0, 1.0], size=b - a)
    d["k"] = bf16_bits_from_f32(k) if d["dtype"] == "bf16" else k


def orthogonal_closed_form(d):
    q, k, v = f64(d["q"]), f64(d["k"]), f64(d["v"])
    g, beta = d["g"].astype(np.float64), d["beta"].astype(np.float64)
    cu = d["cu_seqlens"]
    o = np.zeros_like(v)
    S = np.zeros((d["N"], d["H"], d["dv"], d["dk"]))
    for n in range(d["N"]):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:
            continue
        for h in range(d["H"]):
            G = np.cumsum(g[a:b, h])
            K, V, Q, B = k[a:b, h], v[a:b, h], q[a:b, h], beta[a:b, h]
            decay = np.exp(np.tril(G[:, None] - G[None, :])) * np.tri(b - a)
            o[a:b, h] = (decay * B[None, :] * (Q @ K.T)) @ V
            S[n, h] = (V * (B * np.exp(G[-1] - G))[:, None]).T @ K
    return o, S


def identity_inputs(d):
    d["beta"][:] = 0.0
    d["g"][:] = 0.0


def identity_outputs(d):
    """o_t = S_0 q_t for the identity case."""
    q = f64(d["q"])
    o = np.zeros((d["T"], d["H"], d["dv"]))
    cu = d["cu_seqlens"]
    for n in range(d["N"]):
        a, b = int(cu[n]), int(cu[n + 1])
        o[a:b] = np.einsum("hij,thj->thi", d["state0"][n].astype(np.float64), q[a:b])
    return o


def decay_closed_form(d):
    """beta = 0: o_t = e^{G_t} S_0 q_t and S_T = e^{G_T} S_0 per sequence."""
    q = f64(d["q"])
    g = d["g"].astype(np.float64)
    cu = d["cu_seqlens"]
    o = np.zeros((d["T"], d["H"], d["dv"]))
    S = d["state0"].astype(np.float64).copy()
    for n in range(d["N"]):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:
            continue
        G = np.cumsum(g[a:b], axis=0)                       # [t, h]
        s0 = d["state0"][n].astype(np.float64)
        o[a:b] = np.exp(G)[:, :, None] * np.einsum("hij,thj->thi", s0, q[a:b])
        S[n] = np.exp(G[-1])[:, None, None] * s0
    return o, S


# ---- prefill (both schedules) ----

# name: (sequence lengths, H, d, dtype, chunk); fp32 inputs take the
# chunk-parallel form at either chunk size.  The orthogonal-key test clips each
# length to d.
PREFILL = {
    "bf16-ragged": ([128, 64, 1, 100, 0, 77], 3, 128, "bf16", 64),
    "bf16-d64": ([64, 30, 65, 129], 2, 64, "bf16", 64),
    "f32-ragged-C16": ([128, 17, 0, 90], 2, 128, "f32", 16),
    "f32-ragged-C64": ([128, 17, 0, 90], 2, 128, "f32", 64),
}


def run_prefill(d, keep_lm, chunk):
    import gated_delta_rule_100_amd as gdr
    di = dev_inputs(d)
    T, H, D, N = d["T"], d["H"], d["dk"], d["N"]
    o = torch.full((T, H, D), float("nan"), device="cuda")
    sout = torch.full((N, H, D, D), float("nan"), device="cuda")
    L = M = None
    if keep_lm:  # asking for L and M selects the chunk-parallel schedule
        mc = gdr.gdr_max_chunks(T, N, chunk)
        L = torch.empty(mc, H, D, D, device="cuda")
        M = torch.empty(mc, H, D, D, device="cuda")
    gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"], di["state0"],
                          sout, o, chunk=chunk, L_out=L, M_out=M)
    torch.cuda.synchronize()
    return o, sout


@pytest.mark.parametrize("keep_lm", [False, True], ids=["scan", "chunk-parallel"])
@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_identity_steps(name, keep_lm):
    lens, H, dd, dtype, chunk = PREFILL[name]
    say(f"prefill identity steps {name} {'chunk-parallel' if keep_lm else 'scan'}")
    d = generate(lens, H, dd, dd, dtype=dtype, state0=True, seed=800)
    identity_inputs(d)
    o, sout = run_prefill(d, keep_lm, chunk)
    s0 = torch.from_numpy(d["state0"]).cuda()
    if chunk != 64 or dtype == "f32":
        # the chunk-parallel schedule (chunk 16 and fp32 inputs) multiplies by
        # M = I on bf16 planes: equal to rounding
        assert rel_err(host64(sout), d["state0"]) <= tol_for(d)
    else:
        assert torch.equal(sout, s0), "the state must come back unchanged"
    assert rel_err(host64(o), identity_outputs(d)) <= tol_for(d)


@pytest.mark.parametrize("keep_lm", [False, True], ids=["scan", "chunk-parallel"])
@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_orthogonal_keys(name, keep_lm):
    lens, H, dd, dtype, chunk = PREFILL[name]
    say(f"prefill orthogonal keys {name} {'chunk-parallel' if keep_lm else 'scan'}")
    d = generate([min(x, dd) for x in lens], H, dd, dd, dtype=dtype, state0=False, seed=810)
    onehot_keys(d, 811)
    o, sout = run_prefill(d, keep_lm, chunk)
    o_ref, s_ref = orthogonal_closed_form(d)
    e_o, e_s = rel_err(host64(o), o_ref), rel_err(host64(sout), s_ref)
    say(f"  o {e_o:.2e} state {e_s:.2e}")
    assert e_o <= tol_for(d) and e_s <= tol_for(d)


@pytest.mark.parametrize("keep_lm", [False, True], ids=["scan", "chunk-parallel"])
@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_pure_decay(name, keep_lm):
    lens, H, dd, dtype, chunk = PREFILL[name]
    say(f"prefill pure decay {name} {'chunk-parallel' if keep_lm else 'scan'}")
    d = generate(lens, H, dd, dd, dtype=dtype, state0=True, seed=840, gate="slow")
    d["beta"][:] = 0.0
    o, sout = run_prefill(d, keep_lm, chunk)
    o_ref, s_ref = decay_closed_form(d)
    e_o, e_s = rel_err(host64(o), o_ref), rel_err(host64(sout), s_ref)
    say(f"  o {e_o:.2e} state {e_s:.2e}")
    assert e_o <= tol_for(d) and e_s <= tol_for(d)


# ---- decode and multi-token decode ----

def decode_chain(d, L):
    """The batch's N sequences of L tokens, one gdr_decode_step per token."""
    import gated_delta_rule_100_amd as gdr
    di = dev_inputs(d)
    N, H, D = d["N"], d["H"], d["dk"]
    state = (di["state0"].clone() if di["state0"] is not None
             else torch.zeros(N, H, D, D, device="cuda"))
    x = {key: di[key].view(N, L, H, -1) for key in ("q", "k", "v")}
    gb = {key: di[key].view(N, L, H) for key in ("g", "beta")}
    o = torch.empty(N, L, H, D, device="cuda")
    for t in range(L):
        sub = {key: x[key][:, t].contiguous() for key in x}
        ot = torch.empty(N, H, D, device="cuda")
        gdr.gdr_decode_step(sub["q"], sub["k"], sub["v"], gb["g"][:, t].contiguous(),
                            gb["beta"][:, t].contiguous(), state, ot)
        o[:, t] = ot
    torch.cuda.synchronize()
    return o.view(N * L, H, D), state


def mtp(d, L, inter):
    import gated_delta_rule_100_amd as gdr
    di = dev_inputs(d)
    N, H, D = d["N"], d["H"], d["dk"]
    state = (di["state0"].clone() if di["state0"] is not None
             else torch.zeros(N, H, D, D, device="cuda"))
    x = {key: di[key].view(N, L, H, -1) for key in ("q", "k", "v")}
    o = torch.empty(N, L, H, D, device="cuda")
    I = torch.empty(N, L, H, D, D, device="cuda") if inter else None
    gdr.gdr_decode_mtp(x["q"], x["k"], x["v"], di["g"].view(N, L, H), di["beta"].view(N, L, H),
                       state, state, o, I)
    torch.cuda.synchronize()
    return o.view(N * L, H, D), state


DECODE = {
    # name: (N, tokens per sequence, H, d, dtype, path)
    "chain-bf16-d128": (3, 24, 2, 128, "bf16", "chain"),
    "chain-f32-d64": (2, 16, 2, 64, "f32", "chain"),
    "mtp-chunked-bf16-T8": (4, 8, 3, 128, "bf16", "mtp"),
    "mtp-chunked-f32-T5": (3, 5, 2, 64, "f32", "mtp"),
    "mtp-tokens-bf16-T4": (3, 4, 2, 128, "bf16", "mtp-inter"),
}


def run_decode_case(d, L, path):
    if path == "chain":
        return decode_chain(d, L)
    return mtp(d, L, inter=path == "mtp-inter")


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_identity_steps(name):
    N, L, H, dd, dtype, path = DECODE[name]
    say(f"decode identity steps {name}")
    d = generate([L] * N, H, dd, dd, dtype=dtype, state0=True, seed=820)
    identity_inputs(d)
    o, state = run_decode_case(d, L, path)
    assert torch.equal(state, torch.from_numpy(d["state0"]).cuda()), "the state must come back unchanged"
    assert rel_err(host64(o), identity_outputs(d)) <= tol_for(d)


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_orthogonal_keys(name):
    N, L, H, dd, dtype, path = DECODE[name]
    say(f"decode orthogonal keys {name}")
    d = generate([L] * N, H, dd, dd, dtype=dtype, state0=False, seed=830)
    onehot_keys(d, 831)
    o, state = run_decode_case(d, L, path)
    o_ref, s_ref = orthogonal_closed_form(d)
    e_o, e_s = rel_err(host64(o), o_ref), rel_err(host64(state), s_ref)
    say(f"  o {e_o:.2e} state {e_s:.2e}")
    assert e_o <= tol_for(d) and e_s <= tol_for(d)


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_pure_decay(name):
    N, L, H, dd, dtype, path = DECODE[name]
    say(f"decode pure decay {name}")
    d = generate([L] * N, H, dd, dd, dtype=dtype, state0=True, seed=850)
    d["beta"][:] = 0.0
    o, state = run_decode_case(d, L, path)
    o_ref, s_ref = decay_closed_form(d)
    e_o, e_s = rel_err(host64(o), o_ref), rel_err(host64(state), s_ref)
    say(f"  o {e_o:.2e} state {e_s:.2e}")
    assert e_o <= tol_for(d) and e_s <= tol_for(d)


# ---- the fixup scan on its own ----

@pytest.mark.parametrize("with_state", [True, False])
@pytest.mark.parametrize("D,H,chunks", [(128, 3, [5, 0, 40, 1]), (64, 2, [300, 7]),
                                        (128, 1, [600])])  # one long chain
def test_fixup_scaled_identity_transfer(with_state, D, H, chunks):
    """gdr_state_fixup with M_c = a_c I: fixed[c] = a_c fixed[c-1] + L_c, a
    running sum (fixed[first] = L when there is no initial state)."""
    import gated_delta_rule_100_amd as gdr
    say(f"fixup scaled identity D={D} H={H} chunks={chunks} with_state={with_state}")
    rng = np.random.Generator(np.random.PCG64(860 + D))
    offs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    nch = int(offs[-1])
    L = rng.standard_normal((nch, H, D, D)).astype(np.float32)
    a = np.exp(-rng.random((nch, H))).astype(np.float32)          # in (1/e, 1]
    M = np.zeros((nch, H, D, D), dtype=np.float32)
    M[:, :, np.arange(D), np.arange(D)] = a[:, :, None]             # symmetric: layout-free
    s0 = (0.5 * rng.standard_normal((len(chunks), H, D, D))).astype(np.float32)
    fixed = torch.full((nch, H, D, D), float("nan"), device="cuda")
    gdr.gdr_state_fixup(torch.from_numpy(L).cuda(), torch.from_numpy(M).cuda(),
                        torch.from_numpy(s0).cuda() if with_state else None,
                        torch.from_numpy(offs).cuda(), fixed)
    torch.cuda.synchronize()
    ref = np.zeros((nch, H, D, D))
    for n in range(len(chunks)):
        prev = s0[n].astype(np.float64) if with_state else None
        for c in range(int(offs[n]), int(offs[n + 1])):
            if prev is None:
                ref[c] = L[c]
            else:
                ref[c] = a[c].astype(np.float64)[:, None, None] * prev + L[c]
            prev = ref[c]
    e = rel_err(host64(fixed), ref)
    say(f"  fixed {e:.2e}")
    assert e <= 1e-5
