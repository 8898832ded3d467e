"""Pins for the fp64 oracle: every check here compares the oracle with
something other than itself -- closed forms, brute-force matrix products,
exact invariants -- chosen so that a dropped term, a wrong sign or index or a
transposed operand in O1 (recurrent, C) or O2 (chunked, numpy) fails.

Closed forms used (all exact in exact arithmetic):
  * beta = 0 (pure decay):      S_t = exp(G_t) S_0, o_t = exp(G_t) S_0 q_t
  * beta = 0, alpha = 1:        S_t = S_0
  * alpha = 1, S_0 = 0, orthonormal keys: S_T = sum_s beta_s v_s k_s^T,
                                o_t = sum_{s<=t} beta_s v_s (k_s . q_t)
  * orthonormal keys, any gates:
        S_T = gamma_T S_0 (I - sum_s beta_s k_s k_s^T) + sum_s (gamma_T/gamma_s) beta_s v_s k_s^T
    and with beta = 1: S_t k_t = v_t after every step, S_T k_s = (gamma_T/gamma_s) v_s.
  * brute force: S_T = S_0 Phi_1..Phi_T + sum_s beta_s v_s k_s^T Phi_{s+1}..Phi_T,
    Phi_t = alpha_t (I - beta_t k_t k_t^T)  (dense products, tiny sizes)
"""
import numpy as np
import pytest

import oracle
from gdr_synth import generate


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = np.max(np.abs(b))
    if scale == 0:
        return float(np.max(np.abs(a)))
    return float(np.max(np.abs(a - b)) / scale)


def rand_problem(rng, seqlens, H, dk, dv, state0=True, gmin=-2.0):
    T = int(sum(seqlens))
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = rng.uniform(gmin, 0.0, size=(T, H))
    beta = rng.uniform(0.0, 1.0, size=(T, H))
    s0 = rng.standard_normal((len(seqlens), H, dv, dk)) if state0 else None
    return q, k, v, g, beta, cu, s0


def orthonormal_keys(rng, T, dk):
    qm, _ = np.linalg.qr(rng.standard_normal((dk, T)))
    return qm.T.copy()  # rows orthonormal


# --------------------------------------------------------------------------
# T1: brute force on tiny problems


@pytest.mark.parametrize("dk,dv", [(2, 2), (3, 2), (4, 3), (8, 8), (3, 5)])
def test_T1_recurrent_equals_bruteforce_product(dk, dv):
    rng = np.random.default_rng(1000 + dk * 10 + dv)
    for T in (1, 2, 5, 8):
        q, k, v, g, beta, cu, s0 = rand_problem(rng, [T], 1, dk, dv)
        o, sT, _ = oracle.recurrent(q, k, v, g, beta, cu, s0)
        ref = oracle.state_bruteforce(s0[0, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0])
        assert rel_err(sT[0, 0], ref) < 1e-13
        for t in range(T):
            St = oracle.state_bruteforce(s0[0, 0], k[: t + 1, 0], v[: t + 1, 0],
                                         g[: t + 1, 0], beta[: t + 1, 0])
            assert rel_err(o[t, 0], St @ q[t, 0]) < 1e-13


def test_T1_chunk_local_equals_bruteforce_product():
    rng = np.random.default_rng(11)
    for dk, dv, c in ((2, 3, 1), (4, 4, 5), (8, 3, 8), (5, 7, 6)):
        _, k, v, g, beta, _, _ = rand_problem(rng, [c], 1, dk, dv, state0=False)
        loc = oracle.chunk_local(k[:, 0], v[:, 0], g[:, 0], beta[:, 0])
        assert rel_err(loc["M"], oracle.transfer_bruteforce(k[:, 0], g[:, 0], beta[:, 0])) < 1e-13
        L_ref = oracle.state_bruteforce(np.zeros((dv, dk)), k[:, 0], v[:, 0], g[:, 0], beta[:, 0])
        assert rel_err(loc["L"], L_ref) < 1e-13


# --------------------------------------------------------------------------
# T2: pure decay (beta = 0)


@pytest.mark.parametrize("chunk", [1, 16, 64])
def test_T2_pure_decay_closed_form(chunk):
    rng = np.random.default_rng(2)
    dk = dv = 16
    T = 50
    q, k, v, g, beta, cu, s0 = rand_problem(rng, [T], 2, dk, dv)
    beta[:] = 0.0
    g[:, 1] = -3.0  # head 1: G_T = -150, far below float32's exp range
    G = np.cumsum(g, axis=0)
    o, sT, _ = oracle.recurrent(q, k, v, g, beta, cu, s0)
    r = oracle.chunked(q, k, v, g, beta, cu, chunk, s0)
    for h in range(2):
        S_ref = np.exp(G[-1, h]) * s0[0, h]
        o_ref = np.exp(G[:, h])[:, None] * (q[:, h] @ s0[0, h].T)
        for got_s, got_o in ((sT, o), (r["state_out"], r["o"])):
            assert np.allclose(got_s[0, h], S_ref, rtol=1e-12, atol=1e-300)
            assert np.allclose(got_o[:, h], o_ref, rtol=1e-12, atol=1e-300)


# --------------------------------------------------------------------------
# T3a / T3b: identity and cumulative linear attention


def test_T3a_identity_when_beta0_alpha1():
    rng = np.random.default_rng(3)
    q, k, v, g, beta, cu, s0 = rand_problem(rng, [37], 2, 8, 6)
    beta[:] = 0.0
    g[:] = 0.0
    o, sT, _ = oracle.recurrent(q, k, v, g, beta, cu, s0)
    r = oracle.chunked(q, k, v, g, beta, cu, 16, s0)
    for h in range(2):
        for got_s, got_o in ((sT, o), (r["state_out"], r["o"])):
            assert rel_err(got_s[0, h], s0[0, h]) < 1e-14
            assert rel_err(got_o[:, h], q[:, h] @ s0[0, h].T) < 1e-14


def test_T3b_linear_attention_with_orthogonal_keys():
    rng = np.random.default_rng(4)
    dk, dv, T = 32, 8, 20
    q, k, v, g, beta, cu, _ = rand_problem(rng, [T], 1, dk, dv, state0=False)
    k[:, 0] = orthonormal_keys(rng, T, dk)
    g[:] = 0.0
    o, sT, _ = oracle.recurrent(q, k, v, g, beta, cu, None)
    r = oracle.chunked(q, k, v, g, beta, cu, 8, None)
    S_ref = sum(beta[s, 0] * np.outer(v[s, 0], k[s, 0]) for s in range(T))
    o_ref = np.stack([sum(beta[s, 0] * v[s, 0] * (k[s, 0] @ q[t, 0]) for s in range(t + 1))
                      for t in range(T)])
    for got_s, got_o in ((sT, o), (r["state_out"], r["o"])):
        assert rel_err(got_s[0, 0], S_ref) < 1e-13
        assert rel_err(got_o[:, 0], o_ref) < 1e-13
    # beta = 1: exactly the cumulative sum of v k^T
    beta[:] = 1.0
    _, sT1, _ = oracle.recurrent(q, k, v, g, beta, cu, None)
    assert rel_err(sT1[0, 0], sum(np.outer(v[s, 0], k[s, 0]) for s in range(T))) < 1e-13


# --------------------------------------------------------------------------
# T4: orthonormal keys, any gates


def test_T4_orthonormal_keys_closed_form():
    rng = np.random.default_rng(5)
    dk, dv, T = 16, 12, 16
    q, k, v, g, beta, cu, s0 = rand_problem(rng, [T], 1, dk, dv)
    k[:, 0] = orthonormal_keys(rng, T, dk)
    G = np.cumsum(g[:, 0])
    o, sT, _ = oracle.recurrent(q, k, v, g, beta, cu, s0)
    r = oracle.chunked(q, k, v, g, beta, cu, 4, s0)
    P = sum(beta[s, 0] * np.outer(k[s, 0], k[s, 0]) for s in range(T))
    S_ref = np.exp(G[-1]) * s0[0, 0] @ (np.eye(dk) - P)
    S_ref = S_ref + sum(np.exp(G[-1] - G[s]) * beta[s, 0] * np.outer(v[s, 0], k[s, 0])
                        for s in range(T))
    assert rel_err(sT[0, 0], S_ref) < 1e-13
    assert rel_err(r["state_out"][0, 0], S_ref) < 1e-13


def test_T4_beta1_writes_value_exactly():
    rng = np.random.default_rng(6)
    dk, dv, T = 16, 8, 12
    q, k, v, g, beta, cu, s0 = rand_problem(rng, [T], 1, dk, dv)
    k[:, 0] = orthonormal_keys(rng, T, dk)
    beta[:] = 1.0
    G = np.cumsum(g[:, 0])
    # after step t, S_t k_t = v_t: take q_t = k_t so o_t = S_t k_t
    q[:, 0] = k[:, 0]
    o, sT, _ = oracle.recurrent(q, k, v, g, beta, cu, s0)
    assert rel_err(o[:, 0], v[:, 0]) < 1e-13
    r = oracle.chunked(q, k, v, g, beta, cu, 5, s0)
    assert rel_err(r["o"][:, 0], v[:, 0]) < 1e-13
    for s in range(T):
        assert rel_err(sT[0, 0] @ k[s, 0], np.exp(G[-1] - G[s]) * v[s, 0]) < 1e-12


# --------------------------------------------------------------------------
# T5: recurrent == chunked, varlen with empty / length-1 / ragged sequences


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 64, 200])
def test_T5_recurrent_equals_chunked(chunk):
    rng = np.random.default_rng(50 + chunk)
    seqlens = [33, 0, 1, 64, 17, 0, 130]
    for state0 in (True, False):
        q, k, v, g, beta, cu, s0 = rand_problem(rng, seqlens, 2, 8, 6, state0=state0)
        o1, s1, _ = oracle.recurrent(q, k, v, g, beta, cu, s0)
        r = oracle.chunked(q, k, v, g, beta, cu, chunk, s0)
        assert rel_err(r["o"], o1) < 1e-12
        assert rel_err(r["state_out"], s1) < 1e-12


def test_T5_generated_inputs_all_dtypes():
    # bf16 and f32 encodings of the synthetic recipe, decoded by the oracle
    for dtype in ("bf16", "f32"):
        d = generate([40, 0, 25], 2, 16, 16, dtype=dtype, state0=True, seed=7)
        o1, s1, _ = oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                     d["cu_seqlens"], d["state0"])
        r = oracle.chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], 16,
                           d["state0"])
        assert rel_err(r["o"], o1) < 1e-12
        assert rel_err(r["state_out"], s1) < 1e-12


def test_T5_chunk1_is_one_step():
    rng = np.random.default_rng(8)
    dk, dv = 6, 4
    _, k, v, g, beta, _, _ = rand_problem(rng, [1], 1, dk, dv, state0=False)
    loc = oracle.chunk_local(k[:, 0], v[:, 0], g[:, 0], beta[:, 0])
    kt = k[0, 0]
    M_ref = np.exp(g[0, 0]) * (np.eye(dk) - beta[0, 0] * np.outer(kt, kt))
    L_ref = beta[0, 0] * np.outer(v[0, 0], kt)
    assert rel_err(loc["M"], M_ref) < 1e-15
    assert rel_err(loc["L"], L_ref) < 1e-15


# --------------------------------------------------------------------------
# T6: L and M


def test_T6_transfer_closed_form_orthonormal():
    rng = np.random.default_rng(9)
    dk, dv, c = 16, 8, 10
    _, k, v, g, beta, _, _ = rand_problem(rng, [c], 1, dk, dv, state0=False)
    k[:, 0] = orthonormal_keys(rng, c, dk)
    loc = oracle.chunk_local(k[:, 0], v[:, 0], g[:, 0], beta[:, 0])
    G = np.cumsum(g[:, 0])
    P = sum(beta[t, 0] * np.outer(k[t, 0], k[t, 0]) for t in range(c))
    assert rel_err(loc["M"], np.exp(G[-1]) * (np.eye(dk) - P)) < 1e-13


def test_T6_local_state_is_recurrence_from_zero():
    rng = np.random.default_rng(10)
    dk, dv, c = 12, 10, 16
    q, k, v, g, beta, cu, _ = rand_problem(rng, [c], 1, dk, dv, state0=False)
    loc = oracle.chunk_local(k[:, 0], v[:, 0], g[:, 0], beta[:, 0])
    _, sT, _ = oracle.recurrent(q, k, v, g, beta, cu, None)
    assert rel_err(loc["L"], sT[0, 0]) < 1e-13
    assert rel_err(loc["M"], oracle.transfer_bruteforce(k[:, 0], g[:, 0], beta[:, 0])) < 1e-13


# --------------------------------------------------------------------------
# T7: composition / resume


def test_T7_fixed_states_are_chunk_end_states():
    rng = np.random.default_rng(12)
    seqlens = [70, 5, 0, 128]
    for state0 in (True, False):
        q, k, v, g, beta, cu, s0 = rand_problem(rng, seqlens, 2, 8, 8, state0=state0)
        _, _, cs = oracle.recurrent(q, k, v, g, beta, cu, s0, chunk=16)
        r = oracle.chunked(q, k, v, g, beta, cu, 16, s0)
        assert cs.shape == r["fixed"].shape
        assert rel_err(r["fixed"], cs) < 1e-12


def test_T7_split_prefill_resumes_exactly():
    rng = np.random.default_rng(13)
    T1, T2 = 45, 38
    q, k, v, g, beta, cu, s0 = rand_problem(rng, [T1 + T2], 2, 8, 8)
    o_full, s_full, _ = oracle.recurrent(q, k, v, g, beta, cu, s0)
    cu1 = np.array([0, T1])
    cu2 = np.array([0, T2])
    sl1 = slice(0, T1)
    sl2 = slice(T1, T1 + T2)
    for impl in ("rec", "chunk"):
        if impl == "rec":
            o_a, s_a, _ = oracle.recurrent(q[sl1], k[sl1], v[sl1], g[sl1], beta[sl1], cu1, s0)
            o_b, s_b, _ = oracle.recurrent(q[sl2], k[sl2], v[sl2], g[sl2], beta[sl2], cu2, s_a)
        else:
            ra = oracle.chunked(q[sl1], k[sl1], v[sl1], g[sl1], beta[sl1], cu1, 16, s0)
            rb = oracle.chunked(q[sl2], k[sl2], v[sl2], g[sl2], beta[sl2], cu2, 16,
                                ra["state_out"])
            o_a, o_b, s_b = ra["o"], rb["o"], rb["state_out"]
        assert rel_err(np.concatenate([o_a, o_b]), o_full) < 1e-12
        assert rel_err(s_b, s_full) < 1e-12


def test_T7_decode_steps_equal_prefill():
    rng = np.random.default_rng(14)
    T = 20
    q, k, v, g, beta, cu, s0 = rand_problem(rng, [T], 2, 8, 8)
    o_full, s_full, _ = oracle.recurrent(q, k, v, g, beta, cu, s0)
    s = s0
    for t in range(T):
        sl = slice(t, t + 1)
        o_t, s, _ = oracle.recurrent(q[sl], k[sl], v[sl], g[sl], beta[sl], np.array([0, 1]), s)
        assert rel_err(o_t[0], o_full[t]) < 1e-13
    assert rel_err(s, s_full) < 1e-13


def test_T7_transfer_pairs_compose_as_a_semigroup():
    # (L_a, M_a) then (L_b, M_b) == (L_a M_b + L_b, M_a M_b) == the pair of the
    # concatenated chunk
    rng = np.random.default_rng(15)
    dk, dv, ca, cb = 8, 6, 9, 7
    _, k, v, g, beta, _, _ = rand_problem(rng, [ca + cb], 1, dk, dv, state0=False)
    K, V, G, B = k[:, 0], v[:, 0], g[:, 0], beta[:, 0]
    a = oracle.chunk_local(K[:ca], V[:ca], G[:ca], B[:ca])
    b = oracle.chunk_local(K[ca:], V[ca:], G[ca:], B[ca:])
    ab = oracle.chunk_local(K, V, G, B)
    assert rel_err(a["L"] @ b["M"] + b["L"], ab["L"]) < 1e-13
    assert rel_err(a["M"] @ b["M"], ab["M"]) < 1e-13


# --------------------------------------------------------------------------
# T8: layout


def brute_layout(cu, chunk):
    """Walk the tokens one by one; a new chunk starts at every sequence start
    and after every `chunk` tokens of the same sequence."""
    N = len(cu) - 1
    chunks = []  # (n, j, first_token, last_token_exclusive)
    for n in range(N):
        pos = 0
        for t in range(cu[n], cu[n + 1]):
            if pos % chunk == 0:
                chunks.append([n, pos // chunk, t, t + 1])
            else:
                chunks[-1][3] = t + 1
            pos += 1
    return chunks


@pytest.mark.parametrize("chunk", [1, 16, 64])
def test_T8_layout_matches_token_walk(chunk):
    rng = np.random.default_rng(80 + chunk)
    for trial in range(30):
        N = int(rng.integers(1, 12))
        lens = rng.integers(0, 200, size=N)
        lens[rng.random(N) < 0.2] = 0
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        offs, idx = oracle.layout(cu, chunk)
        ref = brute_layout(list(cu), chunk)
        assert idx.shape[0] == len(ref) == offs[-1]
        for c, (n, j, a, b) in enumerate(ref):
            assert tuple(idx[c]) == (n, j)
            assert oracle.chunk_token_range(cu, chunk, n, j) == (a, b)
        for n in range(N):
            assert offs[n + 1] - offs[n] == -(-int(lens[n]) // chunk)
        max_chunks = int(cu[-1]) // chunk + N
        offs2, idx2 = oracle.layout(cu, chunk, max_chunks)
        assert np.array_equal(offs2, offs)
        assert np.all(idx2[len(ref):] == -1)


# --------------------------------------------------------------------------
# pairs subset and threads do not change results


def test_recurrent_pairs_subset_and_threads():
    rng = np.random.default_rng(16)
    q, k, v, g, beta, cu, s0 = rand_problem(rng, [10, 7, 12], 3, 8, 8)
    o, s, _ = oracle.recurrent(q, k, v, g, beta, cu, s0, threads=1)
    o2, s2, _ = oracle.recurrent(q, k, v, g, beta, cu, s0, threads=4)
    assert np.array_equal(o, o2) and np.array_equal(s, s2)
    o3, s3, _ = oracle.recurrent(q, k, v, g, beta, cu, s0, pairs=[(1, 2), (2, 0)])
    assert np.array_equal(s3[1, 2], s[1, 2]) and np.array_equal(s3[2, 0], s[2, 0])
    assert np.all(s3[0] == 0)
    assert np.array_equal(o3[10:17, 2], o[10:17, 2])
