"""Plain, slow, fp64 CPU oracle for the gated delta rule.

TEST INFRASTRUCTURE.  Only tests/, the smoke check and the benchmark's CPU
baseline may import this package.  The GPU product path never calls it, and it
imports nothing from the product package (nor the other way round).

The method (the gated delta rule, GDN-style linear attention):
    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t,      alpha_t = exp(g_t),
with a per-head state S of shape dv x dk.  Two forms are computed here:

O1  recurrent  -- the definition, token by token (C, gdr_oracle.c).
O2  chunked    -- the chunk-parallel ("CP") form: per chunk a local state L_c
                  and a transfer matrix M_c (S_end = S_start M_c + L_c), a
                  sequential fixup over chunks, then the chunk outputs.  The
                  FlashInfer PR #3866 page ("CP delta-rule precompute
                  optimisation for ultra-low parallelism", code changes §2)
                  gives the fixup's structure: init_state_tile (start from the
                  given initial state at chunk 0, or without one seed with the
                  first local state and begin at chunk 1),
                  accumulate_state_fragment (acc[i] += S[i,k] M[k,col]: the
                  state multiplies M from the left) and run_simt_fixup_loop
                  (chunks in order, each result published as that chunk's fixed
                  state).  The intra-chunk algebra (UT/WY transform) is derived
                  from the recurrence; it is an exact re-association, so O1 and
                  O2 agree up to rounding.
O3  layout     -- varlen packing of chunks (plain integer loops).
O4  brute force transfer matrices Phi_t = alpha_t (I - beta_t k_t k_t^T) and
                  their products (dense, tiny sizes).

Pins (closed forms, brute force, invariants) live in tests/test_oracle_*.py.
Every function here is pinned there; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np
import scipy.linalg

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_gdr.so")

_BF16, _F32, _F64 = 0, 1, 2


def build_oracle(force: bool = True) -> str:
    """Compile gdr_oracle.c with gcc into oracle/liboracle_gdr.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB_PATH):
            build_oracle(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_recurrent.argtypes = [p, p, p, i, p, p, p, i, p, p, p, i, i, i,
                                         p, i, i, p, p, i]
        lib.oracle_recurrent.restype = i
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i
        _lib_handle = lib
    return _lib_handle


def max_threads() -> int:
    return int(_lib().oracle_max_threads())


# ----------------------------------------------------------------------------
# input decoding


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray) -> np.ndarray:
    """Decode an input tensor (bf16 bits as uint16, float32 or float64)."""
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float64)


def _qkv_code(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return _BF16
    if x.dtype == np.float32:
        return _F32
    if x.dtype == np.float64:
        return _F64
    raise TypeError(f"unsupported q/k/v dtype {x.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------
# O1: the recurrence, token by token


def recurrent(q, k, v, g, beta, cu_seqlens, state_in=None, *, pairs=None,
              chunk: int = 0, threads: int = 0):
    """O1.  q, k [T, H, dk]; v [T, H, dv] (uint16 bf16 bits, float32 or float64,
    all three the same dtype); g, beta [T, H]; cu_seqlens [N+1]; state_in
    [N, H, dv, dk] or None (zero).  Returns (o [T, H, dv], state_out
    [N, H, dv, dk], chunk_states [n_chunks, H, dv, dk] or None) in float64.

    pairs: optional list of (n, h) to compute; other entries of o / state_out
    stay zero (and chunk_states stays zero for them).
    chunk > 0 records the state at the end of every chunk (packed order of O3).
    """
    T, H, dk = q.shape
    dv = v.shape[2]
    code = _qkv_code(q)
    assert _qkv_code(k) == code and _qkv_code(v) == code
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    g = np.ascontiguousarray(g, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == T
    sin = None if state_in is None else np.ascontiguousarray(state_in, dtype=np.float64)
    sout = np.zeros((N, H, dv, dk), dtype=np.float64)
    o = np.zeros((T, H, dv), dtype=np.float64)
    pr = None
    npairs = 0
    if pairs is not None:
        pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
        npairs = pr.shape[0]
    cs = None
    offs = None
    if chunk > 0:
        offs, _ = layout(cu, chunk)
        offs = np.ascontiguousarray(offs, dtype=np.int64)
        cs = np.zeros((int(offs[-1]), H, dv, dk), dtype=np.float64)
    rc = _lib().oracle_recurrent(_ptr(q), _ptr(k), _ptr(v), code, _ptr(g), _ptr(beta),
                                 _ptr(cu), N, _ptr(sin), _ptr(sout), _ptr(o), H, dk, dv,
                                 _ptr(pr), npairs, int(chunk), _ptr(offs), _ptr(cs),
                                 int(threads))
    if rc != 0:
        raise MemoryError("oracle_recurrent: allocation failed")
    return o, sout, cs


# ----------------------------------------------------------------------------
# O3: varlen chunk layout


def layout(cu_seqlens, chunk: int, max_chunks: int | None = None):
    """O3.  For packed sequences with token offsets cu_seqlens [N+1] and chunk
    size `chunk`:
        chunk_offsets[0] = 0,
        chunk_offsets[n+1] = chunk_offsets[n] + ceil(len_n / chunk),
        chunk_indices[chunk_offsets[n] + j] = (n, j)  for j < ceil(len_n / chunk).
    Chunk j of sequence n covers tokens [cu[n] + j*chunk, min(cu[n] + (j+1)*chunk, cu[n+1])).
    With max_chunks given, chunk_indices has max_chunks rows and the rows past
    the real chunk count hold (-1, -1).
    Returns (chunk_offsets int64 [N+1], chunk_indices int64 [n, 2])."""
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    offsets = [0]
    indices = []
    for n in range(N):
        length = cu[n + 1] - cu[n]
        count = 0
        start = 0
        while start < length:
            indices.append((n, count))
            count += 1
            start += chunk
        offsets.append(offsets[-1] + count)
    if max_chunks is not None:
        assert max_chunks >= len(indices)
        indices += [(-1, -1)] * (max_chunks - len(indices))
    return (np.asarray(offsets, dtype=np.int64),
            np.asarray(indices, dtype=np.int64).reshape(-1, 2))


def chunk_token_range(cu_seqlens, chunk: int, n: int, j: int):
    """Token range [a, b) of chunk j of sequence n."""
    a = int(cu_seqlens[n]) + j * chunk
    b = min(a + chunk, int(cu_seqlens[n + 1]))
    return a, b


# ----------------------------------------------------------------------------
# O2: the chunked (CP) form, phase by phase, in float64


def chunk_gates(gc: np.ndarray):
    """Gate prefix of one chunk of length c (P1).
    G_t = sum_{s<=t} g_s (restarting at the chunk start), gamma_t = exp(G_t),
    Gamma[t, s] = exp(G_t - G_s) for s <= t (0 above the diagonal),
    D_s = exp(G_c - G_s).  Every exponent is <= 0 when g <= 0."""
    G = np.cumsum(gc)
    gamma = np.exp(G)
    lower = np.tril(np.ones((len(gc), len(gc)), dtype=bool))
    Gamma = np.exp(np.where(lower, G[:, None] - G[None, :], -np.inf))
    D = np.exp(G[-1] - G) if len(gc) else np.zeros(0)
    return G, gamma, Gamma, D


def chunk_local(Kc, Vc, gc, bc):
    """Chunk-local precompute (P1-P5) for one chunk (c tokens, c >= 1).

    Kc [c, dk], Vc [c, dv], gc, bc [c] in float64.  With u_t the corrected
    value beta_t (v_t - alpha_t S_{t-1} k_t), the state inside the chunk is
    S_t = gamma_t S_0 + sum_{s<=t} (gamma_t / gamma_s) u_s k_s^T; substituting
    gives (I + A) U = diag(beta) V - diag(beta gamma) K S_0^T with
        A[t, s] = beta_t Gamma[t, s] (k_t . k_s)   for s < t, else 0.
    T = (I + A)^{-1},  W = T diag(beta gamma) K,  Ut = T diag(beta) V,
    so U = Ut - W S_0^T, and at the chunk end S_c = S_0 M + L with
        L = Ut^T diag(D) K          [dv, dk]
        M = gamma_c I - W^T diag(D) K   [dk, dk].
    Returns dict(W, Ut, L, M, gamma, Gamma, D)."""
    c, dk = Kc.shape
    G, gamma, Gamma, D = chunk_gates(gc)
    KK = Kc @ Kc.T
    A = np.tril(bc[:, None] * Gamma * KK, k=-1)
    Tm = scipy.linalg.solve_triangular(np.eye(c) + A, np.eye(c), lower=True,
                                       unit_diagonal=True)
    W = Tm @ ((bc * gamma)[:, None] * Kc)
    Ut = Tm @ (bc[:, None] * Vc)
    DK = D[:, None] * Kc
    L = Ut.T @ DK
    M = gamma[-1] * np.eye(dk) - W.T @ DK
    return dict(W=W, Ut=Ut, L=L, M=M, gamma=gamma, Gamma=Gamma, D=D, T=Tm, A=A)


def fixup(L_list, M_list, state_in):
    """Inter-chunk fixup (P6) for one (sequence, head): chunk states at the
    end of each chunk, fixed[c] = fixed[c-1] M_c + L_c with fixed[-1] = the
    initial state.  Without an initial state (state_in None) the first fixed
    state is L_0 and the loop starts at chunk 1 (the same result as a zero
    initial state).  Returns a list of [dv, dk] arrays."""
    fixed = []
    if not L_list:
        return fixed
    if state_in is None:
        S = L_list[0].copy()
        fixed.append(S)
        start = 1
    else:
        S = np.asarray(state_in, dtype=np.float64)
        start = 0
    for c in range(start, len(L_list)):
        S = S @ M_list[c] + L_list[c]
        fixed.append(S)
    return fixed


def chunk_out(Qc, Kc, loc, S0):
    """Chunk outputs (P7) given the chunk's start state S0 [dv, dk]:
        U = Ut - W S0^T
        O = diag(gamma) Q S0^T + (Q K^T (.) Gamma) U      (Gamma lower incl. diagonal)
    Returns O [c, dv]."""
    U = loc["Ut"] - loc["W"] @ S0.T
    P = (Qc @ Kc.T) * loc["Gamma"]
    return loc["gamma"][:, None] * (Qc @ S0.T) + P @ U


def chunked(q, k, v, g, beta, cu_seqlens, chunk: int, state_in=None, *,
            heads=None, seqs=None, keep_local: bool = True):
    """O2.  The whole chunked form: P0 layout, P1-P5 for every chunk, P6 fixup
    over each sequence's chunks in order, P7 outputs, P8 final states.

    Inputs as in `recurrent` (any of uint16 bf16 bits / float32 / float64).
    heads / seqs restrict the work to a subset (others stay zero).
    Returns dict(o [T,H,dv], state_out [N,H,dv,dk], L, M [n_chunks,H,...] (if
    keep_local), fixed [n_chunks,H,dv,dk], chunk_offsets, chunk_indices)."""
    Q = as_f64(q)
    K = as_f64(k)
    V = as_f64(v)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, H, dk = K.shape
    dv = V.shape[2]
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    offs, idx = layout(cu, chunk)
    nch = int(offs[-1])
    heads = range(H) if heads is None else heads
    seqs = range(N) if seqs is None else seqs
    o = np.zeros((T, H, dv))
    sout = np.zeros((N, H, dv, dk))
    fixed_all = np.zeros((nch, H, dv, dk))
    L_all = np.zeros((nch, H, dv, dk)) if keep_local else None
    M_all = np.zeros((nch, H, dk, dk)) if keep_local else None
    for n in seqs:
        nc = int(offs[n + 1] - offs[n])
        for h in heads:
            s_init = None if state_in is None else np.asarray(state_in[n, h], dtype=np.float64)
            locs = []
            for j in range(nc):
                a, b = chunk_token_range(cu, chunk, n, j)
                locs.append(chunk_local(K[a:b, h], V[a:b, h], g[a:b, h], beta[a:b, h]))
            fixed = fixup([x["L"] for x in locs], [x["M"] for x in locs], s_init)
            for j in range(nc):
                a, b = chunk_token_range(cu, chunk, n, j)
                if j == 0:
                    S0 = np.zeros((dv, dk)) if s_init is None else s_init
                else:
                    S0 = fixed[j - 1]
                o[a:b, h] = chunk_out(Q[a:b, h], K[a:b, h], locs[j], S0)
                c_id = int(offs[n]) + j
                fixed_all[c_id, h] = fixed[j]
                if keep_local:
                    L_all[c_id, h] = locs[j]["L"]
                    M_all[c_id, h] = locs[j]["M"]
            if nc:
                sout[n, h] = fixed[-1]
            else:
                sout[n, h] = 0.0 if s_init is None else s_init
    return dict(o=o, state_out=sout, L=L_all, M=M_all, fixed=fixed_all,
                chunk_offsets=offs, chunk_indices=idx)


# ----------------------------------------------------------------------------
# O4: brute-force transfer products


def step_matrix(kt, gt, bt):
    """Phi_t = alpha_t (I - beta_t k_t k_t^T), alpha_t = exp(g_t), dense."""
    kt = np.asarray(kt, dtype=np.float64)
    return np.exp(gt) * (np.eye(kt.shape[0]) - bt * np.outer(kt, kt))


def transfer_bruteforce(Kc, gc, bc):
    """M = Phi_1 Phi_2 ... Phi_c (time order), so that S_c = S_0 M + L."""
    dk = Kc.shape[1]
    M = np.eye(dk)
    for t in range(Kc.shape[0]):
        M = M @ step_matrix(Kc[t], gc[t], bc[t])
    return M


def state_bruteforce(S0, Kc, Vc, gc, bc):
    """Final state by the explicit product
        S_T = S_0 Phi_1...Phi_T + sum_s beta_s v_s k_s^T Phi_{s+1}...Phi_T."""
    c, dk = Kc.shape
    acc = np.asarray(S0, dtype=np.float64) @ transfer_bruteforce(Kc, gc, bc)
    for s in range(c):
        tail = np.eye(dk)
        for t in range(s + 1, c):
            tail = tail @ step_matrix(Kc[t], gc[t], bc[t])
        acc = acc + bc[s] * np.outer(Vc[s], Kc[s]) @ tail
    return acc
