"""Rounding budget of the factored scan's operand planes (CPU, numpy).

The scan kernel (bf16 inputs, chunk 64) carries every fp32 operand of its
matrix products as planes of 16-bit floats, and the error of the whole path
must stay within 1e-3 of max|ref| (R14).  This module emulates the scan's
chunk step in numpy with the kernel's operand representation -- each operand
rounded into planes (bf16 or fp16, round to nearest even), products of plane
pairs summed in fp32 -- and measures each choice against the oracle's
token-by-token recurrence, to show which plane counts the budget allows:

  * the kernel's choice: the state S and diag(D) U as two bf16 planes, T as
    one fp16 plane (scaled by 16) against R as two fp16 planes (scaled by
    1/16), and P as one fp16 plane (scaled by 16) against U as two fp16
    planes (scaled by 1/16), stays within a third of the budget;
  * any one of the bf16 operands cut to a single plane spends most of the
    budget or more (a bf16 plane keeps 8 significant bits: 2^-9 relative);
  * T or P in one bf16 plane does too, while one fp16 plane (11 bits) does
    not.

The chunk step (Appendix A of the derivation, in factored form):
  Z = K S^T,  Y = Q S^T,  R = diag(beta) (V - diag(gamma) Z),  U = T R,
  O = diag(gamma) Y + P U,  S <- gamma_C S + (diag(D) U)^T K,
with T = (I + A)^{-1}, A_ts = beta_t Gamma_ts (k_t . k_s) (s < t) and
P = (Q K^T) (.) Gamma (s <= t), formed here in fp64 and rounded into planes.
"""
import numpy as np
import pytest

import oracle
from gdr_synth import workload

TOL = 1e-3  # R14, bf16 inputs


def _bf16(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.view(np.float32)


def _planes(x, spec):
    """x (fp32) as planes: spec = (kind, count), kind "bf16" or "fp16"; None
    keeps x in fp64 (the exact product, for the emulation's own check)."""
    if spec is None:
        return [np.asarray(x, dtype=np.float64)]
    kind, count = spec
    r = np.asarray(x, dtype=np.float32)
    out = []
    for _ in range(count):
        h = _bf16(r) if kind == "bf16" else r.astype(np.float16).astype(np.float32)
        out.append(h)
        r = (r - h).astype(np.float32)
    return out


def _mm(a, sa, b, sb):
    """Plane products with i + j < max(planes), smallest terms first, fp32
    accumulation (fp64 when either side is exact)."""
    ap, bp = _planes(a, sa), _planes(b, sb)
    if sa is None or sb is None:
        return _planes(a, None)[0] @ _planes(b, None)[0]
    pm = max(len(ap), len(bp))
    acc = np.zeros((a.shape[0], b.shape[1]), dtype=np.float32)
    for s in range(pm - 1, -1, -1):
        for i in range(len(ap)):
            j = s - i
            if 0 <= j < len(bp):
                acc = (acc + (ap[i] @ bp[j]).astype(np.float32)).astype(np.float32)
    return acc


KERNEL = dict(S=("bf16", 2), R=("fp16", 2), T=("fp16", 1), U=("fp16", 2), DU=("bf16", 2),
              P=("fp16", 1), scale=16.0)
EXACT = dict(S=None, R=None, T=None, U=None, DU=None, P=None, scale=1.0)
BF16_2 = ("bf16", 2)


def _scan(q, k, v, g, beta, s0, cfg, C=64):
    """One (sequence, head); q, k, v [T, d] exact input values."""
    exact = cfg["S"] is None
    ft = np.float64 if exact else np.float32
    T, d = q.shape
    S = np.zeros((d, d), ft) if s0 is None else s0.astype(ft)
    o = np.zeros((T, d))
    bf1 = None if exact else ("bf16", 1)  # q, k, v: exact in one bf16 plane
    for c0 in range(0, T, C):
        Q, K, V = q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C]
        gc, bc = g[c0:c0 + C].astype(np.float64), beta[c0:c0 + C].astype(np.float64)
        G = np.cumsum(gc)
        Gam = np.tril(np.exp(G[:, None] - G[None, :]))
        A = np.tril(bc[:, None] * Gam * (K @ K.T), -1)
        Tm = np.linalg.inv(np.eye(len(gc)) + A).astype(ft)
        P = np.tril(Gam * (Q @ K.T)).astype(ft)
        gam, D, b = np.exp(G).astype(ft), np.exp(G[-1] - G).astype(ft), bc.astype(ft)
        Kf, Qf, Vf = K.astype(ft), Q.astype(ft), V.astype(ft)
        Z = _mm(Kf, bf1, S.T, cfg["S"])
        Y = _mm(Qf, bf1, S.T, cfg["S"])
        sc = ft(cfg["scale"])
        R = ((b / sc)[:, None] * (Vf - gam[:, None] * Z)).astype(ft)
        U = _mm((Tm * sc).astype(ft), cfg["T"], R, cfg["R"])
        o[c0:c0 + C] = gam[:, None] * Y + _mm(P, cfg["P"], U, cfg["U"])
        DU = (D[:, None] * U).astype(ft)
        S = (gam[-1] * S + _mm(DU.T, cfg["DU"], Kf, bf1)).astype(ft)
    return o, S


_CASES = {}


def _case(gate):
    if gate not in _CASES:
        d = workload(2, seed=2, seqlens=[1024], H=1, gate=gate)
        ref_o, ref_s, _ = oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                           d["cu_seqlens"], d["state0"])
        args = (oracle.as_f64(d["q"])[:, 0], oracle.as_f64(d["k"])[:, 0],
                oracle.as_f64(d["v"])[:, 0], d["g"][:, 0], d["beta"][:, 0], d["state0"][0, 0])
        _CASES[gate] = (args, ref_o[:, 0], ref_s[0, 0])
    return _CASES[gate]


def _err(gate, **over):
    cfg = dict(KERNEL)
    cfg.update(over)
    args, ref_o, ref_s = _case(gate)
    o, s = _scan(*args, cfg)
    return max(np.abs(o - ref_o).max() / np.abs(ref_o).max(),
               np.abs(s - ref_s).max() / np.abs(ref_s).max())


GATES = ["std", "slow", "unit"]


@pytest.mark.parametrize("gate", GATES)
def test_emulation_in_fp64_is_the_recurrence(gate):
    # with every operand exact the factored step reproduces the oracle: the
    # emulation computes the method, so its rounding figures mean something
    assert _err(gate, **EXACT) < 1e-11


@pytest.mark.parametrize("gate", GATES)
def test_kernel_planes_leave_most_of_the_budget(gate):
    assert _err(gate) < TOL / 3


def test_no_bf16_operand_fits_in_one_plane():
    # S (both its products), R, U, diag(D) U and P each cut to one bf16 plane
    worst = {}
    for name, over in {"S": dict(S=("bf16", 1)), "R": dict(R=("bf16", 1), T=BF16_2, scale=1.0),
                       "U": dict(U=("bf16", 1), P=BF16_2), "DU": dict(DU=("bf16", 1)),
                       "P": dict(P=("bf16", 1), U=BF16_2)}.items():
        worst[name] = max(_err(gate, **over) for gate in GATES)
    assert all(e > TOL / 2 for e in worst.values()), worst


def test_t_needs_fp16_for_one_plane():
    # T alone (P and U at two bf16 planes): one bf16 plane spends about half
    # the budget, one fp16 plane a small part of it
    bf = max(_err(gate, T=("bf16", 1), R=BF16_2, scale=1.0, P=BF16_2, U=BF16_2) for gate in GATES)
    h = max(_err(gate, P=BF16_2, U=BF16_2) for gate in GATES)
    assert bf > 3 * TOL / 10 and h < TOL / 10, (bf, h)


def test_p_in_one_fp16_plane():
    # P in one fp16 plane against U in two fp16 planes (the kernel): under a
    # third of the budget, where one bf16 plane of P spends more than all of it
    h = max(_err(gate) for gate in GATES)
    bf = max(_err(gate, P=("bf16", 1), U=BF16_2) for gate in GATES)
    assert h < TOL / 3 and bf > 2 * TOL, (h, bf)
