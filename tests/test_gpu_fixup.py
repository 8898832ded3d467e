"""GPU fixup scan against the oracle's fixup, fed with L and M from the
oracle's chunk-local phase (slow gates, so M is far from zero)."""
import numpy as np
import pytest
import torch

import oracle
from gdr_synth import generate
from gpu_util import host64, rel_err, say

pytestmark = pytest.mark.gpu


def oracle_locals(d, chunk):
    K, V = oracle.as_f64(d["k"]), oracle.as_f64(d["v"])
    g, b = d["g"].astype(np.float64), d["beta"].astype(np.float64)
    cu = d["cu_seqlens"]
    offs, idx = oracle.layout(cu, chunk)
    nch = int(offs[-1])
    H, dk, dv = d["H"], d["dk"], d["dv"]
    L = np.zeros((nch, H, dv, dk))
    M = np.zeros((nch, H, dk, dk))
    for c in range(nch):
        n, j = idx[c]
        a, bnd = oracle.chunk_token_range(cu, chunk, n, j)
        for h in range(H):
            loc = oracle.chunk_local(K[a:bnd, h], V[a:bnd, h], g[a:bnd, h], b[a:bnd, h])
            L[c, h], M[c, h] = loc["L"], loc["M"]
    return offs, L, M


@pytest.mark.parametrize("with_state", [True, False])
@pytest.mark.parametrize("d_,H,lens", [(64, 2, [700, 0, 130, 64, 1]),
                                       (128, 2, [700, 0, 130, 64, 1]),
                                       (128, 64, [200, 65]),     # 32 rows per workgroup
                                       (128, 128, [130])])       # 64 rows per workgroup
def test_fixup_matches_oracle(with_state, d_, H, lens):
    import gated_delta_rule_100_amd as gdr
    chunk = 64 if d_ == 128 else 16
    d = generate(lens, H, d_, d_, dtype="f32", state0=True, seed=300 + d_ + H,
                 gate="slow")
    offs, L, M = oracle_locals(d, chunk)
    s0 = d["state0"].astype(np.float64) if with_state else None
    say(f"fixup d={d_} H={H} chunk={chunk} with_state={with_state} n_chunks={L.shape[0]}")
    Lg = torch.from_numpy(L.astype(np.float32)).cuda()
    Mg = torch.from_numpy(M.astype(np.float32)).cuda()  # M[c, h] = M_c as the oracle forms it
    fixed = torch.full_like(Lg, float("nan"))
    sin = torch.from_numpy(d["state0"]).cuda() if with_state else None
    gdr.gdr_state_fixup(Lg, Mg, sin, torch.from_numpy(offs.astype(np.int32)).cuda(), fixed)
    torch.cuda.synchronize()
    # reference: the oracle fixup on the same fp32 L, M (rounded) in float64
    L32 = L.astype(np.float32).astype(np.float64)
    M32 = M.astype(np.float32).astype(np.float64)
    got = host64(fixed)
    ref = np.zeros_like(got)
    for n in range(len(offs) - 1):
        for h in range(d["H"]):
            sl = range(int(offs[n]), int(offs[n + 1]))
            st = None if s0 is None else d["state0"][n, h].astype(np.float64)
            fx = oracle.fixup([L32[c, h] for c in sl], [M32[c, h] for c in sl], st)
            for c, f in zip(sl, fx):
                ref[c, h] = f
    assert rel_err(got, ref) <= 1e-5
