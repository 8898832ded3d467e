"""Seeded synthetic inputs for the gated delta rule workloads.

This module only draws and encodes inputs.  It holds none of the method's
arithmetic and is shared by the oracle tests, the GPU parity tests and the
benchmark, so that both sides see the same input bits.

Recipe (numpy PCG64, seed = workload index unless stated):
  * draws in float64, in this order: [sequence lengths (varlen only)], q, k, v,
    g_pre, beta_pre, [S0 (only when the workload has an initial state)];
  * q and k are L2-normalised per (token, head) over dk, in float64;
  * g = -softplus(g_pre) (so alpha = exp(g) lies in (0, 1)), beta = sigmoid(beta_pre);
    the "slow" gate variant uses g = -0.01 * softplus(g_pre), the "steep"
    variant g = -4 * softplus(g_pre) (in-chunk decays far below e^-87, so
    that decay factors underflow) and the "unit" variant g = 0 (alpha = 1),
    beta unchanged;
  * S0 = 0.02 * N(0, 1) (standard deviation 0.02);
  * everything is cast to float32; q, k, v are then rounded to bfloat16 with
    round-to-nearest-even where the workload is bf16.  Gates and states stay
    float32.

bf16 tensors are returned as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "WORKLOADS",
    "bf16_bits_from_f32",
    "generate",
    "workload",
    "varlen_lengths",
]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns.  Inputs here are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def varlen_lengths(rng: np.random.Generator, n_seq: int, total: int, cap: int,
                   mu: float = 8.0, sigma: float = 1.0) -> np.ndarray:
    """Lengths drawn lognormal(mu, sigma), clipped to [1, cap], rescaled to sum
    to `total` exactly.  Integer rounding: floor (at least 1), then the
    remaining tokens go one each by largest fractional remainder (ties to the
    lower index); lengths above `cap` are clipped and the excess is handed out
    the same way to sequences still below the cap."""
    x = np.clip(rng.lognormal(mu, sigma, size=n_seq), 1.0, float(cap))
    scaled = x * (total / x.sum())
    lens = np.maximum(1, np.floor(scaled)).astype(np.int64)
    rem = scaled - np.floor(scaled)
    order = sorted(range(n_seq), key=lambda i: (-rem[i], i))

    def hand_out(count: int) -> None:
        i = 0
        guard = 0
        while count > 0:
            j = order[i % n_seq]
            if lens[j] < cap:
                lens[j] += 1
                count -= 1
            i += 1
            guard += 1
            if guard > 100 * n_seq + 10 * total:
                raise ValueError("cannot place tokens under the cap")

    def take_back(count: int) -> None:
        # only reachable when the max(1, .) floor overshoots; remove from the
        # longest sequences
        while count > 0:
            j = int(np.argmax(lens))
            lens[j] -= 1
            count -= 1

    diff = total - int(lens.sum())
    if diff > 0:
        hand_out(diff)
    elif diff < 0:
        take_back(-diff)
    excess = int(np.maximum(lens - cap, 0).sum())
    lens = np.minimum(lens, cap)
    if excess:
        hand_out(excess)
    assert int(lens.sum()) == total and lens.min() >= 1 and lens.max() <= cap
    return lens


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def generate(seqlens, H: int, dk: int, dv: int, dtype: str = "bf16",
             state0: bool = True, seed: int = 0, gate: str = "std",
             lengths_from_rng=None, keys: str = "gauss") -> dict:
    """Draw one packed batch.

    seqlens: list of per-sequence token counts (zeros allowed), or None when
        `lengths_from_rng` = (n_seq, total, cap) asks for the varlen recipe.
    dtype: "bf16" or "f32" for q, k, v.
    gate: "std" | "slow" | "steep" | "unit".
    keys: "gauss" (the default recipe) or "orthonormal": per sequence and head
        the keys are the rows of an orthonormal set (QR of a Gaussian draw),
        which needs each sequence no longer than dk.
    Returns a dict: q, k, v (uint16 bf16 bits or float32), g, beta (float32
    [T, H]), state0 (float32 [N, H, dv, dk] or None), cu_seqlens (int32
    [N+1]), seqlens (int64), and the shape fields.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if lengths_from_rng is not None:
        n_seq, total, cap = lengths_from_rng
        lens = varlen_lengths(rng, n_seq, total, cap)
    else:
        lens = np.asarray(seqlens, dtype=np.int64)
    N = int(lens.shape[0])
    T = int(lens.sum())
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)

    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g_pre = rng.standard_normal((T, H))
    b_pre = rng.standard_normal((T, H))
    s0 = 0.02 * rng.standard_normal((N, H, dv, dk)) if state0 else None

    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    if keys == "orthonormal":
        for n in range(N):
            a, b = int(cu[n]), int(cu[n + 1])
            if b - a > dk:
                raise ValueError("orthonormal keys need sequences no longer than dk")
            for h in range(H):
                if b > a:
                    qm, _ = np.linalg.qr(rng.standard_normal((dk, b - a)))
                    k[a:b, h, :] = qm.T
    else:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)

    if gate == "std":
        g = -_softplus(g_pre)
    elif gate == "slow":
        g = -0.01 * _softplus(g_pre)
    elif gate == "steep":
        g = -4.0 * _softplus(g_pre)
    elif gate == "unit":
        g = np.zeros_like(g_pre)
    else:
        raise ValueError(f"unknown gate variant {gate!r}")
    beta = _sigmoid(b_pre)

    out = {
        "g": g.astype(np.float32),
        "beta": beta.astype(np.float32),
        "state0": None if s0 is None else s0.astype(np.float32),
        "cu_seqlens": cu.astype(np.int32),
        "seqlens": lens,
        "N": N, "T": T, "H": H, "dk": dk, "dv": dv, "dtype": dtype,
    }
    for name, arr in (("q", q), ("k", k), ("v", v)):
        f = arr.astype(np.float32)
        out[name] = bf16_bits_from_f32(f) if dtype == "bf16" else f
    return out


# The five workloads.  `kind` says which path they exercise.
WORKLOADS = {
    0: dict(name="tiny-gdr-T64-H2-d64-C16-f32", kind="both", seqlens=[64], H=2,
            dk=64, dv=64, chunk=16, dtype="f32", state0=False),
    1: dict(name="decode-N64-H32-d128-bf16", kind="decode", seqlens=[1] * 64, H=32,
            dk=128, dv=128, chunk=0, dtype="bf16", state0=True),
    2: dict(name="prefill-B4-T4096-H16-d128-C64-bf16", kind="prefill",
            seqlens=[4096] * 4, H=16, dk=128, dv=128, chunk=64, dtype="bf16", state0=True),
    3: dict(name="varlen-8seq-32768tok-H32-d128-C64-bf16", kind="prefill",
            seqlens=None, varlen=(8, 32768, 16384), H=32, dk=128, dv=128, chunk=64,
            dtype="bf16", state0=True),
    4: dict(name="long-B1-T131072-H4-d128-C64-bf16", kind="prefill",
            seqlens=[131072], H=4, dk=128, dv=128, chunk=64, dtype="bf16", state0=False),
}


def workload(index: int, seed: int | None = None, **overrides) -> dict:
    """Inputs for workload `index` (seed defaults to the index).  Overrides may
    replace seqlens (e.g. a reduced T), H, gate, state0, dtype, keys."""
    spec = dict(WORKLOADS[index])
    spec.update(overrides)
    seed = index if seed is None else seed
    lengths_from_rng = spec.get("varlen") if spec.get("seqlens") is None else None
    d = generate(spec.get("seqlens"), spec["H"], spec["dk"], spec["dv"],
                 dtype=spec["dtype"], state0=spec["state0"], seed=seed,
                 gate=spec.get("gate", "std"), lengths_from_rng=lengths_from_rng,
                 keys=spec.get("keys", "gauss"))
    d["chunk"] = spec["chunk"]
    d["name"] = spec["name"]
    d["seed"] = seed
    return d
