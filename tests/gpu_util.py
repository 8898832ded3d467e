"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
compare against the oracle in float64 on the host."""
import sys

import numpy as np
import torch

BF16_TOL = 1e-3   # max|gpu - ref| / max|ref| for bf16 inputs
FP32_TOL = 1e-5   # the same for fp32 inputs


def say(msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev_inputs(d, device="cuda"):
    """q, k, v (bf16 or fp32), g, beta (fp32), state0 (fp32 or None), cu (int32)."""
    def io(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    out = {name: io(d[name]) for name in ("q", "k", "v")}
    out["g"] = torch.from_numpy(d["g"]).to(device)
    out["beta"] = torch.from_numpy(d["beta"]).to(device)
    out["state0"] = None if d["state0"] is None else torch.from_numpy(d["state0"]).to(device)
    out["cu"] = torch.from_numpy(d["cu_seqlens"].astype(np.int32)).to(device)
    return out


def host64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    diff = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    return diff / scale if scale > 0 else diff


def tol_for(d):
    return BF16_TOL if d["dtype"] == "bf16" else FP32_TOL


def bf16_rne_of(t32):
    """Round an fp32 tensor to bf16 (torch's conversion is round-to-nearest-even)."""
    return t32.to(torch.bfloat16)
