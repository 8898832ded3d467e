"""GPU varlen layout is bit-exact with the oracle's integer layout."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunk", [16, 64])
def test_layout_bit_exact(chunk):
    import gated_delta_rule_100_amd as gdr
    rng = np.random.default_rng(200 + chunk)
    for trial in range(20):
        N = int(rng.integers(1, 3000 if trial == 0 else 40))
        lens = rng.integers(0, 300, size=N)
        lens[rng.random(N) < 0.25] = 0
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        T = int(cu[-1])
        mc = gdr.gdr_max_chunks(T, N, chunk)
        say(f"layout chunk={chunk} trial={trial} N={N} T={T}")
        offs = torch.empty(N + 1, dtype=torch.int32, device="cuda")
        idx = torch.empty(mc, 2, dtype=torch.int32, device="cuda")
        gdr.gdr_chunk_layout(torch.from_numpy(cu).cuda(), chunk, offs, idx)
        torch.cuda.synchronize()
        ref_offs, ref_idx = oracle.layout(cu, chunk, max_chunks=mc)
        assert np.array_equal(offs.cpu().numpy().astype(np.int64), ref_offs)
        assert np.array_equal(idx.cpu().numpy().astype(np.int64), ref_idx)


@pytest.mark.parametrize("N", [1, 255, 256, 1024, 1025, 3000])
def test_layout_bit_exact_around_single_launch_limit(N):
    """Up to 1024 sequences the layout is built in one launch (each workgroup
    scans in LDS); beyond that by a scan workgroup and a second launch.  Both
    sides of the limit, with empty sequences mixed in, and an all-empty batch."""
    import gated_delta_rule_100_amd as gdr
    rng = np.random.default_rng(7000 + N)
    for empty in (False, True):
        lens = np.zeros(N, dtype=np.int64) if empty else rng.integers(0, 200, size=N)
        if not empty:
            lens[rng.random(N) < 0.2] = 0
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        T = int(cu[-1])
        mc = gdr.gdr_max_chunks(T, N, 64)
        say(f"layout N={N} T={T} empty={empty}")
        offs = torch.empty(N + 1, dtype=torch.int32, device="cuda")
        idx = torch.empty(max(mc, 1), 2, dtype=torch.int32, device="cuda")
        gdr.gdr_chunk_layout(torch.from_numpy(cu).cuda(), 64, offs, idx[:mc])
        torch.cuda.synchronize()
        ref_offs, ref_idx = oracle.layout(cu, 64, max_chunks=mc)
        assert np.array_equal(offs.cpu().numpy().astype(np.int64), ref_offs)
        assert np.array_equal(idx[:mc].cpu().numpy().astype(np.int64), ref_idx)
