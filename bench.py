#!/usr/bin/env python3
"""Benchmark of the gated delta rule hot path on one MI355X.

One step = one pass over both forms of the path on synthetic inputs:
  * decode:  one token for 64 sequences x 32 heads, dk = dv = 128, bf16 q/k/v,
             fp32 state (128 MiB) updated in place, bf16 output;
  * prefill: chunked prefill of 4 sequences x 4096 tokens, 16 heads,
             dk = dv = 128, chunk 64, bf16 q/k/v, fp32 gates and states.
The headline `value` is the decode state bandwidth (state bytes read + written
per launch / decode launch time); the prefill throughput is reported beside it.
Timed after the step, outside it, and reported beside it:
  * `prefill_varlen`: 8 sequences, 32768 tokens, 32 heads;
  * `prefill_long`: one 131072-token sequence, 4 heads (segmented scan);
  * `prefill_cp` / `prefill_long_cp`: the prefill and long workloads with
    every chunk's L and M returned as well (the chunk-local kernel writes them
    beside the scan);
  * `fixup_long`: gdr_state_fixup alone over the long workload's 2048 chunks
    per head (L and M returned by its prefill): the dependent chain of
    S_{c+1} = S_c M_c + L_c, reported per step;
  * `decode_mtp`: multi-token decode (8 draft tokens per sequence on the decode
    workload's shape).

Timing.  HIP events recorded on the launch stream.  A short GPU spin is queued
before each timed batch, so the host has enqueued the launches before the GPU
reaches them and they run back to back (host overhead between launches does
not enter the events).  Prefill figures are the median over per-launch
durations (two events around each launch).  The decode and multi-token
kernels (42 and 49 us) are timed as the average launch duration over a region
of back-to-back launches between two events, because an event pair around
every launch adds about 1.5 us of marker gap to each; the per-launch median is
reported beside it.  Decode is cold: four state buffers (512 MiB, more than
the 256 MB Infinity Cache) in rotation.  Prefill writes a 1 GiB scrub buffer
before every timed launch (outside its events).  Warm figures (one decode
state buffer, prefill without the scrub) are reported as `warm`, for context.
Inputs are resident in HBM before timing starts.

Records.  HBM traffic, instruction mix and per-kernel durations come from
rocprofv3 runs of this script committed under profiles/ as JSON records; each
lists the sources it was taken on, and a record is used only while those
sources are unchanged (else its fields are null).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-other-prefill] [--only NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MIN_SAMPLES = 20       # per-launch samples of every figure outside the step

# decode workload: N=64, H=32, d=128
DEC_N, DEC_H, DEC_D = 64, 32, 128
DEC_STATE_BYTES = DEC_N * DEC_H * DEC_D * DEC_D * 4 * 2          # read + write
DEC_ALG_BYTES = DEC_STATE_BYTES + DEC_N * DEC_H * (3 * DEC_D * 2 + DEC_D * 2 + 8)
# prefill workload: B=4, T=4096, H=16, d=128, C=64
PRE_B, PRE_T, PRE_H, PRE_D, PRE_C = 4, 4096, 16, 128, 64
PRE_TOKENS = PRE_B * PRE_T
PRE_IO_BYTES = PRE_TOKENS * PRE_H * (3 * PRE_D * 2 + PRE_D * 2 + 8) \
    + 2 * PRE_B * PRE_H * PRE_D * PRE_D * 4
PRE_CHUNK_HEADS = PRE_B * (PRE_T // PRE_C) * PRE_H
PRE_CP_BYTES = PRE_IO_BYTES + PRE_CHUNK_HEADS * 393216
# The sequential-scan schedule (taken for this workload) moves per chunk-head
# the factors the chunk kernel writes (T and P compact lower-triangular, each
# one fp16 plane of 6 KiB, and 1 KiB of gates),
# which the scan reads back once, together with a second read of the chunk's
# q and k rows (16 KiB each; the factors kernel and the scan both read them),
# on top of the unavoidable input/output.
PRE_FACTOR_W = 6144 + 6144 + 1024
PRE_FACTOR_R = PRE_FACTOR_W + 2 * 16384
PRE_SCAN_BYTES = PRE_IO_BYTES + PRE_CHUNK_HEADS * (PRE_FACTOR_W + PRE_FACTOR_R)
# long workload: one sequence of 131072 tokens, 4 heads: 2048 chunks per head
LONG_T, LONG_H, LONG_CHUNKS = 131072, 4, 2048
# one fixup step per (chunk, head): read M_c and L_c, write fixed[c] (64 KiB each)
FIX_STEP_BYTES = 3 * 128 * 128 * 4


def io_min_bytes(idx):
    """Bytes any implementation must move for prefill workload idx: q, k, v, o
    (bf16), g and beta (fp32) per token and head, and the fp32 states in and
    out (the long workload has no initial state)."""
    from gdr_synth import WORKLOADS
    spec = WORKLOADS[idx]
    tokens = {2: PRE_TOKENS, 3: 32768, 4: 131072}[idx]
    n_seq = {2: PRE_B, 3: 8, 4: 1}[idx]
    H, D = spec["H"], spec["dk"]
    states = (2 if spec["state0"] else 1) * n_seq * H * D * D * 4
    return tokens * H * (3 * D * 2 + D * 2 + 8) + states


def cp_form_bytes(idx):
    """The chunk-parallel form's bytes: the I/O minimum plus L and M written and
    read once and the chunk-end states written and read once (6 states of
    64 KiB per chunk-head at d = 128)."""
    chunk_heads = {2: PRE_CHUNK_HEADS, 4: LONG_CHUNKS * LONG_H}[idx]
    return io_min_bytes(idx) + chunk_heads * 393216


def lm_request_bytes(idx):
    """Bytes of a bf16 prefill that also returns L and M: the I/O minimum, L and
    M written once (2 states of 64 KiB per chunk-head), and the scan's chunk
    factors written and read back with the second read of q and k."""
    chunk_heads = {2: PRE_CHUNK_HEADS, 4: LONG_CHUNKS * LONG_H}[idx]
    return io_min_bytes(idx) + chunk_heads * (2 * 65536 + PRE_FACTOR_W + PRE_FACTOR_R)


ONLY = ("decode", "prefill", "varlen", "long", "prefill_cp", "long_cp", "fixup_long", "mtp",
        "copy")


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-prefill", action="store_true",
                    help="skip the figures outside the step (other prefill workloads, the "
                         "chunk-parallel forms, the long fixup chain, multi-token decode, warm)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--only", choices=ONLY, default=None,
                    help="time only this figure (--steps launches) and print one JSON line; "
                         "for per-kernel profiles")
    return ap.parse_args(argv)


def to_dev(d, torch):
    def io(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out = {k: io(d[k]) for k in ("q", "k", "v")}
    out["g"] = torch.from_numpy(d["g"]).cuda()
    out["beta"] = torch.from_numpy(d["beta"]).cuda()
    out["state0"] = None if d["state0"] is None else torch.from_numpy(d["state0"]).cuda()
    out["cu"] = torch.from_numpy(d["cu_seqlens"].astype(np.int32)).cuda()
    return out


_SPIN = {}


def _spin(torch, stream, ms):
    """Queue about `ms` milliseconds of GPU spinning on `stream` (torch's sleep
    kernel, calibrated once), so that the launches queued after it run back to
    back on the GPU."""
    if "cycles_per_ms" not in _SPIN:
        try:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            torch.cuda._sleep(1_000_000)
            e1.record()
            torch.cuda.synchronize()
            _SPIN["cycles_per_ms"] = 1_000_000 / max(e0.elapsed_time(e1), 1e-3)
        except (AttributeError, RuntimeError):
            _SPIN["cycles_per_ms"] = None
    if _SPIN["cycles_per_ms"]:
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(ms * _SPIN["cycles_per_ms"]))


def region(torch, launch, n, stream, lead_ms=None):
    """n back-to-back launches between two events on `stream`: the average
    launch duration over the timed region (ms) and the host wall time."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _spin(torch, stream, lead_ms if lead_ms is not None else min(5.0 + 1.0 * n, 60.0))
    e0.record(stream)
    for i in range(n):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n, time.perf_counter() - t0


def per_launch(torch, launch, n, stream, before=None, lead_ms=None):
    """n launches, each between two events on `stream`; returns the per-launch
    durations (ms) and the host wall time.  before(i) runs ahead of launch i,
    outside its events."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _spin(torch, stream, lead_ms if lead_ms is not None else min(5.0 + 1.0 * n, 60.0))
    for i in range(n):
        if before is not None:
            before(i)
        ev[i][0].record(stream)
        launch(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    return dict(ms=float(np.median(ms)), ms_mean=float(np.mean(ms)), ms_min=float(np.min(ms)),
                ms_max=float(np.max(ms)), n=int(n), wall_s=wall)


def bench_decode(torch, gdr, steps, warmup, nbuf=4):
    """Decode step, in place, rotating over nbuf state buffers: 4 (512 MiB) is
    cold HBM; 1 reuses one 128 MiB state, which the 256 MB Infinity Cache could
    hold."""
    from gdr_synth import workload
    d = workload(1)
    di = to_dev(d, torch)
    bufs = [di["state0"].clone() for _ in range(nbuf)]
    o = torch.empty(DEC_N, DEC_H, DEC_D, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def launch(i):
        gdr.gdr_decode_step(di["q"], di["k"], di["v"], di["g"], di["beta"], bufs[i % nbuf], o,
                            stream=stream)

    for i in range(warmup):
        launch(i)
    r = per_launch(torch, launch, steps, stream)
    r["ms_median"] = r["ms"]
    r["ms"], r["wall_s"] = region(torch, launch, steps, stream)
    return r


def bench_mtp(torch, gdr, steps, warmup, T=8):
    """Multi-token decode on the decode workload's shape (64 sequences x 32
    heads, d = 128, bf16) with T draft tokens each and no per-token states,
    cold (4 rotating state buffers, each updated in place)."""
    from gdr_synth import generate
    d = generate([T] * DEC_N, DEC_H, DEC_D, DEC_D, dtype="bf16", state0=True, seed=1)
    di = to_dev(d, torch)
    x = {key: di[key].view(DEC_N, T, DEC_H, -1) for key in ("q", "k", "v")}
    g, b = di["g"].view(DEC_N, T, DEC_H), di["beta"].view(DEC_N, T, DEC_H)
    bufs = [di["state0"].clone() for _ in range(4)]
    o = torch.empty(DEC_N, T, DEC_H, DEC_D, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def launch(i):
        gdr.gdr_decode_mtp(x["q"], x["k"], x["v"], g, b, bufs[i % 4], bufs[i % 4], o, None,
                           stream=stream)

    for i in range(warmup):
        launch(i)
    r = per_launch(torch, launch, steps, stream)
    r["ms_median"] = r["ms"]
    r["ms"], r["wall_s"] = region(torch, launch, steps, stream)
    r["T"] = T
    return r


def copy_bandwidth(torch, reps=10):
    """Device-to-device copy of 1 GiB (read + write bytes per second), for context."""
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    stream = torch.cuda.current_stream()
    r = per_launch(torch, lambda i: dst.copy_(src), reps, stream)
    del src, dst
    return 2 * (1 << 30) / (r["ms"] / 1e3) / 1e9


def _sha256(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def load_record(name):
    """A committed profile record (profiles/<name>), or None if it is missing
    or any source it was taken on has changed since."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", name)))
        for path, digest in rec["sources"].items():
            if _sha256(os.path.join(ROOT, path)) != digest:
                return None
    except (OSError, ValueError, KeyError):
        return None
    return rec


def bench_prefill(torch, gdr, steps, warmup, idx=2, cp_form=False, cold=True, keep=False):
    """One prefill workload; cold writes a 1 GiB scrub buffer before every timed
    launch, warm (cold=False) times back-to-back launches.  keep returns the
    device buffers too."""
    from gdr_synth import workload
    d = workload(idx)
    di = to_dev(d, torch)
    T, H, D, N, C = d["T"], d["H"], d["dk"], d["N"], d["chunk"]
    o = torch.empty(T, H, D, dtype=torch.bfloat16, device="cuda")
    sout = torch.empty(N, H, D, D, device="cuda")
    ws = torch.empty(gdr.gdr_chunk_prefill_workspace_bytes(T, N, H, D, D, C, gdr.GDR_BF16),
                     dtype=torch.uint8, device="cuda")
    scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if cold else None  # 1 GiB
    stream = torch.cuda.current_stream()
    L = M = None
    if cp_form:  # every chunk's L and M returned as well
        mc = gdr.gdr_max_chunks(T, N, C)
        L = torch.empty(mc, H, D, D, device="cuda")
        M = torch.empty(mc, H, D, D, device="cuda")

    def launch(i):
        gdr.gdr_chunk_prefill(di["q"], di["k"], di["v"], di["g"], di["beta"], di["cu"],
                              di["state0"], sout, o, chunk=C, L_out=L, M_out=M, workspace=ws,
                              stream=stream)

    def before(i):
        if cold:
            scrub.fill_(float(i))

    for i in range(warmup):
        launch(i)
    r = per_launch(torch, launch, steps, stream, before=before)
    r.update(workload=d["name"], tokens=T)
    del scrub, ws
    if keep:
        r["buffers"] = dict(d=d, L=L, M=M)
    return r


def bench_fixup_long(torch, gdr, steps, warmup):
    """gdr_state_fixup alone over the long workload's chunks: L and M of its
    2048 chunks per head (returned by a prefill) through the chain
    fixed[c] = fixed[c-1] M_c + L_c, no initial state.  L + M + fixed are
    1.5 GiB, so every launch is cold."""
    r0 = bench_prefill(torch, gdr, 1, 1, 4, cp_form=True, cold=False, keep=True)
    b = r0["buffers"]
    L, M = b["L"], b["M"]
    n = LONG_CHUNKS
    offs = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    L, M = L[:n].contiguous(), M[:n].contiguous()
    fixed = torch.empty_like(L)
    stream = torch.cuda.current_stream()

    def launch(i):
        gdr.gdr_state_fixup(L, M, None, offs, fixed, stream=stream)

    for i in range(warmup):
        launch(i)
    r = per_launch(torch, launch, steps, stream)
    del L, M, fixed, b
    return r


def cpu_baseline(budget_s):
    """The fp64 oracle (token-by-token recurrence, OpenMP over (sequence, head))
    on the host cores: the whole decode workload repeated for about half the
    budget, and whole 4096-token sequences of the prefill workload (every
    (sequence, head) pair costs the same) for about the other half; then one
    (sequence, head) pair of the prefill workload on one thread."""
    import oracle
    from gdr_synth import workload
    threads = oracle.max_threads()
    d1 = workload(1)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.recurrent(d1["q"], d1["k"], d1["v"], d1["g"], d1["beta"], d1["cu_seqlens"],
                         d1["state0"], threads=threads)
        reps += 1
        if time.perf_counter() - t0 > budget_s / 2 or reps >= 500:
            break
    dec_s = (time.perf_counter() - t0) / reps
    del d1
    d2 = workload(2)
    pairs = [(n, h) for n in range(PRE_B) for h in range(PRE_H)]
    t0 = time.perf_counter()
    done = 0
    while done < len(pairs):
        batch = pairs[done:done + max(threads, 1)]
        oracle.recurrent(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], d2["cu_seqlens"],
                         d2["state0"], pairs=batch, threads=threads)
        done += len(batch)
        if time.perf_counter() - t0 > budget_s / 2:
            break
    pre_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.recurrent(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], d2["cu_seqlens"],
                     d2["state0"], pairs=[(0, 0)], threads=1)
    pair_1t = time.perf_counter() - t0
    return {
        "value": round(DEC_STATE_BYTES / dec_s / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 token-by-token recurrence: the whole decode workload (64x32 states, "
                  f"d=128) {reps} time(s), {dec_s * 1e3:.1f} ms each; prefill: {done} of the 64 "
                  f"(sequence, head) pairs of 4096 tokens in {pre_s:.1f} s; one pair on one "
                  f"thread in {pair_1t:.2f} s",
        "prefill_tokens_per_s": round(done * PRE_T / pre_s / PRE_H, 1),
        "one_thread_s_per_pair": round(pair_1t, 3),
        "one_thread_prefill_tokens_per_s": round(PRE_T / pair_1t / PRE_H, 1),
        "cpu": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _timing(r):
    """ms: the figure's time (per-launch median, or the region average where
    ms_median is given: then ms_mean and ms_min are per-launch too)."""
    out = {"ms": round(r["ms"], 5), "ms_mean": round(r["ms_mean"], 5),
           "ms_min": round(r["ms_min"], 5), "samples": r["n"]}
    if "ms_median" in r:
        out["ms_per_launch_median"] = round(r["ms_median"], 5)
    return out


def prefill_line(r, idx, lm=False):
    t = r["ms"] / 1e3
    line = {"workload": r["workload"] + (" with L and M returned" if lm else ""),
            "value": round(r["tokens"] / t, 1), "unit": "tokens/s", **_timing(r),
            "io_min_frac": round(io_min_bytes(idx) / t / 1e9 / HBM_PEAK_GBS, 4)}
    if lm:
        line["schedule"] = ("chunk-local L and M written in parallel, states and outputs by the "
                            "factored scan")
        line["own_bytes_frac"] = round(lm_request_bytes(idx) / t / 1e9 / HBM_PEAK_GBS, 4)
    return line


def record_summary(name, keys=("avg_us", "per_launch", "hbm_bytes", "hbm_gbs", "l2_hit_rate",
                                 "mfma_busy", "mean_waves_per_cu", "chain_steps",
                                 "us_per_chain_step", "valu_per_compute_wave_step",
                                 "mfma_per_compute_wave_step", "lds_per_compute_wave_step",
                                 "lds_busy", "lds_bank_conflict_per_busy")):
    """Per-kernel figures of a committed profile record (None when stale)."""
    rec = load_record(name)
    if rec is None:
        return None, None
    kern = {k: {f: v[f] for f in keys if f in v} for k, v in rec["kernels"].items()}
    return rec, kern


def prefill_roofline(pre_ms):
    """The prefill's roofline: the I/O-minimum bytes over the measured call
    time, and what binds it from the committed counter record -- the scan
    kernel is a chain of 64 dependent chunk steps per (sequence, head) that
    keeps its compute units' matrix cores busy about a fifth of the time."""
    rec, kern = record_summary("prefill_B4_T4096_H16_record.json")
    out = {"kernel": "chunk_scan_kernel<128, 64, bf16, true, 2> after chunk_factors_kernel",
           "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "achieved": round(PRE_IO_BYTES / (pre_ms / 1e3) / 1e9, 1),
           "frac": round(PRE_IO_BYTES / (pre_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
           "algorithmic_bytes": PRE_IO_BYTES,
           "binding": "latency of the dependent chunk chain (64 steps per sequence and head)",
           "record": None, "traffic": None}
    if rec is None:
        return out
    out["record"] = "profiles/prefill_B4_T4096_H16_record.json"
    out["traffic"] = rec.get("hbm_bytes_per_launch")
    out["kernel_us_per_launch"] = rec.get("kernel_us_per_launch")
    out["kernels"] = kern
    return out


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by sequence and head with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    import torch
    import gated_delta_rule_100_amd as gdr
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    K, W = args.steps, args.warmup

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.only is not None:
        what = args.only
        if what == "decode":
            r = bench_decode(torch, gdr, K, W)
        elif what == "mtp":
            r = bench_mtp(torch, gdr, K, W)
        elif what == "fixup_long":
            r = bench_fixup_long(torch, gdr, K, W)
        elif what == "copy":  # the counters' calibration: 1 GiB read and written per launch
            src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            r = per_launch(torch, lambda i: dst.copy_(src), K, torch.cuda.current_stream())
        else:
            idx = {"prefill": 2, "varlen": 3, "long": 4, "prefill_cp": 2, "long_cp": 4}[what]
            r = bench_prefill(torch, gdr, K, W, idx, cp_form=what.endswith("_cp"))
        print(json.dumps({"only": what, **_timing(r), "steps": K, "warmup": W}))
        return

    log(f"decode: warmup {W}, steps {K}")
    dec = bench_decode(torch, gdr, K, W)
    log(f"decode {dec}")
    pre = bench_prefill(torch, gdr, K, W)
    log(f"prefill {pre}")
    # figures outside the step
    others = {}
    warm = None
    if not args.no_other_prefill:
        n = max(K, MIN_SAMPLES)
        w = min(W, 2)
        for idx, key in ((3, "prefill_varlen"), (4, "prefill_long")):
            r = bench_prefill(torch, gdr, n, w, idx)
            log(f"{key} {r}")
            others[key] = prefill_line(r, idx)
        for idx, key in ((2, "prefill_cp"), (4, "prefill_long_cp")):
            r = bench_prefill(torch, gdr, n, w, idx, cp_form=True)
            log(f"{key} {r}")
            others[key] = prefill_line(r, idx, lm=True)
        r = bench_fixup_long(torch, gdr, n, w)
        log(f"fixup_long {r}")
        t = r["ms"] / 1e3
        others["fixup_long"] = {
            "workload": "gdr_state_fixup over the long workload's L and M: 2048 dependent chunk "
                        "steps per head, 4 heads, d=128, no initial state",
            **_timing(r), "us_per_step": round(r["ms"] * 1e3 / LONG_CHUNKS, 3),
            "hbm_frac": round(LONG_CHUNKS * LONG_H * FIX_STEP_BYTES / t / 1e9 / HBM_PEAK_GBS, 4)}
        m = bench_mtp(torch, gdr, n, W)
        log(f"decode_mtp {m}")
        t = m["ms"] / 1e3
        others["decode_mtp"] = {
            "workload": f"multi-token decode N=64 T={m['T']} H=32 dk=dv=128 bf16, no per-token states",
            "value": round(DEC_STATE_BYTES / t / 1e9, 2), "unit": "state GB/s",
            "us": round(m["ms"] * 1e3, 2), **_timing(m),
            "tokens_per_s": round(DEC_N * m["T"] / t, 1)}
        # warm figures for context: decode on one state buffer, prefill without the scrub
        dec_w = bench_decode(torch, gdr, n, W, nbuf=1)
        pre_w = bench_prefill(torch, gdr, n, W, cold=False)
        log(f"warm decode {dec_w} prefill {pre_w}")
        warm = {
            "note": "context, not the headline: decode reuses one 128 MiB state buffer (small "
                    "enough for the 256 MB Infinity Cache) and prefill runs back to back "
                    "without the scrub",
            "decode_ms": round(dec_w["ms"], 5),
            "decode_state_gbs": round(DEC_STATE_BYTES / (dec_w["ms"] / 1e3) / 1e9, 2),
            "prefill_ms": round(pre_w["ms"], 5),
            "prefill_tokens_per_s": round(PRE_TOKENS / (pre_w["ms"] / 1e3), 1),
        }
        for key, name in (("prefill_varlen", "prefill_varlen_32768tok_H32_record.json"),
                          ("prefill_long", "prefill_long_T131072_H4_record.json"),
                          ("prefill_cp", "prefill_B4_T4096_H16_LM_record.json"),
                          ("prefill_long_cp", "prefill_long_T131072_H4_LM_record.json"),
                          ("fixup_long", "fixup_long_2048chunks_H4_record.json"),
                          ("decode_mtp", "decode_mtp_N64_T8_H32_d128_record.json")):
            rec, kern = record_summary(name)
            others[key]["record"] = None if rec is None else "profiles/" + name
            if rec is not None:
                others[key]["traffic"] = rec.get("hbm_bytes_per_launch")
                others[key]["kernels"] = kern
                for f in ("phases_us", "segment_fixup_us_per_step"):
                    if f in rec:
                        others[key][f] = rec[f]
    copy_gbs = copy_bandwidth(torch)
    log(f"device copy {copy_gbs:.1f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds)
        log(f"cpu {cpu}")

    dec_s = dec["ms"] / 1e3
    pre_s = pre["ms"] / 1e3
    dec_gbs = DEC_STATE_BYTES / dec_s / 1e9
    achieved = DEC_ALG_BYTES / dec_s / 1e9
    dec_rec = load_record("decode_N64_H32_d128_record.json")
    out = {
        "metric": "GDR decode state GB/s (% HBM peak); chunked-prefill tokens/s at H=16,d=128",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(dec["ms"] + pre["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 inputs, fp32 state and accumulation",
        "data": "synthetic (seeded numpy PCG64; q,k L2-normalised; g=-softplus(N(0,1)); "
                "beta=sigmoid(N(0,1)); S0~N(0,0.02))",
        "config": {"workload": "decode N=64 H=32 dk=dv=128 bf16, state 128 MiB in place "
                               "(cold: 4 rotating buffers) + chunked prefill B=4 T=4096 H=16 "
                               "dk=dv=128 C=64 bf16",
                   "decode_ms": round(dec["ms"], 5), "prefill_ms": round(pre["ms"], 5),
                   "timing": "decode: average launch duration over the timed region of back-to-"
                             "back launches (HIP events on the launch stream); prefill: median of "
                             "per-launch HIP events"},
        "pct_hbm_peak": round(100.0 * dec_gbs / HBM_PEAK_GBS, 2),
        "device_copy_gbs": round(copy_gbs, 1),
        "decode": _timing(dec),
        "prefill": {
            "value": round(PRE_TOKENS / pre_s, 1), "unit": "tokens/s", **_timing(pre),
            "schedule": "chunk factors + sequential chunk scan (factored fixup)",
            "io_min_frac": round(PRE_IO_BYTES / pre_s / 1e9 / HBM_PEAK_GBS, 4),
            "scan_form_frac": round(PRE_SCAN_BYTES / pre_s / 1e9 / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "bound": "hbm", "kernel": "decode_kernel<128,128,bf16,bf16,2> (32 state rows per workgroup)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if dec_rec is None else dec_rec.get("hbm_bytes_per_launch"),
        },
        "prefill_roofline": prefill_roofline(pre["ms"]),
        "cpu_baseline": cpu,
    }
    if warm is not None:
        out["warm"] = warm
    out.update(others)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
