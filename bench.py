#!/usr/bin/env python3
"""Benchmark: exact tiled attention forward + backward on one MI355X.

One step = the whole path on one batch: fa_fwd, then the backward's four
stages (fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq), on synthetic bf16 inputs
already resident in HBM.  Default workload: causal, B=2, H=32, N=8192, d=128
(the shape the targets are stated at), Q/K/V/dO i.i.d. N(0,1).  After it, the
fp8 forward (fa_fwd_fp8) is timed on the same inputs quantised to e4m3
("fwd_fp8"), the dropout forward and backward (p 0.1) on the same inputs
("dropout"), and the split-KV decode (fa_decode) on its own workload
("decode", with its HBM roofline).

Counted FLOPs: forward 4 N^2 d B H, backward 10 N^2 d B H (2.5x forward), both
halved under a causal mask.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--decode NAME|none] [--no-cpu-baseline]
    python bench.py --configs   # one JSON line: every configuration's kernel times, plus the oracle's
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (256 CUs x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
PEAK_F32_TFLOPS = 157.3  # MI355X fp32 vector (the fp32 forward runs on fp32 MFMA, whose dense peak is the same)
KERNEL_SOURCES = ("io_aware_tiled_fwd_amd/csrc/fa_fwd.hip", "io_aware_tiled_fwd_amd/csrc/fa_bwd.hip",
                  "io_aware_tiled_fwd_amd/csrc/fa_common.h")
# Split-KV decode leg: one new token of a Llama-3-70B-like attention layer
# (64 query heads, 8 key/value heads, d 128) at batch 1 over a 131072-token
# cache.  name: (B, Hq, Hkv, Nk, d)
DECODE_WORKLOADS = {
    "decode_b1_hq64_hkv8_nk131072_d128": (1, 64, 8, 131072, 128),
    "decode_b8_hq64_hkv8_nk32768_d128": (8, 64, 8, 32768, 128),
}
DEFAULT_DECODE = "decode_b1_hq64_hkv8_nk131072_d128"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_causal_b2_h32_n8192_d128.json")

WORKLOADS = {
    # name: (B, H, N, d, causal)
    "causal_fwdbwd_b2_h32_n8192_d128": (2, 32, 8192, 128, True),
    "causal_fwdbwd_b4_h16_n4096_d128": (4, 16, 4096, 128, True),
    "fwdbwd_b4_h16_n2048_d64": (4, 16, 2048, 64, False),
    "fwdbwd_b1_h16_n18000_d128": (1, 16, 18000, 128, False),
}
DEFAULT_WORKLOAD = "causal_fwdbwd_b2_h32_n8192_d128"


def counted_flops(B, H, N, d, causal):
    f = 4.0 * N * N * d * B * H * (0.5 if causal else 1.0)
    return f, 2.5 * f


def kernel_flops(B, H, N, d, causal):
    """Algorithmic MFMA FLOPs of each stage per launch: every visible
    (query, key) pair costs 2 d per matrix product the stage performs
    (fwd: S, PV; dK/dV: S, dP, dV, dK at d = 128, where one kernel of paired
    wavefronts computes S once, and S twice at d = 64, where the dV and dK
    kernels run; dQ: S, dP, dQ)."""
    pairs = N * N * B * H * (0.5 if causal else 1.0)
    return {"fwd": 2 * 2 * d * pairs, "bwd_dkdv": (4 if d == 128 else 5) * 2 * d * pairs,
            "bwd_dq": 3 * 2 * d * pairs, "bwd_preprocess": 2.0 * N * d * B * H}


def kernel_bytes(B, H, N, d):
    """Compulsory HBM bytes per launch (each tensor read or written once)."""
    t = 2.0 * B * H * N * d  # one bf16 [B,H,N,d] tensor
    f = 4.0 * B * H * N * d  # one fp32 [B,H,N,d] tensor
    r = 4.0 * B * H * N      # one fp32 [B,H,N] vector
    return {"fwd": 4 * t + r, "bwd_preprocess": 2 * t + r, "bwd_dkdv": 4 * t + 2 * r + 2 * f,
            "bwd_dq": 4 * t + 2 * r + f}


def kernel_source_hash():
    """sha256 over the kernel sources: a recorded HBM-traffic figure is only
    reported while the kernels it was measured on are unchanged."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (scaled by the plain-copy calibration), or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch", {}).get(kernel)


def copy_calibration(mib):
    """A plain device copy of a known size, for calibrating the byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)
    return 0


def timed_rounds(calls, iters, rounds=3, gap_s=0.05):
    """Per-iteration HIP-event times of `calls` (a list of callables run in
    order each iteration, each timed separately) over `rounds` rounds of
    `iters` iterations, a short pause between rounds.  Returns (the per-call
    medians of the middle round by summed median, every round's medians).
    On some boxes one stretch of a run occasionally went about 2.4x slower
    throughout while a standalone timing was normal; the middle of three
    rounds keeps one such stretch, or one unusually fast round, from setting
    the figure, and the list of all rounds keeps it visible."""
    import time

    import numpy as np
    import torch

    stream = torch.cuda.current_stream()
    per_round = []
    for r in range(rounds):
        if r:
            time.sleep(gap_s)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(iters)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record(stream)
            for j, c in enumerate(calls):
                c()
                e[j + 1].record(stream)
        torch.cuda.synchronize()
        per_round.append([float(np.median([e[j].elapsed_time(e[j + 1]) for e in ev])) for j in range(len(calls))])
    mid = sorted(per_round, key=sum)[len(per_round) // 2]
    return mid, per_round


def fp8_leg(t, B, H, N, d, causal, scale, iters=10, warmup=3):
    """Time fa_fwd_fp8 on the step's own Q, K, V quantised on the device to
    OCP e4m3 with one factor per tensor (max |x| / 448); HIP events on the
    launch stream.  FLOPs counted as for the bf16 forward."""
    import numpy as np
    import torch

    from io_aware_tiled_fwd_amd import binding

    q8, ds = {}, {}
    for n in ("q", "k", "v"):
        x = t[n].float()
        ds[n] = float(x.abs().max()) / 448.0
        q8[n] = (x / ds[n]).to(torch.float8_e4m3fn)
        del x
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        binding.fa_fwd_fp8(q8["q"], q8["k"], q8["v"], o, lse, ds["q"], ds["k"], ds["v"], causal, scale, stream)

    for _ in range(warmup):
        call()
    (ms,), rounds = timed_rounds([call], iters)
    ff, _ = counted_flops(B, H, N, d, causal)
    tf = ff / (ms / 1e3) / 1e12
    return {"ms_median": round(ms, 4), "round_medians_ms": [round(r[0], 4) for r in rounds], "tflops": round(tf, 2),
            "frac_peak_fp8": round(tf / PEAK_FP8_TFLOPS, 4),
            "inputs": "the step's Q, K, V quantised on the device to e4m3, one factor per tensor"}


def dropout_leg(t, B, H, N, d, causal, scale, p=0.1, iters=5, warmup=2):
    """Time fa_fwd_dropout and fa_bwd_dropout (dropout p, Philox mask) on the
    step's inputs; HIP events on the launch stream; FLOPs counted as for the
    plain step."""
    import numpy as np
    import torch

    from io_aware_tiled_fwd_amd import binding

    o = torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)
    stream = torch.cuda.current_stream()

    def fwd():
        binding.fa_fwd_dropout(t["q"], t["k"], t["v"], o, lse, p, 2026, 0, causal, scale, stream)

    def bwd():
        binding.fa_bwd_dropout(t["q"], t["k"], t["v"], o, lse, t["do"], dq, dk, dv, delta, p, 2026, 0, causal,
                               scale, stream)

    for _ in range(warmup):
        fwd()
        bwd()
    (fms, bms), rounds = timed_rounds([fwd, bwd], iters)
    ff, fb = counted_flops(B, H, N, d, causal)
    return {"p": p, "fwd_ms": round(fms, 4), "bwd_ms": round(bms, 4),
            "round_medians_ms": [[round(x, 4) for x in r] for r in rounds],
            "fwd_tflops": round(ff / (fms / 1e3) / 1e12, 2), "bwd_tflops": round(fb / (bms / 1e3) / 1e12, 2)}


def decode_leg(name, iters=20, warmup=5):
    """Time fa_decode (split kernel + merge kernel) with HIP events on the
    launch stream; rate = compulsory bytes (K, V, q, o, L once) / median time
    (the middle of three rounds, see timed_rounds)."""
    import numpy as np
    import torch

    from io_aware_tiled_fwd_amd import binding, inputs

    B, Hq, Hkv, Nk, d = DECODE_WORKLOADS[name]
    ts = inputs.decode_qkv(B, Hq, Hkv, Nk, d, seed=20284, with_f64=False)
    t = {n: torch.from_numpy(ts.bits[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ts.names}
    del ts
    splits, ws_bytes = binding.fa_decode_plan(B, Hq, Hkv, Nk, d)
    ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device="cuda") if ws_bytes else None
    o = torch.empty_like(t["q"])
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    scale = inputs.default_scale(d)

    def call():
        binding.fa_decode(t["q"], t["k"], t["v"], o, lse, workspace=ws, scale=scale, stream=stream)

    for _ in range(warmup):
        call()
    (ms,), rounds = timed_rounds([call], iters)
    med_us = ms * 1e3
    nbytes = 2 * B * Hkv * Nk * d * 2 + 2 * B * Hq * d * 2 + 4 * B * Hq
    gbs = nbytes / (med_us / 1e6) / 1e9
    return {"workload": name, "B": B, "Hq": Hq, "Hkv": Hkv, "Nk": Nk, "d": d, "splits": splits,
            "us_median": round(med_us, 2), "round_medians_us": [round(r[0] * 1e3, 2) for r in rounds],
            "bytes_compulsory": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def probe_leg(mfma_blocks=1024, mfma_iters=2000, read_mib=1024, reps=3):
    """Measured ceilings beside the published peaks: the library's bf16 MFMA
    loop and its non-temporal HBM read sweep (include/fa_probe.h), timed with
    HIP events on the launch stream (best of `reps` after one warm-up).  The
    roofline fractions above stay against the published peaks."""
    import torch

    from io_aware_tiled_fwd_amd import binding

    stream = torch.cuda.current_stream()

    def best_ms(call):
        call()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    sink = torch.empty(mfma_blocks * 512, dtype=torch.float32, device="cuda")
    ms = best_ms(lambda: binding.fa_probe_mfma(mfma_blocks, mfma_iters, sink, stream))
    tflops = mfma_blocks * 8 * mfma_iters * 16 * 32768 / (ms / 1e3) / 1e12
    nbytes = read_mib * 2**20 // binding.PROBE_READ_UNIT * binding.PROBE_READ_UNIT
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    rsink = torch.empty(256 * 512, dtype=torch.int32, device="cuda")
    ms_r = best_ms(lambda: binding.fa_probe_hbm_read(buf, rsink, stream))
    del buf
    return {"mfma_bf16_tflops": round(tflops, 1), "hbm_read_gbs": round(nbytes / (ms_r / 1e3) / 1e9, 1),
            "how": f"{mfma_blocks} workgroups x 8 waves of v_mfma_f32_32x32x16_bf16 on four chains; "
                   f"{nbytes >> 20} MiB read once with 16-byte non-temporal loads (fa_probe.h)"}


def config_table(iters=30, warmup=10, oracle=True):
    """Every workload of the parity tests (inputs.WORKLOADS: the five configurations),
    each on its own seeded inputs: GPU time of the forward (and of the backward
    where the workload has one, plus the causal B2 H32 N8192 backward), the
    counted TFLOP/s and fraction of the 2.5 PF bf16 peak; beside it the oracle's
    time on a sample of the same inputs (all heads of the two small workloads,
    the parity tests' four sampled heads otherwise), with the full-workload time
    extrapolated by head count.  Returns {workload: {...}}."""
    import numpy as np
    import torch

    import oracle
    from io_aware_tiled_fwd_amd import binding, inputs

    stream = torch.cuda.current_stream()
    out = {}
    for name, w in inputs.WORKLOADS.items():
        B, H, N, d, causal, dt = w["B"], w["H"], w["N"], w["d"], w["causal"], w["dtype"]
        with_bwd = bool(w.get("backward")) or name.startswith("c3")
        ts = inputs.normal_qkv(B, H, N, d, w["seed"], dtype=dt, with_dout=with_bwd and dt == "bf16")
        if dt == "bf16":
            t = {n: torch.from_numpy(ts.bits[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ts.names}
        else:
            t = {n: torch.from_numpy(ts.bits[n]).cuda() for n in ts.names}
        scale = inputs.default_scale(d)
        o = torch.empty_like(t["q"])
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        fwd = binding.fa_fwd_f32 if dt == "f32" else binding.fa_fwd
        calls = [lambda: fwd(t["q"], t["k"], t["v"], o, lse, causal, scale, stream)]
        if with_bwd:
            g = [torch.empty((B, H, N, d), dtype=torch.float32, device="cuda") for _ in range(3)]
            delta = torch.empty_like(lse)
            calls.append(lambda: binding.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], *g, delta, causal, scale,
                                                stream))
        for _ in range(warmup):
            for c in calls:
                c()
        meds, _ = timed_rounds(calls, iters)
        ff, fb = counted_flops(B, H, N, d, causal)
        rec = {"B": B, "H": H, "N": N, "d": d, "causal": causal, "dtype": dt,
               "fwd_ms": round(meds[0], 4), "fwd_tflops": round(ff / (meds[0] / 1e3) / 1e12, 2),
               "fwd_frac_peak": None if dt == "f32" else round(ff / (meds[0] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        if dt == "f32":
            rec["fwd_frac_peak_fp32"] = round(ff / (meds[0] / 1e3) / 1e12 / PEAK_F32_TFLOPS, 4)
        if with_bwd:
            rec.update({"bwd_ms": round(meds[1], 4), "bwd_tflops": round(fb / (meds[1] / 1e3) / 1e12, 2),
                        "bwd_frac_peak": round(fb / (meds[1] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
        del t, o, lse, calls
        if with_bwd:
            del g, delta
        torch.cuda.empty_cache()
        if oracle:
            heads = list(range(B * H)) if B * H <= 64 and N <= 2048 else inputs.sample_heads(B * H, 4, w["seed"] + 1000)
            arr = {n: ts.f64[n].reshape(B * H, N, d)[heads] for n in ts.names}
            t0 = time.perf_counter()
            oracle.attn_fwd(arr["q"], arr["k"], arr["v"], scale, causal)
            t1 = time.perf_counter()
            rec["oracle_fwd_s"] = round(t1 - t0, 3)
            if with_bwd:
                oracle.attn_bwd(arr["q"], arr["k"], arr["v"], arr["do"], scale, causal)
                rec["oracle_bwd_s"] = round(time.perf_counter() - t1, 3)
            rec["oracle_heads"] = len(heads)
            rec["oracle_full_s"] = round((time.perf_counter() - t0) * (B * H) / len(heads), 1)
            rec["oracle_threads"] = oracle.default_threads()
        del ts
        out[name] = rec
        print(json.dumps({name: rec}), file=sys.stderr, flush=True)
    return out


def cpu_baseline(heads, causal):
    """The fp64 oracle, as it stands, on host cores: forward + backward of the
    first few heads of the benchmark's own inputs (batch 0), each over all N
    positions.  Rate = counted FLOPs of that sample / wall time."""
    import oracle
    from io_aware_tiled_fwd_amd import inputs

    nh, n, d = heads["q"].shape
    arr = [heads[x] for x in ("q", "k", "v", "do")]
    scale = inputs.default_scale(d)
    threads = oracle.default_threads()
    oracle.attn_fwd(arr[0][:1, :8], arr[1][:1, :8], arr[2][:1, :8], scale, causal)  # load the library
    t0 = time.perf_counter()
    oracle.attn_fwd(*arr[:3], scale, causal, threads=threads)
    oracle.attn_bwd(*arr, scale, causal, threads=threads)
    dt = time.perf_counter() - t0
    ff, fb = counted_flops(1, nh, n, d, causal)
    return {"value": (ff + fb) / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"batch 0, heads 0..{nh - 1} of the same inputs (N={n}, d={d}), "
                       f"{'causal ' if causal else ''}fwd+bwd in fp64; {dt:.2f} s wall, "
                       f"counted FLOPs {ff + fb:.3e}"),
            "seconds": dt}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (counter calibration)")
    ap.add_argument("--decode", default=DEFAULT_DECODE, choices=sorted(DECODE_WORKLOADS) + ["none"],
                    help="split-KV decode workload timed after the training step ('none' to skip)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 forward leg")
    ap.add_argument("--no-dropout", action="store_true", help="skip the dropout fwd+bwd leg")
    ap.add_argument("--no-probe", action="store_true", help="skip the measured MFMA / HBM-read ceilings")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the step: time every configuration of the parity tests, with the oracle's "
                         "time on a sample of each, and print one JSON line with the table")
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="heads of batch 0 the CPU baseline computes (about 10-20 s)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the forward and backward shard by (batch, head) with no communication).",
              file=sys.stderr)
        return 2

    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.configs:
        from io_aware_tiled_fwd_amd import binding
        binding.load_library()
        table = config_table(oracle=not args.no_cpu_baseline)
        print(json.dumps({"configs": table, "peak_bf16_tflops": PEAK_BF16_TFLOPS}), flush=True)
        return 0

    import numpy as np
    import torch

    from io_aware_tiled_fwd_amd import binding, inputs

    binding.load_library()
    B, H, N, d, causal = WORKLOADS[args.workload]
    scale = inputs.default_scale(d)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ts = inputs.normal_qkv(B, H, N, d, seed=20263, with_dout=True)
    t = {n: torch.from_numpy(ts.bits[n].view(np.int16)).view(torch.bfloat16).to(dev) for n in ts.names}
    cpu_heads = {n: ts.f64[n][0, :max(1, min(args.cpu_heads, H))].copy() for n in ts.names}
    del ts
    o = torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)
    stream = torch.cuda.current_stream()
    names = ["fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq"]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        binding.fa_fwd(t["q"], t["k"], t["v"], o, lse, causal, scale, stream)
        if ev is not None:
            ev[1].record(stream)
        binding.fa_bwd_preprocess(o, t["do"], delta, stream)
        if ev is not None:
            ev[2].record(stream)
        binding.fa_bwd_dkdv(t["q"], t["k"], t["v"], lse, t["do"], delta, dk, dv, causal, scale, stream)
        if ev is not None:
            ev[3].record(stream)
        binding.fa_bwd_dq(t["q"], t["k"], t["v"], lse, t["do"], delta, dq, causal, scale, stream)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {n: [] for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]))
    med = {n: float(np.median(per[n])) for n in names}
    avg = {n: float(np.mean(per[n])) for n in names}

    ms_step = wall / args.steps * 1e3
    ff, fb = counted_flops(B, H, N, d, causal)
    value = (ff + fb) / (ms_step / 1e3) / 1e12
    bwd_ms = sum(med[n] for n in names if n.startswith("bwd_"))
    kflops = kernel_flops(B, H, N, d, causal)
    kbytes = kernel_bytes(B, H, N, d)
    kernels = {n: {"ms_median": round(med[n], 4), "ms_mean": round(avg[n], 4),
                   "ms_p10": round(float(np.percentile(per[n], 10)), 4),
                   "ms_p90": round(float(np.percentile(per[n], 90)), 4),
                   "tflops": round(kflops[n] / (avg[n] / 1e3) / 1e12, 2),
                   "gbs_compulsory": round(kbytes[n] / (avg[n] / 1e3) / 1e9, 1)} for n in names}
    dominant = max(("fwd", "bwd_dkdv", "bwd_dq"), key=lambda n: avg[n])
    achieved = kflops[dominant] / (avg[dominant] / 1e3) / 1e12

    out = {
        "metric": "attention fwd/bwd TFLOP/s at B,H,N,d + % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: Q, K, V, dO i.i.d. N(0,1), bf16 (RNE), seed 20263",
        "config": {"workload": args.workload, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                   "scale": scale, "flops_per_step_counted": ff + fb},
        "fwd": {"tflops": round(ff / (med["fwd"] / 1e3) / 1e12, 2),
                "frac_peak": round(ff / (med["fwd"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "ms": round(med["fwd"], 4)},
        "bwd": {"tflops": round(fb / (bwd_ms / 1e3) / 1e12, 2),
                "frac_peak": round(fb / (bwd_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "ms": round(bwd_ms, 4)},
        "step_frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernels": kernels,
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(dominant, args.workload)},
        "peak_bf16_tflops": PEAK_BF16_TFLOPS,
    }
    del o, lse, delta, dq, dk, dv
    if not args.no_fp8:
        out["fwd_fp8"] = fp8_leg(t, B, H, N, d, causal, scale)
    if not args.no_dropout:
        out["dropout"] = dropout_leg(t, B, H, N, d, causal, scale)
    del t
    if args.decode != "none":
        out["decode"] = decode_leg(args.decode)
    if not args.no_probe:
        out["measured_ceilings"] = probe_leg()
    if not args.no_cpu_baseline:
        cb = cpu_baseline(cpu_heads, causal)
        out["cpu_baseline"] = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in cb.items()
                               if k != "seconds"}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
