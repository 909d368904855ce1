#!/usr/bin/env python3
"""Benchmark of the bit-nested quantized linear on one MI355X.

Workload: the 7B/8B-class projections (4096x4096, 1024x4096, 14336x4096,
4096x14336), 2-bit base + 6-bit residual with fp16 group-128 scales, bf16
N(0,1) activations.  One step = draft and verify passes over all four
projections at T = 1, 4, 8, 16 and 32 draft-tree tokens (40 calls), captured
in one HIP graph.  Weights rotate through a pool of distinct copies larger
than the 256 MB Infinity Cache, so every call streams its weights from HBM.

value = effective weight GB/s of a step (algorithmic bytes: codes + fp16
scales, 0.265625 B/weight draft, 1.03125 B/weight verify, over the step's
time).  Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

SHAPES = [("q/o", 4096, 4096), ("k/v", 1024, 4096), ("gate/up", 14336, 4096), ("down", 4096, 14336)]
TS = [1, 4, 8, 16, 32]
BITS = 6
HBM_PEAK_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--pool-gib", type=float, default=1.2)
    ap.add_argument("--reps", type=int, default=10, help="graph replays per per-case timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU path only; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_nested_quantized_amd as nl
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    nl.lib()
    dev = "cuda"
    torch.cuda.set_device(0)

    # ---- weights: one synthetic linear per shape, repacked into a pool of copies
    set_bytes = sum(o * i for _, o, i in SHAPES) * synth.bytes_per_weight(BITS)
    ncopy = max(2, math.ceil(args.pool_gib * 2 ** 30 / set_bytes))
    lins, handles, xs, wss, ys = [], [], [], [], []
    t0 = time.time()
    for si, (name, o, i) in enumerate(SHAPES):
        lin = synth.make_linear(o, i, BITS, cfg=1, idx=si)
        lins.append(lin)
        d = {k: (None if lin[k] is None else torch.from_numpy(np.ascontiguousarray(lin[k]).view(dt)).to(dev))
             for k, dt in [("base_codes", np.uint8), ("base_scales", np.int16), ("resid_codes", np.uint8),
                           ("resid_scales", np.int16), ("sign_in", np.int8), ("sign_out", np.int8)]}
        handles.append([nl.nested_linear_create(o, i, BITS, levels=lin["levels"], **d) for _ in range(ncopy)])
        del d
        xs.append(torch.from_numpy(synth.make_x(max(TS), i, cfg=1, idx=si).view(np.int16)).to(dev))
        wss.append(torch.zeros(nl.nested_linear_workspace_bytes(handles[-1][0], max(TS)), dtype=torch.uint8,
                               device=dev))
        ys.append(torch.empty((max(TS), o), dtype=torch.float32, device=dev))
        log(f"[bench] {name} {o}x{i}: {ncopy} copies created ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()

    def bpw(verify):
        return synth.bytes_per_weight(BITS if verify else 0)

    def call(si, copy, T, verify, stream):
        fn = nl.nested_linear_verify if verify else nl.nested_linear_draft
        fn(handles[si][copy], xs[si], T, ys[si], wss[si], stream)

    # ---- the step: 40 calls, weights rotating through the pool
    seq, c = [], 0
    for T in TS:
        for verify in (True, False):
            for si in range(len(SHAPES)):
                seq.append((si, c % ncopy, T, verify))
                c += 1
    step_bytes = sum(SHAPES[si][1] * SHAPES[si][2] * bpw(v) for si, _, _, v in seq)

    def capture(calls):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for cl in calls:
                call(*cl, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream()
            for cl in calls:
                call(*cl, stream=cs)
        return g

    g = capture(seq)
    # replay check: a replay reproduces the eager outputs bit for bit
    eager = [y.clone() for y in ys]
    for y in ys:
        y.zero_()
    g.replay()
    torch.cuda.synchronize()
    for a, b in zip(eager, ys):
        assert torch.equal(a, b), "graph replay differs from eager run"

    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(args.steps):
        g.replay()
    e1.record()
    e1.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] step: {ms_per_step:.3f} ms, {value:.1f} GB/s ({args.steps} steps)")

    # ---- per case: graphs of `ncopy` calls of one (shape, mode, T), amortised launches
    per_case = {}
    for T in TS:
        for verify in (True, False):
            tot_us, tot_b = 0.0, 0.0
            shp = {}
            for si, (name, o, i) in enumerate(SHAPES):
                gc = capture([(si, cp, T, verify) for cp in range(ncopy)])
                gc.replay()
                torch.cuda.synchronize()
                e0.record()
                for _ in range(args.reps):
                    gc.replay()
                e1.record()
                e1.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (args.reps * ncopy)
                b = o * i * bpw(verify)
                shp[name] = {"us": round(us, 2), "GBps": round(b / us / 1e3, 1)}
                tot_us += us
                tot_b += b
                del gc
            key = f"{'verify' if verify else 'draft'}_T{T}"
            per_case[key] = {"us_per_pass": round(tot_us, 2), "GBps": round(tot_b / tot_us / 1e3, 1),
                             "frac_hbm_peak": round(tot_b / tot_us / 1e3 / HBM_PEAK_GBPS, 3), "shapes": shp}
            log(f"[bench] {key}: {tot_us:.1f} us per pass over the 4 projections, "
                f"{tot_b / tot_us / 1e3:.0f} GB/s")

    # ---- roofline of the dominant kernel: the verify contraction (T <= 16),
    # per-launch HIP events on the launch stream, eager launches
    stream = torch.cuda.current_stream()
    evs, launches = [], []
    for si, (name, o, i) in enumerate(SHAPES):
        for T in (1, 4, 8, 16):
            nl.nested_linear_prepare_input(handles[si][0], xs[si], T, wss[si], stream)
            for r in range(2):
                for cp in range(ncopy):
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    nl.nested_linear_contract(handles[si][cp], True, T, ys[si], wss[si], stream)
                    b.record(stream)
                    evs.append((a, b))
                    launches.append(o * i * bpw(True))
    torch.cuda.synchronize()
    durs = [a.elapsed_time(b) * 1e3 for a, b in evs]  # us
    avg_us = sum(durs) / len(durs)
    avg_bytes = sum(launches) / len(launches)
    achieved = avg_bytes / avg_us / 1e3
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                "kernel": "gemm_kernel<6,1> (verify contraction, T<=16)",
                "avg_launch_us": round(avg_us, 2), "avg_algorithmic_bytes": int(avg_bytes),
                "launches": len(durs)}
    log(f"[bench] roofline gemm_kernel<6,1>: {avg_us:.2f} us/launch, {achieved:.0f} GB/s")

    # ---- streaming reference on the same GPU (torch reduction over 2 GiB)
    big = torch.ones(2 ** 29, dtype=torch.float32, device=dev)
    big.sum()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        big.sum()
    e1.record()
    e1.synchronize()
    stream_gbps = 5 * big.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del big

    # ---- CPU baseline: the fp64 oracle on the same step's calls, host cores
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        xh = [synth.make_x(max(TS), i, cfg=1, idx=si) for si, (_, o, i) in enumerate(SHAPES)]
        log(f"[bench] cpu baseline: oracle on one step (40 calls), {oracle.num_threads()} threads")
        t0 = time.time()
        for si, _, T, verify in seq:
            oracle.forward(lins[si], xh[si][:T], verify)
        dt = time.time() - t0
        cpu = {"value": round(step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": f"one full step (40 calls, {step_bytes / 1e9:.2f} GB of weights) "
                                           f"in {dt:.1f} s"}
        log(f"[bench] cpu baseline: {dt:.1f} s, {cpu['value']} GB/s")

    out = {
        "metric": "effective weight GB/s of draft+verify passes (us per pass vs T in per_case)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16-mfma/fp32", "data": "synthetic",
        "config": {"workload": "7B/8B-class projections 4096x4096, 1024x4096, 14336x4096, 4096x14336; "
                               "2-bit Lloyd-Max base + 6-bit residual, fp16 group-128 scales; bf16 x; "
                               "draft and verify at T=1,4,8,16,32; two-sided rotation",
                   "calls_per_step": len(seq), "weight_bytes_per_step": int(step_bytes),
                   "pool_copies": ncopy, "pool_bytes": int(ncopy * set_bytes)},
        "per_case": per_case,
        "stream_read_GBps_torch_sum": round(stream_gbps, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
