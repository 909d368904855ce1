#!/usr/bin/env python3
"""Benchmark of the bit-nested quantized linear on one MI355X.

Workload of the headline: the 7B/8B-class projections (4096x4096, 1024x4096,
14336x4096, 4096x14336), 2-bit Lloyd-Max base + 6-bit residual with fp16
group-128 scales, bf16 N(0,1) activations, one-sided y = (Q_b + Q_r) H S x.
One step = a verify pass over the four projections at each of T = 1, 4, 8,
16 and 32 draft-tree tokens (20 calls, one kernel launch each), captured in
one HIP graph.  Weights rotate through a pool of distinct copies larger than
the 256 MB Infinity Cache, so every call streams its weights from HBM.
Inputs are resident in HBM before the timed region.

value = effective weight GB/s of the verify step: algorithmic bytes (codes +
fp16 scales, 1.03125 B/weight at 6 bits) over the step time.  per_case gives,
for verify and draft at T = 1, 4, 8, 16, 32 and 64, the microseconds per pass
over the four projections (median, p10, p90 over graph replays), the weight
GB/s and its fraction of the 8 TB/s peak and of the measured streaming-read
reference, and max|dy| / max|y_oracle| of that case on sampled rows.  Further
rows: the 1024x1024 int8 linear, the two-sided form, one decoder layer with
q/k/v and gate/up fused into one launch each, whole Llama-8B-shaped and
31B-class passes, the MoE block (correlated and iid routing), and the NEXT
formats (W4/W8 planes, draft tree, nested KV, encoder).
Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SHAPES = [("q/o", 4096, 4096), ("k/v", 1024, 4096), ("gate/up", 14336, 4096), ("down", 4096, 14336)]
STEP_TS = [1, 4, 8, 16, 32]
CASE_TS = [1, 4, 8, 16, 32, 64]
BITS = 6
HBM_PEAK_GBPS = 8000.0
LAYERS = 32             # decoder layers of the 7B/8B-class model
ERR_ROWS = 512          # output rows per projection checked against the oracle in each case
FWD_SOURCES = ("nl_fwd.hip", "nl_fwd.h", "nl_dev.h", "nl_layout.h", "nl_kernels.hip", "nl_kernels.h")
# mode -> (kernel, bits, the T of its launches, traffic summary).  The verify
# step's largest share of time is the single launch at T = 4 and 8; the draft
# (not in the step) runs the staged-x' launch at every T.
ROOF = {
    "verify": ("fwd_kernel<6, 1, 12, false>", 6, (4, 8),
               os.path.join(ROOT, "profiles", "fwd_kernel_6bit_verify_T4_T8_proj7b8b_traffic.txt")),
    "draft": ("forward_kernel<0, 1, 4>", 0, (8, 16),
              os.path.join(ROOT, "profiles", "forward_kernel_draft_T8_T16_proj7b8b_traffic.txt")),
}
UTIL_FILE = os.path.join(ROOT, "profiles", "forward_utilisation_roofline_launches_proj7b8b.txt")
STREAM_BYTES = 4 << 30  # streaming-read reference buffer (16x the Infinity Cache)
ENC_BITS = 7            # the encoder leg writes 7-bit residuals (the post's bf16-noise-floor width)
ENC_KERNEL = "tile_kernel<0, 7,"   # fused 7-bit encode, any block size (kernel-name match)
ENC_KERNEL_NAME = "tile_kernel<0, 7, LOG2B>"
ENC_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "encoder_tile_kernel_7bit_fused_proj7b8b_traffic.txt")
FIT_ROWS = 512          # 512 x 4096 = 2^21 samples, the post's ~2M
W48_TS = (1, 16, 64)
W48_KERNEL = "w48_kernel<true, 1, 8>"   # verify, one 16-token tile, 128-row workgroups
W48_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w48_kernel_verify_T16_proj7b8b_traffic.txt")
W48_SOURCES = ("nl_w4w8.hip",)
KV_KERNEL = "kv_attn_mfma_kernel<true, false>"   # verify attention over KV8, query rows split over waves
KV_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kv_attn_mfma_kernel_verify_T16_L32768_traffic.txt")
KV_SOURCES = ("nl_kv.hip",)
KV_TITLE = ("verify over KV8, 16-token tree, 32768 context positions, 32 query heads over 8 KV heads,\n"
            "d = 128; algorithmic bytes: the K and V planes and scales read, 69239808 per launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest(files=FWD_SOURCES):
    """Digest of the kernel sources, to tie stored counter readings to them."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "bit_nested_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


ENC_SOURCES = ("nl_encode.hip",)


def stored_traffic(digest, path):
    """HBM bytes per launch of a kernel from its committed counter summary,
    when the summary was taken on the current kernel sources."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel source digest:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm bytes per launch:\s*([0-9.]+)", text)
    if not m_src or not m_val or m_src.group(1) != digest:
        return None
    return float(m_val.group(1))


def pstats(samples):
    """Median, p10 and p90 of a list of microsecond samples."""
    import numpy as np
    a = np.asarray(samples, np.float64)
    return {"us": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "samples": int(a.size)}


def replay_samples(torch, g, reps):
    """Per-replay microseconds of a captured graph: one event pair around each
    of `reps` back-to-back replays (after one untimed replay)."""
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def capture(torch, fn):
    """fn(stream) once eagerly on a side stream (warm-up), then captured."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(torch.cuda.current_stream())
    return g


def rate(bytes_, us, stream_gbps):
    gbps = bytes_ / us / 1e3
    return {"GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "frac_stream_ref": None if not stream_gbps else round(gbps / stream_gbps, 4)}


def rel_err(y, ref):
    import numpy as np
    return float(np.abs(y.astype(np.float64) - ref).max() / max(float(np.abs(ref).max()), 1e-300))


def dev_arrays(torch, lin):
    import numpy as np
    return {k: (None if lin[k] is None else torch.from_numpy(np.ascontiguousarray(lin[k]).view(dt)).cuda())
            for k, dt in [("base_codes", np.uint8), ("base_scales", np.int16), ("resid_codes", np.uint8),
                          ("resid_scales", np.int16), ("sign_in", np.int8), ("sign_out", np.int8)]}


def check_status(nl, ws, what):
    """A wait that gave up would leave NaN outputs and a nonzero error word."""
    e = nl.nested_linear_workspace_status(ws)
    if e:
        raise SystemExit(f"bench: {e} wait(s) gave up in {what}")


# --- the streaming-read reference ---------------------------------------------

def stream_ref_leg(nl, torch, reps=8):
    """Read rate of a plain hand-written streaming-read kernel (16-byte
    nontemporal loads, nothing computed) over a 4 GiB buffer: the measured
    ceiling the weight streams are set against."""
    src = torch.ones(STREAM_BYTES // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    out = {}
    for grid in (1024, 2048, 4096):
        nl.nested_linear_stream_read(src, sink, grid)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            nl.nested_linear_stream_read(src, sink, grid)
        e1.record()
        e1.synchronize()
        out[grid] = STREAM_BYTES * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, sink
    torch.cuda.empty_cache()
    best = max(out, key=out.get)
    log(f"[bench] streaming-read reference: {out[best]:.0f} GB/s (grid {best})")
    return {"GBps": round(out[best], 1), "frac_hbm_peak": round(out[best] / HBM_PEAK_GBPS, 4),
            "kernel": "stream_read_kernel (16-byte nontemporal loads, 8 per lane in flight, 256 threads)",
            "bytes": STREAM_BYTES, "grid": best, "by_grid": {str(k): round(v, 1) for k, v in out.items()}}


# --- the roofline kernels -------------------------------------------------------

def roofline_leg(nl, call, ncopy, stream, bpw, mode):
    """Roofline of one forward kernel: eager launches over the four
    projections at the T values that select it, each timed by a HIP event
    pair attached to its own dispatch (the library's timing hook), so a
    duration is the kernel's execution as the kernel trace reports it."""
    import torch
    kernel, bits, ts, traffic_file = ROOF[mode]
    verify = mode == "verify"
    if kernel.startswith("fwd_kernel"):
        for _, o, i in SHAPES:
            for T in ts:
                p = nl.nested_linear_describe_call([o], i, bits, False, T)
                assert p["mt"] == 1 and not p["local"] and p["waves"] == 12, (o, i, T, p)
    plan = []
    for si, (name, o, i) in enumerate(SHAPES):
        for T in ts:
            for r in range(2):
                for cp in range(ncopy):
                    plan.append((si, cp, T, o * i * bpw(verify)))
    for si, cp, T, _ in plan[:8]:          # warm the code objects
        call(si, cp, T, verify, stream)
    torch.cuda.synchronize()
    nl.nested_linear_timing_begin(len(plan))
    for si, cp, T, _ in plan:
        call(si, cp, T, verify, stream)
    durs = nl.nested_linear_timing_end(len(plan))
    assert len(durs) == len(plan), (len(durs), len(plan))
    avg_us = sum(durs) / len(durs)
    avg_bytes = sum(b for *_, b in plan) / len(plan)
    achieved = avg_bytes / avg_us / 1e3
    digest = kernel_source_digest()
    traffic = stored_traffic(digest, traffic_file)
    log(f"[bench] roofline {kernel}: {avg_us:.2f} us/launch, {achieved:.0f} GB/s")
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None if traffic is None else round(traffic),
            "kernel": f"{kernel} ({mode}, T = {' and '.join(map(str, ts))}, the four projections)",
            "avg_launch_us": round(avg_us, 2), "avg_algorithmic_bytes": int(avg_bytes),
            "launches": len(durs), "timing": "HIP events attached to each dispatch",
            "kernel_source_digest": digest}


# --- the 1024x1024 int8 linear ----------------------------------------------------

def single1024_leg(nl, torch, synth, reps, stream_gbps, pool_bytes=512 << 20):
    """1024x1024 linear with an int8 residual, verify and draft at T = 1 and
    16; a graph of calls over a pool of copies (so weights come from HBM)."""
    import numpy as np
    import oracle
    lin = synth.make_linear(1024, 1024, 8, cfg=0, idx=0, two_sided=False)
    d = dev_arrays(torch, lin)
    bpw8 = synth.bytes_per_weight(8)
    ncopy = max(2, math.ceil(pool_bytes / (1024 * 1024 * bpw8)))
    hs = [nl.nested_linear_create(1024, 1024, 8, levels=lin["levels"], **d) for _ in range(ncopy)]
    del d
    x = synth.make_x(16, 1024, cfg=0, idx=16)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    ws = torch.zeros(nl.nested_linear_workspace_bytes(hs[0], 16), dtype=torch.uint8, device="cuda")
    y = torch.empty((16, 1024), dtype=torch.float32, device="cuda")
    out = {"workload": "1024x1024, 2-bit base + int8 residual, one-sided", "pool_copies": ncopy}
    for T in (1, 16):
        for verify in (True, False):
            fn = nl.nested_linear_verify if verify else nl.nested_linear_draft
            fn(hs[0], xd, T, y, ws)
            check_status(nl, ws, "1024x1024")
            err = rel_err(y[:T].cpu().numpy(), oracle.forward(lin, x[:T], verify))

            def calls(s):
                for h in hs:
                    fn(h, xd, T, y, ws, s)

            g = capture(torch, calls)
            st = pstats([u / ncopy for u in replay_samples(torch, g, reps)])
            del g
            b = 1024 * 1024 * synth.bytes_per_weight(8 if verify else 0)
            out[f"{'verify' if verify else 'draft'}_T{T}"] = dict(st, **rate(b, st["us"], stream_gbps),
                                                                  max_rel_err=float(f"{err:.3g}"))
            log(f"[bench] 1024x1024 {'verify' if verify else 'draft'} T={T}: {st['us']:.2f} us")
    check_status(nl, ws, "1024x1024")
    for h in hs:
        nl.nested_linear_destroy(h)
    return out


# --- a decoder layer with fused launches ---------------------------------------------

LAYER = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096), ("gate", 14336, 4096),
         ("up", 14336, 4096), ("down", 4096, 14336)]


def make_layer_launches(nl, torch, handles, xs, ys, ws, T, verify):
    """The four launches of one decoder layer: q, k, v fused (one launch on
    the shared input), o, gate and up fused, down.  handles: dict name -> h."""
    single = nl.nested_linear_verify if verify else nl.nested_linear_draft
    multi = nl.nested_linear_verify_multi if verify else nl.nested_linear_draft_multi

    def run(s):
        multi([handles["q"], handles["k"], handles["v"]], xs[4096], T, [ys["q"], ys["k"], ys["v"]], ws, s)
        single(handles["o"], xs[4096], T, ys["o"], ws, s)
        multi([handles["gate"], handles["up"]], xs[4096], T, [ys["gate"], ys["up"]], ws, s)
        single(handles["down"], xs[14336], T, ys["down"], ws, s)
    return run


def layer_workspace_bytes(nl, h, T):
    return max(nl.nested_linear_multi_workspace_bytes([h["q"], h["k"], h["v"]], T),
               nl.nested_linear_multi_workspace_bytes([h["gate"], h["up"]], T),
               nl.nested_linear_workspace_bytes(h["o"], T), nl.nested_linear_workspace_bytes(h["down"], T))


def decoder_layer_leg(nl, torch, synth, reps, stream_gbps, pool_gib):
    """One decoder layer of the 7B/8B-class model, 6-bit: q/k/v fused into one
    launch and gate/up into another (they share their input), o and down
    alone; layers rotate through a pool of copies; verify and draft at T = 1
    and 16 (and verify at 32 and 64)."""
    import numpy as np
    import oracle
    bpw = lambda v: synth.bytes_per_weight(BITS if v else 0)
    layer_bytes = sum(o * i for _, o, i in LAYER) * bpw(True)
    ncopy = max(2, math.ceil(pool_gib * 2 ** 30 / layer_bytes))
    lins = {name: synth.make_linear(o, i, BITS, cfg=5, idx=k, two_sided=False) for k, (name, o, i) in enumerate(LAYER)}
    pool = []
    for _ in range(ncopy):
        pool.append({name: nl.nested_linear_create(lin["d_out"], lin["d_in"], BITS, levels=lin["levels"],
                                                   **dev_arrays(torch, lin)) for name, lin in lins.items()})
    xh = {4096: synth.make_x(64, 4096, cfg=5, idx=100), 14336: synth.make_x(64, 14336, cfg=5, idx=101)}
    xs = {k: torch.from_numpy(v.view(np.int16)).cuda() for k, v in xh.items()}
    ys = {name: torch.empty((64, o), dtype=torch.float32, device="cuda") for name, o, _ in LAYER}
    ws = torch.zeros(layer_workspace_bytes(nl, pool[0], 64), dtype=torch.uint8, device="cuda")
    out = {"linears": "q, k, v fused (4096+1024+1024 x 4096); o 4096x4096; gate, up fused (2 x 14336x4096); "
                      "down 4096x14336; four launches per layer", "layers": LAYERS, "pool_copies": ncopy}
    for T in (1, 16, 32, 64):
        for verify in ((True, False) if T <= 16 else (True,)):
            run0 = make_layer_launches(nl, torch, pool[0], xs, ys, ws, T, verify)
            run0(torch.cuda.current_stream())
            check_status(nl, ws, "decoder layer")
            err = 0.0
            for name, o, i in LAYER:
                ref = oracle.forward(lins[name], xh[i][:T], verify, rows=(0, ERR_ROWS))
                err = max(err, rel_err(ys[name][:T, :ERR_ROWS].cpu().numpy(), ref))
            runs = [make_layer_launches(nl, torch, p, xs, ys, ws, T, verify) for p in pool]
            g = capture(torch, lambda s: [r(s) for r in runs])
            st = pstats([u / ncopy for u in replay_samples(torch, g, reps)])
            del g
            key = f"{'verify' if verify else 'draft'}_T{T}"
            out[key] = dict(st, **rate(sum(o * i for _, o, i in LAYER) * bpw(verify), st["us"], stream_gbps),
                            ms_per_model=round(st["us"] * LAYERS / 1e3, 3), max_rel_err=float(f"{err:.3g}"))
            log(f"[bench] decoder layer {key}: {st['us']:.1f} us ({out[key]['GBps']:.0f} GB/s)")
    check_status(nl, ws, "decoder layer")
    for p in pool:
        for h in p.values():
            nl.nested_linear_destroy(h)
    torch.cuda.empty_cache()
    return out


# --- whole dense-model passes ---------------------------------------------------------

# (name, layer shapes q k v o gate up down, layers, residual bits, verify T, draft T, lm_head shape or None,
# synthetic config id)
MODELS = [
    ("llama8b_shaped", [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096), (14336, 4096),
                        (4096, 14336)], 32, 7, 16, 16, (128256, 4096), 2),
    ("dense31b_class", [(5120, 5120), (1024, 5120), (1024, 5120), (5120, 5120), (25600, 5120), (25600, 5120),
                        (5120, 25600)], 64, 8, 64, 1, None, 3),
]


def model_leg(nl, torch, synth, reps, spec, stream_gbps):
    """Verify and draft passes over every linear weight of a dense model, each
    captured as one graph: per layer q/k/v as one fused launch, o, gate/up as
    one fused launch, down, then the lm_head if there is one.  Every linear
    owns its own device copy of its planes, made from one synthetic linear
    per shape (values do not change the work); an lm_head repeats the codes
    of a generated 4096-row block with per-row scales."""
    import numpy as np
    import oracle
    name, layer, n_layers, bits, t_verify, t_draft, head, cfg = spec

    def make(o, i, idx):
        if (o, i) != head:
            return synth.make_linear(o, i, bits, cfg=cfg, idx=idx, two_sided=False)
        lin = dict(synth.make_linear(4096, i, bits, cfg=cfg, idx=idx, two_sided=False))
        lin["d_out"] = o
        for k in ("base_codes", "resid_codes"):
            lin[k] = np.ascontiguousarray(np.tile(lin[k], (-(-o // 4096), 1, 1))[:o])
        lin["base_scales"] = synth.make_scales(o, i, cfg, idx, synth.STREAM_BASE_SCALE)
        lin["resid_scales"] = synth.make_scales(o, i, cfg, idx, synth.STREAM_RESID_SCALE)
        return lin

    names = ["q", "k", "v", "o", "gate", "up", "down"]
    shapes = sorted(set(layer) | ({head} if head else set()))
    lins = {sh: make(*sh, si) for si, sh in enumerate(shapes)}
    dev = {sh: dev_arrays(torch, lin) for sh, lin in lins.items()}
    layers = [{n: nl.nested_linear_create(o, i, bits, levels=lins[(o, i)]["levels"], **dev[(o, i)])
               for n, (o, i) in zip(names, layer)} for _ in range(n_layers)]
    hh = nl.nested_linear_create(*head, bits, levels=lins[head]["levels"], **dev[head]) if head else None
    del dev
    t_max = max(t_verify, t_draft)
    hidden, inter = layer[0][1], layer[6][1]
    ws_b = layer_workspace_bytes(nl, layers[0], t_max)
    if hh is not None:
        ws_b = max(ws_b, nl.nested_linear_workspace_bytes(hh, t_max))
    ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
    xh = {i: synth.make_x(t_max, i, cfg=cfg, idx=200 + i) for i in sorted({i for _, i in shapes})}
    xs = {i: torch.from_numpy(v.view(np.int16)).cuda() for i, v in xh.items()}
    ys = {n: torch.empty((t_max, o), dtype=torch.float32, device="cuda") for n, (o, _) in zip(names, layer)}
    yh = torch.empty((t_max, head[0]), dtype=torch.float32, device="cuda") if head else None
    seq = [sh for _ in range(n_layers) for sh in layer] + ([head] if head else [])
    out = {"linears": len(seq), "layers": n_layers, "launches_per_pass": 4 * n_layers + (1 if head else 0),
           "workload": f"{name}: {n_layers} layers of q, k, v, o, gate, up, down ("
                       + ", ".join(f"{o}x{i}" for o, i in layer) + ")"
                       + (f" + lm_head {head[0]}x{head[1]}" if head else "")
                       + f", {bits}-bit residual; verify at T = {t_verify}, draft at T = {t_draft}; "
                         "q/k/v and gate/up fused into one launch each; one graph per pass"}
    for verify in (True, False):
        T = t_verify if verify else t_draft
        single = nl.nested_linear_verify if verify else nl.nested_linear_draft
        multi = nl.nested_linear_verify_multi if verify else nl.nested_linear_draft_multi

        def passes(s):
            for L in layers:
                multi([L["q"], L["k"], L["v"]], xs[hidden], T, [ys["q"], ys["k"], ys["v"]], ws, s)
                single(L["o"], xs[hidden], T, ys["o"], ws, s)
                multi([L["gate"], L["up"]], xs[hidden], T, [ys["gate"], ys["up"]], ws, s)
                single(L["down"], xs[inter], T, ys["down"], ws, s)
            if hh is not None:
                single(hh, xs[head[1]], T, yh, ws, s)

        passes(torch.cuda.current_stream())
        check_status(nl, ws, name)
        err = 0.0
        for n, (o, i) in zip(names, layer):      # the last layer's outputs, sampled rows
            ref = oracle.forward(lins[(o, i)], xh[i][:T], verify, rows=(0, ERR_ROWS))
            err = max(err, rel_err(ys[n][:T, :ERR_ROWS].cpu().numpy(), ref))
        if head:
            ref = oracle.forward(lins[head], xh[head[1]][:T], verify, rows=(0, ERR_ROWS))
            err = max(err, rel_err(yh[:T, :ERR_ROWS].cpu().numpy(), ref))
        g = capture(torch, passes)
        st = pstats(replay_samples(torch, g, reps))
        del g
        wb = sum(o * i for o, i in seq) * synth.bytes_per_weight(bits if verify else 0)
        out["verify" if verify else "draft"] = dict({"T": T, "us_per_pass": st["us"], "p10": st["p10"],
                                                     "p90": st["p90"], "weight_bytes": int(wb)},
                                                    **rate(wb, st["us"], stream_gbps),
                                                    max_rel_err=float(f"{err:.3g}"))
    check_status(nl, ws, name)
    for L in layers:
        for h in L.values():
            nl.nested_linear_destroy(h)
    if hh is not None:
        nl.nested_linear_destroy(hh)
    torch.cuda.empty_cache()
    return out


# --- the MoE block -----------------------------------------------------------------------

MOE_EXPERTS, MOE_HIDDEN, MOE_INTER, MOE_TOPK, MOE_T, MOE_BITS = 256, 2048, 512, 8, 16, 8
MOE_ROUTINGS = 8


def moe_leg(nl, torch, synth, reps, stream_gbps):
    """MoE block verify and draft: 256 routed experts (hidden 2048, expert
    intermediate 512) plus one shared expert, top-8 routing of a 16-token
    block, 2-bit base + 8-bit residual.  Gate and up share their input, so
    each expert holds them as one stacked matrix (512 gate rows, then 512 up
    rows) and one grouped call on the block's 16 token rows computes both;
    down is a second grouped call on each pair's own 512-wide row (P rows,
    pair_token = 0..P-1).  Two routings: router logits
    correlated across the block (rho = 0.62, about 47 experts awake) and iid
    (rho = 0, about 102).  Every expert owns its own device copy of its planes
    and passes cycle through 8 routings so the expert set streams from HBM."""
    import numpy as np
    import oracle
    n = MOE_EXPERTS + 1
    shapes = {"gate_up": (2 * MOE_INTER, MOE_HIDDEN), "down": (MOE_HIDDEN, MOE_INTER)}
    groups, handles, lins = {}, [], {}
    for k, (o, i) in shapes.items():
        lin = synth.make_linear(o, i, MOE_BITS, cfg=4, idx=len(groups), two_sided=False)
        lins[k] = lin
        d = dev_arrays(torch, lin)
        hs = [nl.nested_linear_create(o, i, MOE_BITS, levels=lin["levels"], **d) for _ in range(n)]
        handles += hs
        groups[k] = nl.nested_linear_group_create(hs)
        del d
    x_np = synth.make_x(MOE_T, MOE_HIDDEN, cfg=4, idx=100)
    x = torch.from_numpy(x_np.view(np.int16)).cuda()
    out = {"workload": (f"{MOE_EXPERTS} experts + 1 shared, hidden {MOE_HIDDEN}, expert intermediate {MOE_INTER}, "
                        f"top-{MOE_TOPK} of a {MOE_T}-token block, {MOE_BITS}-bit residual; gate and up stacked "
                        f"into one {2 * MOE_INTER}x{MOE_HIDDEN} matrix per expert, one grouped call on the token rows; "
                        f"down: one grouped call on per-pair rows")}
    for rho in (0.62, 0.0):
        routes = []
        for r in range(MOE_ROUTINGS):
            _, pt, off = synth.router_topk(MOE_T, MOE_EXPERTS, MOE_TOPK, rho, cfg=4, idx=r)
            pt = np.concatenate([pt, np.arange(MOE_T, dtype=np.int32)]).astype(np.int32)   # shared expert last
            off = np.concatenate([off, [off[-1] + MOE_T]]).astype(np.int32)
            P = len(pt)
            active = int(np.count_nonzero(np.diff(off)))
            routes.append((torch.from_numpy(pt).cuda(), torch.from_numpy(off).cuda(),
                           torch.arange(P, dtype=torch.int32, device="cuda"), P, active, pt, off))
        Pmax = max(r[3] for r in routes)
        ws = {k: torch.zeros(nl.nested_linear_group_workspace_bytes(g, Pmax), dtype=torch.uint8, device="cuda")
              for k, g in groups.items()}
        # down-projection inputs: one synthetic 512-wide row per pair
        h_np = synth.make_x(Pmax, MOE_INTER, cfg=4, idx=101)
        h = torch.from_numpy(h_np.view(np.int16)).cuda()
        ygu = torch.empty((Pmax, 2 * MOE_INTER), dtype=torch.float32, device="cuda")
        yd = torch.empty((Pmax, MOE_HIDDEN), dtype=torch.float32, device="cuda")
        res = {"active_experts_avg": round(sum(r[4] for r in routes) / MOE_ROUTINGS, 1)}
        for verify in (True, False):
            fn = nl.nested_linear_verify_grouped if verify else nl.nested_linear_draft_grouped

            def passes(s):
                for pt, off, ident, P, *_ in routes:
                    fn(groups["gate_up"], pt, off, P, x, MOE_T, MOE_T, ygu, ws["gate_up"], s)
                    fn(groups["down"], ident, off, P, h, P, MOE_T, yd, ws["down"], s)

            # parity of the first routing (all experts share one synthetic linear per projection)
            pt_d, off_d, ident, P, _, pt_np, off_np = routes[0]
            fn(groups["gate_up"], pt_d, off_d, P, x, MOE_T, MOE_T, ygu, ws["gate_up"])
            fn(groups["down"], ident, off_d, P, h, P, MOE_T, yd, ws["down"])
            for k in ("gate_up", "down"):
                check_status(nl, ws[k], "moe")
            e_g = rel_err(ygu[:P].cpu().numpy(), oracle.forward(lins["gate_up"], x_np[pt_np], verify))
            e_d = rel_err(yd[:P].cpu().numpy(), oracle.forward(lins["down"], h_np[:P], verify))
            g = capture(torch, passes)
            st = pstats([u / MOE_ROUTINGS for u in replay_samples(torch, g, reps)])
            del g
            per_expert = 3 * MOE_INTER * MOE_HIDDEN * synth.bytes_per_weight(MOE_BITS if verify else 0)
            touched = res["active_experts_avg"] * per_expert
            res["verify" if verify else "draft"] = dict({"us_per_block": st["us"], "p10": st["p10"],
                                                         "p90": st["p90"]}, **rate(touched, st["us"], stream_gbps),
                                                        weight_bytes=int(touched),
                                                        max_rel_err=float(f"{max(e_g, e_d):.3g}"))
        for k in ws:
            check_status(nl, ws[k], "moe")
        out[f"rho_{rho}"] = res
        log(f"[bench] moe block rho={rho}: {res['active_experts_avg']} experts, verify "
            f"{res['verify']['us_per_block']} us, draft {res['draft']['us_per_block']} us")
    for g in groups.values():
        nl.nested_linear_group_destroy(g)
    for hnd in handles:
        nl.nested_linear_destroy(hnd)
    torch.cuda.empty_cache()
    return out


def graph_us(torch, fn, reps, calls=10):
    """Average GPU time of fn() (launches only, on the current stream) from
    replays of a graph of `calls` calls, so host-side call overhead is not
    measured; events around the replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps / calls


def tree_leg(nl, torch, synth, reps, cpu_seconds=0.0):
    """The draft tree: best-first build of 64 nodes from 8 x 16 rank
    statistics (one workgroup), and greedy acceptance for a batch of 1024
    sequences sharing that tree (one wave each).  Both are latency work;
    each is timed from replays of a graph of launches."""
    import numpy as np
    D, R, N, B = 8, 16, 64, 1024
    p = synth.make_rank_stats(D, R, cfg=90)
    pd = torch.from_numpy(p).cuda()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t = nl.tree_build(pd, N)
    torch.cuda.synchronize()
    build_us = graph_us(torch, lambda: nl.nested_tree_build(pd, D, R, N, t["parent"], t["depth"], t["rank"],
                                                            t["prio"], t["anc"], t["count"],
                                                            torch.cuda.current_stream()), reps)
    par = t["parent"].cpu().numpy()
    draft, argmax = synth.make_tree_tokens(par, B, cfg=90)
    dd = torch.from_numpy(draft).cuda()
    da = torch.from_numpy(argmax).cuda()
    n, path, bonus = nl.tree_accept(t["parent"], dd, da)
    torch.cuda.synchronize()
    acc_us = graph_us(torch, lambda: nl.nested_tree_accept(t["parent"], N, B, dd, da, n, path, bonus,
                                                           torch.cuda.current_stream()), reps)
    mean_acc = float(n.float().mean().item()) + 1.0
    # expected tokens per check from the statistics: the sum of the node priorities + 1
    out = {"build": {"D": D, "R": R, "N": N, "us": round(build_us, 2)},
           "accept": {"B": B, "N": N, "us_per_batch": round(acc_us, 2),
                      "sequences_per_s": round(B / acc_us * 1e6),
                      "mean_tokens_per_check": round(mean_acc, 3)},
           "expected_tokens_per_check_from_stats": round(float(t["prio"].sum().item()) + 1.0, 3),
           "bound": "latency (one wave per tree or sequence)"}
    if cpu_seconds > 0:
        import oracle.tree as otree
        t0, k = time.time(), 0
        while time.time() - t0 < cpu_seconds:
            otree.build(p, N)
            for b in range(B):
                otree.accept(par, draft[b], argmax[b])
            k += 1
        dt = time.time() - t0
        out["cpu_baseline"] = {"value": round(k * B / dt), "unit": "sequences/s", "cores": 1, "kind": "oracle",
                               "sample": f"{k} build(s) + {k * B} acceptances in {dt:.1f} s"}
    log(f"[bench] tree: build {build_us:.1f} us, accept {acc_us:.1f} us per {B} sequences")
    return out


def kv_case(nl, torch, synth, rng, H_q, H_kv, L, T, verify):
    """Synthetic KV planes and scales, queries and masks of one attention call;
    returns (call, bytes of KV the call reads)."""
    import numpy as np
    P = L + T
    rows = P * H_kv
    kb = torch.from_numpy(rng.integers(0, 256, (rows, 64), dtype=np.uint8)).cuda()
    kr = torch.from_numpy(rng.integers(0, 256, (rows, 64), dtype=np.uint8)).cuda()
    vb = torch.from_numpy(rng.integers(0, 256, (rows, 64), dtype=np.uint8)).cuda()
    vr = torch.from_numpy(rng.integers(0, 256, (rows, 64), dtype=np.uint8)).cuda()
    ks = torch.from_numpy(rng.uniform(0.01, 0.05, rows).astype(np.float32)).cuda()
    vs = torch.from_numpy(rng.uniform(0.01, 0.05, rows).astype(np.float32)).cuda()
    q = torch.from_numpy(synth.make_x(T * H_q, 128, cfg=91, idx=T).view(np.int16)).cuda()
    anc = torch.from_numpy(np.array([(1 << (t + 1)) - 1 for t in range(T)], np.uint64).view(np.int64)).cuda()
    ws = torch.empty(nl.nested_kv_attention_workspace_bytes(T, H_q, H_kv, L), dtype=torch.uint8, device="cuda")
    o = torch.empty((T, H_q, 128), dtype=torch.float32, device="cuda")

    def call():
        nl.nested_kv_attention(q, T, H_q, H_kv, L, kb, kr if verify else None, ks, vb,
                               vr if verify else None, vs, anc, verify, o, ws, torch.cuda.current_stream())
    return call, P * H_kv * 2 * ((128 if verify else 64) + 4)


def kv_leg(nl, torch, synth, reps):
    """Nested KV attention of one Llama-8B-like layer (32 query heads, 8 KV
    heads, d = 128): verify (KV8) of a 16-token tree and a draft step (KV4,
    one token) at 4096 and 32768 context positions, plus the writer for 16
    tokens.  Bytes are the KV rows the call reads (planes and scales); times
    come from graph replays (host call overhead excluded)."""
    import numpy as np
    H_q, H_kv = 32, 8
    rng = np.random.default_rng(91)
    out = {"heads": [H_q, H_kv], "cases": {}}
    for L in (4096, 32768):
        for T, verify in ((16, True), (1, False)):
            call, b = kv_case(nl, torch, synth, rng, H_q, H_kv, L, T, verify)
            us = graph_us(torch, call, reps)
            key = f"{'verify' if verify else 'draft'}_T{T}_L{L}"
            out["cases"][key] = {"us": round(us, 2), "kv_bytes": b, "GBps": round(b / us / 1e3, 1),
                                 "frac_hbm_peak": round(b / us / 1e3 / HBM_PEAK_GBPS, 4)}
            log(f"[bench] kv {key}: {us:.1f} us, {b / us / 1e3:.0f} GB/s of KV")
            del call
    tr = stored_traffic(kernel_source_digest(KV_SOURCES), KV_TRAFFIC_FILE)
    # counter traffic of the verify attention launch at 32768 positions (the
    # combine's partials are written here and read by the second launch)
    out["cases"]["verify_T16_L32768"]["attention_launch_traffic_bytes"] = None if tr is None else round(tr)
    # the writer: K and V of 16 tokens x 8 KV heads
    n = 16 * H_kv
    x = torch.from_numpy(synth.make_x(n, 128, cfg=92).view(np.int16)).cuda()
    rowi = torch.arange(n, dtype=torch.int32, device="cuda")
    base = torch.empty((n, 64), dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(base)
    sc = torch.empty(n, dtype=torch.float32, device="cuda")
    out["write_16_tokens_us"] = round(graph_us(torch, lambda: nl.nested_kv_write(x, n, rowi, base, ref, sc,
                                                                                  torch.cuda.current_stream()),
                                               reps), 2)
    out["bound"] = "VALU (K/V decode into LDS and the softmax; both products on MFMA)"
    return out


def encoder_bytes_per_weight(bits):
    """Algorithmic HBM bytes per weight of the fused one-sided encode: the
    fp32 weight read; the 2-bit base planes, the b-bit residual and two fp16
    scales per 128 weights written (the d_in sign bytes are left out)."""
    return 4.0 + (2 + bits) / 8.0 + 4.0 / 128


def encoder_leg(nl, torch, synth, reps, cpu_seconds=0.0):
    """The round-to-nearest encoder on the 7B/8B-class projections (dense
    fp32 W -> 2-bit base + 7-bit residual planes, one-sided: one fused launch
    per linear, back to back on the stream between two events), the
    two-sided form on the 14336x4096 projection, and the level fit on 2^21
    normalised rotated weights (quantile start + 60 Lloyd iterations)."""
    import numpy as np
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    per, tot_b, tot_us = {}, 0.0, 0.0
    keep = None
    for si, (name, o, i) in enumerate(SHAPES):
        Wh = synth.make_dense_weights(o, i, cfg=30, idx=si)
        sh = synth.make_signs(i, 30, si, synth.STREAM_SIGN_IN)
        W, sg = torch.from_numpy(Wh).cuda(), torch.from_numpy(sh).cuda()
        c = nl.Codes(o, i, ENC_BITS, synth.LEVELS)
        for _ in range(2):
            nl.nested_encode(W, sg, None, c.desc)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            nl.nested_encode(W, sg, None, c.desc)
        e1.record()
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        b = o * i * encoder_bytes_per_weight(ENC_BITS)
        per[name] = {"shape": [o, i], "us": round(us, 1), "GBps": round(b / us / 1e3, 1)}
        tot_b += b
        tot_us += us
        if name == "gate/up":
            keep = (Wh, sh, W, sg, o, i)
        del W, c
        log(f"[bench] encode {name} {o}x{i}: {us:.1f} us, {b / us / 1e3:.0f} GB/s")
    layer_us = 2 * per["q/o"]["us"] + 2 * per["k/v"]["us"] + 2 * per["gate/up"]["us"] + per["down"]["us"]
    Wh, sh, W, sg, o, i = keep
    # two-sided form: input-side tiles into an fp64 workspace, column passes, quantise
    so = torch.from_numpy(synth.make_signs(o, 30, 2, synth.STREAM_SIGN_OUT)).cuda()
    c = nl.Codes(o, i, ENC_BITS, synth.LEVELS)
    ws = torch.empty(nl.nested_encode_workspace_bytes(o, i, True), dtype=torch.uint8, device="cuda")
    nl.nested_encode(W, sg, so, c.desc, ws)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(max(1, reps // 4)):
        nl.nested_encode(W, sg, so, c.desc, ws)
    e1.record()
    e1.synchronize()
    two_us = e0.elapsed_time(e1) * 1e3 / max(1, reps // 4)
    del ws, c
    # level fit on 2^21 samples
    wt = torch.empty((FIT_ROWS, i), dtype=torch.float64, device="cuda")
    nl.nested_encode_rotate(FIT_ROWS, i, W[:FIT_ROWS].contiguous(), sg, None, wt)
    v = torch.empty_like(wt)
    nl.nested_encode_normalize(FIT_ROWS, i, wt, v)
    fws = torch.empty(nl.nested_encode_fit_workspace_bytes(v.numel()), dtype=torch.uint8, device="cuda")
    fit = {}
    for iters in (0, 60):
        nl.nested_encode_fit_levels(v, v.numel(), iters, fws)
        t0 = time.perf_counter()
        for _ in range(3):
            lev = nl.nested_encode_fit_levels(v, v.numel(), iters, fws)
        fit[iters] = ((time.perf_counter() - t0) / 3 * 1e3, lev)
    del wt, v, fws
    achieved = tot_b / tot_us / 1e3
    out = {
        "per_linear": per, "decoder_layer_us": round(layer_us, 1),
        "model_32_layers_ms": round(LAYERS * layer_us / 1e3, 2),
        "two_sided_gate_up_us": round(two_us, 1),
        "fit_levels_ms": {"samples": FIT_ROWS * i, "quantile_start_only": round(fit[0][0], 2),
                          "quantile_start_plus_60_iterations": round(fit[60][0], 2),
                          "levels": [round(x, 5) for x in fit[60][1]]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "kernel": ENC_KERNEL_NAME + " (one-sided fused encode, the four projections)",
                     "bytes_per_weight": encoder_bytes_per_weight(ENC_BITS),
                     "avg_launch_us": round(tot_us / len(SHAPES), 2),
                     "avg_algorithmic_bytes": int(tot_b / len(SHAPES)),
                     "timing": "HIP events around back-to-back launches on the stream",
                     "kernel_source_digest": kernel_source_digest(ENC_SOURCES)},
    }
    tr = stored_traffic(kernel_source_digest(ENC_SOURCES), ENC_TRAFFIC_FILE)
    out["roofline"]["traffic"] = None if tr is None else round(tr)
    if cpu_seconds > 0:
        import oracle.encode as oenc
        rows, t0, n = 64, time.time(), 0
        while True:
            r0 = (n * rows) % o
            oenc.encode(Wh[r0:r0 + rows], sh, None, ENC_BITS, synth.LEVELS)
            n += 1
            if time.time() - t0 >= cpu_seconds:
                break
        dt = time.time() - t0
        out["cpu_baseline"] = {"value": round(n * rows * i * encoder_bytes_per_weight(ENC_BITS) / dt / 1e9, 4),
                               "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} blocks of {rows} rows of the 14336x4096 projection in {dt:.1f} s"}
    return out


def w4w8_bytes_per_weight(verify):
    """Algorithmic bytes per weight of the W4/W8 dual-plane linear: one or
    two 4-bit planes and one fp16 scale per 128 weights."""
    return (1.0 if verify else 0.5) + 2.0 / 128


def w4w8_leg(nl, torch, synth, reps, pool_gib, roofline_only=False):
    """The BitNest W4/W8 dual-plane linear on the 7B/8B-class projections:
    draft and verify at T = 1, 16 and 64, each (shape, mode, T) as a graph of
    calls over a pool of distinct weight copies (so weights stream from HBM),
    timed by events around the replays."""
    import numpy as np
    set_bytes = sum(o * i for _, o, i in SHAPES) * w4w8_bytes_per_weight(True)
    ncopy = max(2, math.ceil(pool_gib * 2 ** 30 / set_bytes))
    handles, xs, wss, ys = [], [], [], []
    for si, (name, o, i) in enumerate(SHAPES):
        lin = synth.make_w4w8_linear(o, i, cfg=60, idx=si)
        d = [torch.from_numpy(np.ascontiguousarray(lin[k]).view(dt)).cuda()
             for k, dt in (("base_plane", np.uint8), ("ref_plane", np.uint8), ("scales", np.int16))]
        handles.append([nl.nested_w4w8_create(o, i, *d) for _ in range(ncopy)])
        del d
        xs.append(torch.from_numpy(synth.make_x(max(W48_TS), i, cfg=60, idx=si).view(np.int16)).cuda())
        wss.append(torch.zeros(nl.nested_w4w8_workspace_bytes(handles[-1][0], max(W48_TS)), dtype=torch.uint8,
                               device="cuda"))
        ys.append(torch.empty((max(W48_TS), o), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()

    def call(si, cp, T, verify, stream):
        (nl.nested_w4w8_verify if verify else nl.nested_w4w8_draft)(handles[si][cp], xs[si], T, ys[si], wss[si],
                                                                     stream)

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    per_case, roof = {}, None
    for T in ((16,) if roofline_only else W48_TS):
        for verify in ((True,) if roofline_only else (True, False)):
            tot_us = tot_b = 0.0
            shp = {}
            for si, (name, o, i) in enumerate(SHAPES):
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(s):
                    for cp in range(ncopy):
                        call(si, cp, T, verify, s)
                torch.cuda.current_stream().wait_stream(s)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    cs = torch.cuda.current_stream()
                    for cp in range(ncopy):
                        call(si, cp, T, verify, cs)
                g.replay()
                torch.cuda.synchronize()
                e0.record()
                for _ in range(reps):
                    g.replay()
                e1.record()
                e1.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps / ncopy
                del g
                b = o * i * w4w8_bytes_per_weight(verify)
                shp[name] = {"us": round(us, 2), "GBps": round(b / us / 1e3, 1)}
                tot_us += us
                tot_b += b
            key = f"{'verify' if verify else 'draft'}_T{T}"
            per_case[key] = {"us_per_pass": round(tot_us, 2), "GBps": round(tot_b / tot_us / 1e3, 1),
                             "frac_hbm_peak": round(tot_b / tot_us / 1e3 / HBM_PEAK_GBPS, 3), "shapes": shp}
            log(f"[bench] w4w8 {key}: {tot_us:.1f} us per pass, {tot_b / tot_us / 1e3:.0f} GB/s")
            if verify and T == 16:
                achieved = tot_b / tot_us / 1e3
                digest = kernel_source_digest(W48_SOURCES)
                tr = stored_traffic(digest, W48_TRAFFIC_FILE)
                roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None if tr is None else round(tr),
                        "kernel": W48_KERNEL + " (verify, T = 16, the four projections)",
                        "avg_launch_us": round(tot_us / len(SHAPES), 2),
                        "avg_algorithmic_bytes": int(tot_b / len(SHAPES)),
                        "timing": "HIP events around graph replays of one launch per weight copy",
                        "kernel_source_digest": digest}
    for hs in handles:
        for h in hs:
            nl.nested_w4w8_destroy(h)
    if roofline_only:
        return {"per_case": per_case, "roofline": roof}
    v1, v16 = per_case["verify_T1"]["us_per_pass"], per_case["verify_T16"]["us_per_pass"]
    return {"format": "BitNest W4 base + 4-bit refinement planes, fp16 group-128 scales, no online rotation",
            "pool_copies": ncopy, "per_case": per_case, "verify_T16_over_T1": round(v16 / v1, 3),
            "roofline": roof}


COPY_FLOATS = 64 << 20  # 256 MiB read + 256 MiB written per copy


def copy_calibration(torch):
    """A plain elementwise copy of known size, for scaling the HBM counters."""
    src = torch.ones(COPY_FLOATS, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    return {"kernel": "torch elementwise mul (copy)", "read_bytes": COPY_FLOATS * 4,
            "write_bytes": COPY_FLOATS * 4, "launches": 3}




ROOFLINE_TITLE = ("{mode}, T = {ts}, 4096x4096, 1024x4096, 14336x4096,\n"
                  "4096x14336, 2-bit base{resid}, one-sided")
W48_TITLE = ("verify at T = 16, W4 base + 4-bit refinement planes of 4096x4096, 1024x4096,\n"
             "14336x4096, 4096x14336")
ENC_TITLE = ("one-sided fused encode of dense fp32 4096x4096, 1024x4096, 14336x4096,\n"
             "4096x14336 into 2-bit base + 7-bit residual planes")


def counter_rows(d, counter):
    """(kernel name, value) of every dispatch in the rocprofv3 csv files under d."""
    import csv
    import glob
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def kernel_match(name, kernel, prefix):
    return name.startswith(prefix + kernel) if prefix else kernel in name


def pmc_summary(fetch_dir, write_dir, out_path, kernel, prefix="void nl::", title="", flag="--roofline-only",
                digest=None, display=None):
    """Per-launch HBM traffic of one kernel from two rocprofv3 --pmc runs of
    `bench.py <flag>` (FETCH_SIZE, then WRITE_SIZE), each counter scaled by
    what it reads for the calibration copy of known size."""

    def split(rs):
        fwd = [v for k, v in rs if kernel_match(k, kernel, prefix)]
        cpy = [v for k, v in rs if "elementwise" in k and "MulFunctor" in k]
        return fwd, cpy

    f_fwd, f_cpy = split(counter_rows(fetch_dir, "FETCH_SIZE"))
    w_fwd, w_cpy = split(counter_rows(write_dir, "WRITE_SIZE"))
    if not f_fwd or not w_fwd or not f_cpy or not w_cpy:
        raise SystemExit(f"pmc summary: missing rows ({len(f_fwd)} {len(w_fwd)} {len(f_cpy)} {len(w_cpy)})")
    known = COPY_FLOATS * 4
    kf = known / (sorted(f_cpy)[len(f_cpy) // 2] * 1024)
    kw = known / (sorted(w_cpy)[len(w_cpy) // 2] * 1024)
    fetch = sum(f_fwd) / len(f_fwd) * 1024 * kf
    write = sum(w_fwd) / len(w_fwd) * 1024 * kw
    summ = {"--roofline-only": "--pmc-summary", "--encoder-only": "--pmc-summary-encoder",
            "--w4w8-only": "--pmc-summary-w4w8", "--kv-traffic-only": "--pmc-summary-kv"}[flag]
    text = (f"HBM traffic of {display or kernel} ({title})\n"
            f"commands:\n"
            f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -o p -- python3 bench.py {flag}\n"
            f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -o p -- python3 bench.py {flag}\n"
            f"  python3 bench.py {summ} <fetch_dir> <write_dir>\n"
            f"launches: {len(f_fwd)} (fetch run), {len(w_fwd)} (write run)\n"
            f"FETCH_SIZE per launch (raw): {sum(f_fwd) / len(f_fwd):.1f} KiB\n"
            f"WRITE_SIZE per launch (raw): {sum(w_fwd) / len(w_fwd):.1f} KiB\n"
            f"calibration copy ({known} bytes read and written): FETCH_SIZE {sorted(f_cpy)[len(f_cpy) // 2]:.1f} KiB, "
            f"WRITE_SIZE {sorted(w_cpy)[len(w_cpy) // 2]:.1f} KiB -> scale {kf:.3f} (fetch), {kw:.3f} (write)\n"
            f"hbm read bytes per launch: {fetch:.0f}\n"
            f"hbm write bytes per launch: {write:.0f}\n"
            f"hbm bytes per launch: {fetch + write:.0f}\n"
            f"kernel source digest: {kernel_source_digest() if digest is None else digest}\n")
    with open(out_path, "w") as fh:
        fh.write(text)
    print(text, end="")


def trace_summary(trace_dir):
    """Kernel-trace summary of the two roofline kernels from one
    `rocprofv3 --kernel-trace --stats` run of `bench.py --roofline-only`: the
    launches in the leg's order (8 warm-up launches, then per projection and
    T two rounds over the weight copies), averaged per (projection, T)."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)):
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    stats = []
    for f in sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)):
        stats += list(csv.DictReader(open(f)))
    for mode, (kernel, bits, ts, traffic_file) in ROOF.items():
        mine = [r for r in rows if kernel_match(r["Kernel_Name"], kernel, "void nl::")]
        timed = mine[8:]
        per = len(SHAPES) * len(ts) * 2
        if not timed or len(timed) % per:
            raise SystemExit(f"trace summary: {len(mine)} launches of {kernel}, not 8 + a multiple of {per}")
        ncopy = len(timed) // per
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
        bpw = (0.265625 + (bits / 8.0 + 1.0 / 64.0 if bits else 0.0))
        lines = [f"{kernel}: {mode}, T = {' and '.join(map(str, ts))}, one-sided 2-bit base"
                 + (f" + {bits}-bit residual" if bits else " (draft: base planes only)")
                 + ", group-128 fp16 scales,",
                 "projections " + ", ".join(f"{o}x{i}" for _, o, i in SHAPES)
                 + f" ({ncopy} distinct weight copies per projection)", "",
                 "command:",
                 "  rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o p -- python3 bench.py --roofline-only",
                 "  python3 bench.py --trace-summary <dir>", ""]
        for r in stats:
            if kernel_match(r["Name"], kernel, "void nl::"):
                lines.append(f"kernel_stats.csv: calls {r['Calls']}, average {float(r['AverageNs']) / 1e3:.2f} us "
                             f"(all launches, the first 8 warm the code)")
        lines.append(f"kernel trace, the {len(timed)} timed launches: average {sum(durs) / len(durs):.2f} us")
        k = 0
        for _, o, i in SHAPES:
            for T in ts:
                d = durs[k:k + 2 * ncopy]
                k += 2 * ncopy
                us = sum(d) / len(d)
                lines.append(f"  {o:>5d}x{i:<5d} T={T:2d}: {us:6.2f} us  ({o * i * bpw / us / 1e3:6.0f} GB/s of weights)")
        lines.append(f"kernel source digest: {kernel_source_digest()}")
        name = kernel.split("<")[0] + ("_6bit_verify" if bits else "_draft") + "_T" + "_T".join(map(str, ts))
        out = os.path.join(ROOT, "profiles", f"{name}_proj7b8b_kernel_stats.txt")
        with open(out, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print("\n".join(lines))


def all_stats_summary(trace_dir):
    """Every kernel of one default bench run, from the kernel_stats.csv of
    `rocprofv3 --kernel-trace --stats` around `bench.py --no-cpu-baseline`."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)):
        rows += list(csv.DictReader(open(f)))
    if not rows:
        raise SystemExit(f"all-stats summary: no kernel_stats.csv under {trace_dir}")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["All kernels of one default bench run (the verify step graph, per-case graphs T = 1..64, single",
             "calls, two-sided legs, the roofline legs, the 1024x1024 linear, the decoder layer, the MoE block,",
             "whole Llama-8B-shaped and 31B-class passes, and the W4/W8, nested-KV, draft-tree and encoder legs)",
             "", "command:",
             "  rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- python3 bench.py --no-cpu-baseline",
             "  python3 bench.py --all-stats-summary <dir>", "",
             f"{'kernel':<72s} {'calls':>7s} {'total ms':>10s} {'avg us':>9s} {'share':>6s}"]
    for r in rows:
        name = r["Name"].replace("void ", "")
        name = name if len(name) <= 72 else name[:69] + "..."
        lines.append(f"{name:<72s} {int(r['Calls']):>7d} {float(r['TotalDurationNs']) / 1e6:>10.2f} "
                     f"{float(r['AverageNs']) / 1e3:>9.2f} {float(r['Percentage']):>5.1f}%")
    lines.append(f"kernel source digest: {kernel_source_digest()}")
    out = os.path.join(ROOT, "profiles", "bench_all_kernels_proj7b8b_kernel_stats.txt")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


UTIL_COUNTERS = ("VALUBusy", "MfmaUtil", "OccupancyPercent", "MeanOccupancyPerCU", "MemUnitStalled", "TA_BUSY_avr",
                 "SQ_WAIT_INST_ANY", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VMEM_RD", "SQ_WAVES",
                 "SQ_BUSY_CYCLES")


def util_summary(dirs, out_path):
    """Utilisation counters of the two roofline kernels from rocprofv3 --pmc
    runs of `bench.py --roofline-only` (one pass per directory): the mean per
    dispatch of each counter found."""
    lines = ["Utilisation counters of the roofline kernels (verify: the single launch at T = 4 and 8; draft: the",
             "staged-x' launch at T = 8 and 16; 4096x4096, 1024x4096, 14336x4096, 4096x14336, one-sided),",
             "mean per dispatch over the --roofline-only launches",
             "commands (one counter pass each):"]
    passes = {0: "VALUBusy MfmaUtil OccupancyPercent MemUnitStalled TA_BUSY_avr",
              1: "MeanOccupancyPerCU SQ_WAIT_INST_ANY SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_VMEM_RD SQ_WAVES"}
    for k, d in enumerate(dirs):
        lines.append(f"  rocprofv3 --pmc {passes.get(k, '<counters>')} --output-format csv -d <dir{k}> -o p -- "
                     f"python3 bench.py --roofline-only")
    lines.append(f"  python3 bench.py --util-summary {' '.join(f'<dir{k}>' for k in range(len(dirs)))}")
    for mode, (kernel, *_rest) in ROOF.items():
        vals = {}
        for d in dirs:
            for c in UTIL_COUNTERS:
                rs = [v for k, v in counter_rows(d, c) if kernel_match(k, kernel, "void nl::")]
                if rs:
                    vals[c] = (sum(rs) / len(rs), len(rs))
        lines.append(f"{kernel} ({mode}):")
        for c, (v, n) in vals.items():
            lines.append(f"  {c}: {v:.4g} (mean of {n} dispatches)")
    lines.append(f"kernel source digest: {kernel_source_digest()}")
    text = "\n".join(lines) + "\n"
    with open(out_path, "w") as fh:
        fh.write(text)
    print(text, end="")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--pool-gib", type=float, default=1.2)
    ap.add_argument("--reps", type=int, default=15, help="graph replays per per-case timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle time for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the W4/W8, tree, KV and encoder legs")
    ap.add_argument("--roofline-only", action="store_true",
                    help="run only the roofline launches and the counter calibration copy (for rocprofv3)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the verify and draft traffic summaries from two --pmc runs of --roofline-only")
    ap.add_argument("--all-stats-summary", metavar="DIR",
                    help="write the kernel-stats summary of a --kernel-trace --stats run of the whole bench")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="write the kernel-trace summaries of the roofline kernels from a --kernel-trace run of --roofline-only")
    ap.add_argument("--util-summary", nargs="+", metavar="DIR",
                    help="write the utilisation counter summary from --pmc runs of --roofline-only")
    ap.add_argument("--encoder-only", action="store_true",
                    help="run only the encoder leg and the counter calibration copy (for rocprofv3)")
    ap.add_argument("--pmc-summary-encoder", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the encoder's traffic summary from two rocprofv3 --pmc runs of --encoder-only")
    ap.add_argument("--kv-traffic-only", action="store_true",
                    help="run only eager calls of the 32768-position verify attention, for the HBM counters")
    ap.add_argument("--pmc-summary-kv", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise --kv-traffic-only FETCH_SIZE / WRITE_SIZE runs into the KV traffic file")
    ap.add_argument("--kv-only", action="store_true",
                    help="run only the nested-KV leg (writer and tree attention) and print its JSON")
    ap.add_argument("--w4w8-only", action="store_true",
                    help="run only the W4/W8 leg and the counter calibration copy (for rocprofv3)")
    ap.add_argument("--pmc-summary-w4w8", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the W4/W8 kernel's traffic summary from two rocprofv3 --pmc runs of --w4w8-only")
    args = ap.parse_args()
    if args.pmc_summary:
        for mode, (kernel, bits, ts, path) in ROOF.items():
            pmc_summary(*args.pmc_summary, path, kernel=kernel,
                        title=ROOFLINE_TITLE.format(mode=mode, ts=" and ".join(map(str, ts)),
                                                    resid=" + 6-bit residual" if bits else ""))
        return
    if args.util_summary:
        util_summary(args.util_summary, UTIL_FILE)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.all_stats_summary:
        all_stats_summary(args.all_stats_summary)
        return
    if args.pmc_summary_w4w8:
        pmc_summary(*args.pmc_summary_w4w8, W48_TRAFFIC_FILE, kernel=W48_KERNEL, prefix="", title=W48_TITLE,
                    flag="--w4w8-only", digest=kernel_source_digest(W48_SOURCES))
        return
    if args.pmc_summary_encoder:
        pmc_summary(*args.pmc_summary_encoder, ENC_TRAFFIC_FILE, kernel=ENC_KERNEL, prefix="", title=ENC_TITLE,
                    flag="--encoder-only", digest=kernel_source_digest(ENC_SOURCES), display=ENC_KERNEL_NAME)
        return
    if args.pmc_summary_kv:
        pmc_summary(*args.pmc_summary_kv, KV_TRAFFIC_FILE, kernel=KV_KERNEL, prefix="", title=KV_TITLE,
                    flag="--kv-traffic-only", digest=kernel_source_digest(KV_SOURCES))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run it with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_nested_quantized_amd as nl
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    nl.lib()
    dev = "cuda"
    torch.cuda.set_device(0)

    if args.w4w8_only:
        w48 = w4w8_leg(nl, torch, synth, args.reps, args.pool_gib, roofline_only=True)
        calib = copy_calibration(torch)
        print(json.dumps({"w4w8": w48, "copy_calibration": calib}), flush=True)
        return
    if args.kv_traffic_only:
        call, b = kv_case(nl, torch, synth, np.random.default_rng(91), 32, 8, 32768, 16, True)
        for _ in range(20):
            call()
        torch.cuda.synchronize()
        calib = copy_calibration(torch)
        print(json.dumps({"kv_traffic_case": {"kv_bytes": b, "calls": 20}, "copy_calibration": calib}), flush=True)
        return
    if args.kv_only:
        print(json.dumps({"nested_kv": kv_leg(nl, torch, synth, args.reps)}), flush=True)
        return
    if args.encoder_only:
        enc = encoder_leg(nl, torch, synth, args.reps)
        calib = copy_calibration(torch)
        print(json.dumps({"encoder": enc, "copy_calibration": calib}), flush=True)
        return

    def bpw(verify):
        return synth.bytes_per_weight(BITS if verify else 0)

    # ---- weights: one synthetic linear per shape, repacked into a pool of copies
    set_bytes = sum(o * i for _, o, i in SHAPES) * bpw(True)
    ncopy = max(2, math.ceil(args.pool_gib * 2 ** 30 / set_bytes))
    lins, handles, xs, xh, wss, ys = [], [], [], [], [], []
    t0 = time.time()
    for si, (name, o, i) in enumerate(SHAPES):
        lin = synth.make_linear(o, i, BITS, cfg=1, idx=si, two_sided=False)
        lins.append(lin)
        d = dev_arrays(torch, lin)
        handles.append([nl.nested_linear_create(o, i, BITS, levels=lin["levels"], **d) for _ in range(ncopy)])
        del d
        xh.append(synth.make_x(max(CASE_TS), i, cfg=1, idx=si))
        xs.append(torch.from_numpy(xh[-1].view(np.int16)).to(dev))
        wss.append(torch.zeros(nl.nested_linear_workspace_bytes(handles[-1][0], max(CASE_TS)),
                               dtype=torch.uint8, device=dev))
        ys.append(torch.empty((max(CASE_TS), o), dtype=torch.float32, device=dev))
        log(f"[bench] {name} {o}x{i}: {ncopy} copies created ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()

    def call(si, copy, T, verify, stream=None):
        fn = nl.nested_linear_verify if verify else nl.nested_linear_draft
        fn(handles[si][copy], xs[si], T, ys[si], wss[si], stream)

    stream = torch.cuda.current_stream()
    if args.roofline_only:
        roof = {m: roofline_leg(nl, call, ncopy, stream, bpw, m) for m in ROOF}
        for ws in wss:
            check_status(nl, ws, "roofline")
        calib = copy_calibration(torch)
        print(json.dumps({"roofline": roof, "copy_calibration": calib}), flush=True)
        return

    # ---- the streaming-read reference (the measured ceiling)
    sref = stream_ref_leg(nl, torch)
    stream_gbps = sref["GBps"]

    # ---- the step: 20 verify calls, weights rotating through the pool
    seq, c = [], 0
    for T in STEP_TS:
        for si in range(len(SHAPES)):
            seq.append((si, c % ncopy, T, True))
            c += 1
    step_bytes = sum(SHAPES[si][1] * SHAPES[si][2] * bpw(v) for si, _, _, v in seq)
    g = capture(torch, lambda s: [call(*cl, stream=s) for cl in seq])
    # a replay reproduces the eager outputs bit for bit (rows the step writes)
    rows = max(STEP_TS)
    eager = [y[:rows].clone() for y in ys]
    for y in ys:
        y.zero_()
    g.replay()
    torch.cuda.synchronize()
    for a, b in zip(eager, ys):
        assert torch.equal(a, b[:rows]), "graph replay differs from eager run"
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        g.replay()
    e1.record()
    e1.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    for ws in wss:
        check_status(nl, ws, "the step")
    del g
    log(f"[bench] step: {ms_per_step:.3f} ms, {value:.1f} GB/s ({args.steps} steps)")

    # ---- per case: µs per pass over the four projections (replays of a graph
    # of ncopy passes), per-shape means, and the error on sampled rows
    import oracle
    refs = {(si, v): oracle.forward(lins[si], xh[si], v, rows=(0, ERR_ROWS))
            for si in range(len(SHAPES)) for v in (True, False)}
    per_case = {}
    for T in CASE_TS:
        for verify in (True, False):
            err = 0.0
            for si in range(len(SHAPES)):
                call(si, 0, T, verify)
                err = max(err, rel_err(ys[si][:T, :ERR_ROWS].cpu().numpy(), refs[(si, verify)][:T]))
                check_status(nl, wss[si], f"T={T}")
            gp = capture(torch, lambda s: [call(si, cp, T, verify, s) for cp in range(ncopy)
                                           for si in range(len(SHAPES))])
            st = pstats([u / ncopy for u in replay_samples(torch, gp, args.reps)])
            del gp
            shp, tot_b = {}, 0.0
            for si, (name, o, i) in enumerate(SHAPES):
                gs = capture(torch, lambda s: [call(si, cp, T, verify, s) for cp in range(ncopy)])
                us = float(np.mean(replay_samples(torch, gs, max(3, args.reps // 3)))) / ncopy
                del gs
                b = o * i * bpw(verify)
                tot_b += b
                shp[name] = {"us": round(us, 2), "GBps": round(b / us / 1e3, 1)}
            key = f"{'verify' if verify else 'draft'}_T{T}"
            per_case[key] = dict({"us_per_pass": st["us"], "p10": st["p10"], "p90": st["p90"]},
                                 **rate(tot_b, st["us"], stream_gbps), max_rel_err=float(f"{err:.3g}"),
                                 shapes=shp)
            log(f"[bench] {key}: {st['us']:.1f} us per pass [{st['p10']:.1f}, {st['p90']:.1f}], "
                f"{per_case[key]['GBps']:.0f} GB/s, err {err:.2e}")
    for ws in wss:
        check_status(nl, ws, "per case")

    # ---- launch-inclusive single calls (eager, one call between events), verify
    single = {}
    for T in (1, 16):
        tot = 0.0
        for si in range(len(SHAPES)):
            durs = []
            for r in range(20):
                torch.cuda.synchronize()
                e0.record(stream)
                call(si, r % ncopy, T, True, stream)
                e1.record(stream)
                e1.synchronize()
                durs.append(e0.elapsed_time(e1) * 1e3)
            durs.sort()
            tot += durs[len(durs) // 2]
        single[f"verify_T{T}_us_per_pass_median"] = round(tot, 2)

    # ---- the two-sided form (y = S_o H_o y~) at T = 1 and 16
    two_lins, two_handles, two_ws = [], [], []
    for si, (name, o, i) in enumerate(SHAPES):
        lin2 = synth.make_linear(o, i, BITS, cfg=1, idx=si, two_sided=True)
        two_lins.append(lin2)
        d = dev_arrays(torch, lin2)
        two_handles.append([nl.nested_linear_create(o, i, BITS, levels=lin2["levels"], **d) for _ in range(ncopy)])
        two_ws.append(torch.zeros(nl.nested_linear_workspace_bytes(two_handles[-1][0], 16),
                                  dtype=torch.uint8, device=dev))
        del d

    def call2(si, copy, T, verify, s=None):
        fn = nl.nested_linear_verify if verify else nl.nested_linear_draft
        fn(two_handles[si][copy], xs[si], T, ys[si], two_ws[si], s)

    two_sided = {}
    for T in (1, 16):
        for verify in (True, False):
            err = 0.0
            for si, (name, o, i) in enumerate(SHAPES):
                call2(si, 0, T, verify)
                b_out = nl.nested_linear_info(two_handles[si][0])["block_out"]
                ref = oracle.forward(two_lins[si], xh[si][:T], verify, rows=(0, b_out))
                err = max(err, rel_err(ys[si][:T, :b_out].cpu().numpy(), ref))
                check_status(nl, two_ws[si], "two-sided")
            gp = capture(torch, lambda s: [call2(si, cp, T, verify, s) for cp in range(ncopy)
                                           for si in range(len(SHAPES))])
            st = pstats([u / ncopy for u in replay_samples(torch, gp, args.reps)])
            del gp
            tot_b = sum(o * i * bpw(verify) for _, o, i in SHAPES)
            two_sided[f"{'verify' if verify else 'draft'}_T{T}"] = dict(
                {"us_per_pass": st["us"], "p10": st["p10"], "p90": st["p90"]}, **rate(tot_b, st["us"], stream_gbps),
                max_rel_err=float(f"{err:.3g}"))
    for hs in two_handles:
        for h in hs:
            nl.nested_linear_destroy(h)
    del two_handles, two_ws

    roofline = roofline_leg(nl, call, ncopy, stream, bpw, "verify")
    roofline_draft = roofline_leg(nl, call, ncopy, stream, bpw, "draft")
    for ws in wss:
        check_status(nl, ws, "roofline")
    for hs in handles:
        for h in hs:
            nl.nested_linear_destroy(h)
    torch.cuda.empty_cache()

    # ---- the 1024x1024 int8 linear
    single1024 = single1024_leg(nl, torch, synth, args.reps, stream_gbps)

    # ---- one decoder layer with fused launches
    layer = decoder_layer_leg(nl, torch, synth, args.reps, stream_gbps, args.pool_gib)

    # ---- the MoE block (grouped calls)
    moe = moe_leg(nl, torch, synth, args.reps, stream_gbps)

    # ---- whole dense-model passes (one graph per pass)
    model = {}
    for spec in MODELS:
        m = model_leg(nl, torch, synth, 5, spec, stream_gbps)
        model[spec[0]] = m
        log(f"[bench] {spec[0]} pass: verify T={m['verify']['T']} {m['verify']['us_per_pass']:.0f} us "
            f"({m['verify']['GBps']:.0f} GB/s), draft T={m['draft']['T']} {m['draft']['us_per_pass']:.0f} us "
            f"({m['draft']['GBps']:.0f} GB/s)")

    nxt = {}
    if not args.no_next:
        # ---- the BitNest W4/W8 dual-plane format (same contraction, other planes)
        nxt["w4w8"] = w4w8_leg(nl, torch, synth, args.reps, args.pool_gib)
        # ---- the draft tree (build once from the statistics, accept per step)
        nxt["draft_tree"] = tree_leg(nl, torch, synth, args.reps, cpu_seconds=0.0 if args.no_cpu_baseline else 2.0)
        # ---- nested KV cache: tree-masked attention over KV8 / KV4
        nxt["nested_kv"] = kv_leg(nl, torch, synth, args.reps)
        # ---- the offline encoder (dense W -> planes) and the level fit
        nxt["encoder"] = encoder_leg(nl, torch, synth, args.reps, cpu_seconds=0.0 if args.no_cpu_baseline else 3.0)

    # ---- CPU baseline: the fp64 oracle on the step's calls, host cores
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle over the step's {len(seq)} calls, {oracle.num_threads()} threads")
        t0 = time.time()
        nsteps = 0
        while True:
            for si, _, T, verify in seq:
                oracle.forward(lins[si], xh[si][:T], verify)
            nsteps += 1
            if time.time() - t0 >= args.cpu_seconds:
                break
        dt = time.time() - t0
        cpu = {"value": round(nsteps * step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle",
               "sample": f"{nsteps} full step(s) of the same workload ({len(seq)} verify calls, "
                         f"{step_bytes / 1e9:.3f} GB of weights each) in {dt:.1f} s"}
        log(f"[bench] cpu baseline: {dt:.1f} s, {cpu['value']} GB/s")

    out = {
        "metric": "µs/verify pass + effective weight GB/s (frac of HBM peak) vs tree size T=1..64",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16-mfma/fp32", "data": "synthetic",
        "config": {"workload": "7B/8B-class projections 4096x4096, 1024x4096, 14336x4096, 4096x14336; "
                               "2-bit Lloyd-Max base + 6-bit residual, fp16 group-128 scales; bf16 x; "
                               "one-sided y = (Q_b + Q_r) H S x; verify at T=1,4,8,16,32, one launch per call",
                   "calls_per_step": len(seq), "weight_bytes_per_step": int(step_bytes),
                   "pool_copies": ncopy, "pool_bytes": int(ncopy * set_bytes)},
        "stream_ref": sref,
        "per_case": per_case,
        "single_call": single,
        "two_sided": two_sided,
        "single_1024_int8": single1024,
        "decoder_layer": layer,
        "moe_block": moe,
        "model_pass": model,
        **nxt,
        "roofline": roofline,
        "roofline_draft": roofline_draft,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
