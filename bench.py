#!/usr/bin/env python3
"""Benchmark of one GPU's share of the routed MoE layer on MI355X.

Workload: the decode share of a large MoE (H=7168, I=2048, top-8 over 256
experts, this GPU holding experts 0..31, FP8 activations x MXFP4 weights).
One step runs the whole layer (route, permute, grouped W1 + fused epilogue,
grouped W2, combine) once for each decode batch T in {1, 8, 32, 128}, each
call on a new routing draw (logits and x) over the same experts. The weights
are held in several identical copies and consecutive calls rotate through
them, as consecutive MoE layers of a model would, so a call never finds the
previous call's weights in the 256 MB last-level cache.

The launch sequences of exactly the warm-up steps and of exactly the timed
steps are captured into one HIP graph each and replayed once. Printed JSON
line (stdout): value = algorithmic HBM bytes of the timed steps' layer calls /
wall time of the timed steps, in TB/s. Algorithmic bytes per call: router
logits, x codes + scales, the W1 and W2 codes + scales of the experts that
received at least one token, and the BF16 output. The "roofline" object is
for the dominant kernel (the grouped W1 GEMM): a graph of its launches on
the step sequence's groupings, in step order, timed with HIP events on the
replay stream, with "traffic" the HBM bytes per launch
measured by hardware counters (profiles/decode_w1_hbm_traffic.txt; null once
the kernel sources differ from those the counters were taken with);
"hbm_read_measured" is the HBM read rate of a plain streaming read (the
library's read probe over 2 GiB), with the step value and the W1 rate as
fractions of it; "cpu_baseline" times the CPU oracle on
a bounded sample (the step's calls at T = 1, 8 and 32 of one routing draw). "other_workloads"
gives the layer latency, TB/s, TFLOP/s and roofline fraction of the tiny,
full-expert, 16K-token prefill and shared-expert workloads (graph replay),
each with the oracle timed on a token sample of the same workload
("cpu_oracle").

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-other-workloads]
    python bench.py --only prefill          # one workload's latency line only
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DECODE_T = (1, 8, 32, 128)
N_VARIANTS = 16
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes_per_group(H: int, I: int, fp4: bool) -> int:
    """W1 [2I, H] + W2 [H, I] codes and their E8M0 scales, one expert."""
    n = 3 * I * H
    return (n // 2 if fp4 else n) + n // 32


def layer_bytes(T: int, E: int, H: int, I: int, active: int, fp4: bool) -> int:
    return 4 * T * E + T * H + T * H // 32 + active * weight_bytes_per_group(H, I, fp4) + 2 * T * H


def w1_bytes(R: int, H: int, I: int, active: int, fp4: bool) -> int:
    """The W1 launch: active experts' W1 codes + scales, the grouped x rows
    once, the routing weights, and the h codes + scales it writes."""
    n = 2 * I * H
    wb = (n // 2 if fp4 else n) + n // 32
    return active * wb + R * (H + H // 32) + 4 * R + R * (I + I // 32)


def cpu_baseline(cfgs, moe_bytes_fn, Ts=(1, 8, 32)):
    """Time the oracle on the step's layer calls at T in Ts (routing draw 0),
    three of the step's four calls (T = 128 alone takes longer than the
    three together); the weights of the experts those calls touch are
    quantised by the oracle beforehand (untimed). Returns the calls' bytes
    over their summed wall time."""
    import numpy as np
    from oracle import moe as omoe, mx
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    c0 = cfgs[Ts[0]]
    w1q, w1s, w2q, w2s = [None] * c0.n_local, [None] * c0.n_local, [None] * c0.n_local, [None] * c0.n_local
    total_dt, total_bytes, parts = 0.0, 0.0, []
    for T in Ts:
        c = cfgs[T]
        lg = synth.logits(c, 0)
        xq, xs = mx.quantize_mx(synth.x(c, 0), mx.FMT_E4M3)
        idx, _ = omoe.route(lg, c.k)
        active = sorted({int(e) - c.e0 for e in idx.ravel() if 0 <= int(e) - c.e0 < c.n_local})
        for g in active:
            if w1q[g] is None:
                w1q[g], w1s[g] = mx.quantize_mx(synth.w1(c, g), c.w_fmt)
                w2q[g], w2s[g] = mx.quantize_mx(synth.w2(c, g), c.w_fmt)
        t0 = time.perf_counter()
        omoe.moe_layer(lg, xq, xs, c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I, e0=c.e0, n_local=c.n_local)
        dt = time.perf_counter() - t0
        total_dt += dt
        total_bytes += moe_bytes_fn(T, len(active))
        parts.append(f"T={T} ({len(active)} active experts) {dt:.2f} s")
    return {"value": total_bytes / total_dt / 1e12, "unit": "TB/s", "cores": int(threads), "kind": "oracle",
            "sample": "the step's layer calls at T = " + ", ".join(str(T) for T in Ts)
                      + " (routing draw 0): " + "; ".join(parts)
                      + f"; {total_dt:.1f} s wall on the host CPU, fp64 NumPy",
            "host": host_description()}, total_dt


def host_description():
    """The host CPU's model name, the cores this process may run on, and the
    BLAS library NumPy calls."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                for i in threadpool_info() if i.get("user_api") == "blas"]
        blas = "; ".join(libs) or blas
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "numpy_blas": blas}


# token samples of the other workloads for the oracle's timing (about 1-5 s each)
ORACLE_SAMPLE_TOKENS = {"tiny": 16, "full": 1, "prefill": 4, "shared": 1}


def cpu_oracle_sample(name: str, ntok: int, threads: int):
    """Time the oracle on the first ntok tokens of a workload's routing draw 0
    (same shapes, experts and weights; the weights of the experts the sample
    touches are quantised beforehand, untimed). Rates use the sample's own
    algorithmic bytes and FLOPs."""
    import numpy as np
    from oracle import moe as omoe, mx
    import synth
    c = synth.config(name)
    lg = np.ascontiguousarray(synth.logits(c, 0)[:ntok])
    xq, xs = mx.quantize_mx(np.ascontiguousarray(synth.x(c, 0)[:ntok]), mx.FMT_E4M3)
    idx, _ = omoe.route(lg, c.k)
    local = [int(e) - c.e0 for e in idx.ravel() if 0 <= int(e) - c.e0 < c.n_local]
    active = sorted(set(local))
    w1q, w1s, w2q, w2s = [None] * c.n_local, [None] * c.n_local, [None] * c.n_local, [None] * c.n_local
    for g in active:
        w1q[g], w1s[g] = mx.quantize_mx(synth.w1(c, g), c.w_fmt)
        w2q[g], w2s[g] = mx.quantize_mx(synth.w2(c, g), c.w_fmt)
    shared = None
    if c.shared:
        a1, b1 = mx.quantize_mx(synth.shared_w1(c), c.w_fmt)
        a2, b2 = mx.quantize_mx(synth.shared_w2(c), c.w_fmt)
        shared = (a1, b1, a2, b2)
    t0 = time.perf_counter()
    omoe.moe_layer(lg, xq, xs, c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I, e0=c.e0, n_local=c.n_local,
                   shared=shared, transpose=c.transpose)
    dt = time.perf_counter() - t0
    fp4 = c.w_fmt == "e2m1"
    groups = len(active) + (1 if c.shared else 0)
    rows = len(local) + (ntok if c.shared else 0)
    nbytes = layer_bytes(ntok, c.E, c.H, c.I, groups, fp4)
    flops = 6.0 * rows * c.H * c.I
    return {"tokens": ntok, "wall_s": round(dt, 3), "TBps": nbytes / dt / 1e12,
            "TFLOPs": flops / dt / 1e12, "cores": int(threads), "kind": "oracle",
            "sample": f"the first {ntok} of {c.T} tokens (routing draw 0: {groups} groups, {rows} rows), "
                      f"fp64 NumPy on the host CPU"}


def cpu_oracle_full(names, threads: int, reps: int = 3):
    """The oracle on whole workloads (every token of routing draw 0): the
    median wall time of `reps` runs (one run for the 16K-token prefill), with
    the workload's algorithmic bytes and FLOPs. Minutes of CPU work, so only
    with --cpu-full."""
    import numpy as np
    from oracle import moe as omoe, mx
    import synth
    res = {}
    for name, T in names:
        c = synth.config(name, T)
        lg = synth.logits(c, 0)
        xq, xs = mx.quantize_mx(synth.x(c, 0), mx.FMT_E4M3)
        idx, _ = omoe.route(lg, c.k)
        local = [int(e) - c.e0 for e in idx.ravel() if 0 <= int(e) - c.e0 < c.n_local]
        active = sorted(set(local))
        w1q, w1s, w2q, w2s = [None] * c.n_local, [None] * c.n_local, [None] * c.n_local, [None] * c.n_local
        for g in active:
            w1q[g], w1s[g] = mx.quantize_mx(synth.w1(c, g), c.w_fmt)
            w2q[g], w2s[g] = mx.quantize_mx(synth.w2(c, g), c.w_fmt)
        shared = None
        if c.shared:
            a1, b1 = mx.quantize_mx(synth.shared_w1(c), c.w_fmt)
            a2, b2 = mx.quantize_mx(synth.shared_w2(c), c.w_fmt)
            shared = (a1, b1, a2, b2)
        n = 1 if name == "prefill" else reps
        walls = []
        for _ in range(n):
            t0 = time.perf_counter()
            omoe.moe_layer(lg, xq, xs, c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I, e0=c.e0, n_local=c.n_local,
                           shared=shared, transpose=c.transpose)
            walls.append(time.perf_counter() - t0)
            log(f"oracle {name} T={c.T}: {walls[-1]:.1f} s")
        dt = sorted(walls)[len(walls) // 2]
        fp4 = c.w_fmt == "e2m1"
        groups = len(active) + (1 if c.shared else 0)
        rows = len(local) + (c.T if c.shared else 0)
        nbytes = layer_bytes(c.T, c.E, c.H, c.I, groups, fp4)
        res[f"{name}-{c.T}"] = {"wall_s_median": round(dt, 2), "runs": n, "TBps": nbytes / dt / 1e12,
                                "TFLOPs": 6.0 * rows * c.H * c.I / dt / 1e12, "cores": int(threads),
                                "kind": "oracle", "sample": f"the whole workload (routing draw 0: {groups} groups, "
                                                            f"{rows} rows), fp64 NumPy on the host CPU"}
    return res


def oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


MFMA_FP8_PEAK_TFLOPS = 5000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_w1_hbm_traffic.txt")


def measured_traffic():
    """HBM bytes per W1 launch from the committed counter runs (FETCH_SIZE and
    WRITE_SIZE, calibrated on a 1 GiB copy), or None when the kernel sources
    changed since they were taken."""
    import hashlib
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        h = hashlib.sha256()
        for name in kv["kernel_sources"].split():
            with open(os.path.join(ROOT, "routed_grouped_gemm_amd", "csrc", name), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != kv["kernel_sources_sha256"]:
            return None
        return float(kv["bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def pct(xs, q):
    """The q-quantile of the sorted list xs (nearest rank)."""
    return xs[min(len(xs) - 1, max(0, round(q * (len(xs) - 1))))]


def spread(each):
    """min / median / max and p10 / median / p90 of per-replay latencies (us)."""
    each = sorted(each)
    return {"latency_us_min_median_max": [round(each[0], 2), round(pct(each, 0.5), 2), round(each[-1], 2)],
            "latency_us_p10_median_p90": [round(pct(each, 0.1), 2), round(pct(each, 0.5), 2),
                                          round(pct(each, 0.9), 2)]}


def other_workloads(torch, moe, synth, device, names, reps=10):
    """Layer latency of the other workloads (one GPU, graph replay, HIP events
    on the replay stream): the tiny case, the full-expert case, the 16K-token
    prefill case (MXFP8 weights, transposed copy of h) and the decode share
    at T = 32 with a shared expert. Each call alternates between two routing
    draws and two weight copies, so weights stream from HBM as in a model.
    `reps` back-to-back replays, each between its own pair of events: the
    mean over all of them, and the spread of the per-replay means.
    Algorithmic bytes and FLOPs as for the decode bench; roofline: HBM for
    the bandwidth-bound shapes, dense FP8 MFMA for prefill."""
    out = {}
    for name in names:
        ring = name == "prefill_token_ring"          # the prefill with the token ring
        c = synth.config("prefill" if ring else name)
        flags = moe.MOE_W1_WRITE_TRANSPOSE if c.transpose else 0
        if ring:
            flags |= moe.MOE_LAYER_TOKEN_RING
        dw = device.build_weights(c)
        copies = [dw]
        w1 = moe.PackedWeights.empty(c.n_local, 2 * c.I, c.H, dw.w1.fmt, True)
        w2 = moe.PackedWeights.empty(c.n_local, c.H, c.I, dw.w2.fmt, False)
        w1.buf.copy_(dw.w1.buf)
        w2.buf.copy_(dw.w2.buf)
        copies.append(device.DeviceWeights(w1, w2, dw.shared))
        ins = [device.build_inputs(c, v) for v in range(2)]
        ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I, bool(c.shared), flags)
        hT = (None, None)
        if c.transpose:
            ld = moe.moe_transposed_ld(c.R_max, c.G)
            hT = (torch.empty((c.I, ld), dtype=torch.uint8, device="cuda"),
                  torch.empty((c.I, ld // 32), dtype=torch.uint8, device="cuda"))
        res = torch.empty((c.T, c.H), dtype=torch.uint16, device="cuda")

        def call(v, wcopy):
            lg, xq, xs = ins[v]
            moe.moe_layer(lg, xq, xs, wcopy.w1, wcopy.w2, c.k, c.e0, c.n_local, wcopy.shared, flags,
                          out=res, ws=ws, hTq=hT[0], hTs=hT[1])

        stats = []
        for v in range(2):
            call(v, dw)
            cnt = ws.view("counts").cpu()
            stats.append((int((cnt[:c.n_local] > 0).sum()), int(cnt.sum())))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(4):
                call(i % 2, copies[(i // 2) % 2])
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            g.replay()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[reps]) * 1e3 / (4 * reps)
        each = [ev[i].elapsed_time(ev[i + 1]) * 1e3 / 4 for i in range(reps)]
        fp4 = c.w_fmt == "e2m1"
        bw = 0.5 if fp4 else 1.0
        nbytes, flops = 0.0, 0.0
        for active, R in stats:
            act = active + (1 if c.shared else 0)
            nbytes += (4 * c.T * c.E + c.T * c.H * (1 + 1 / 32) + act * 3 * c.I * c.H * (bw + 1 / 32)
                       + 2 * c.T * c.H) / 2
            flops += 6.0 * R * c.H * c.I / 2
        tbps = nbytes / us / 1e6
        tflops = flops / us / 1e6
        bound = "mfma" if c.name == "prefill" else "hbm"
        frac = tflops / MFMA_FP8_PEAK_TFLOPS if bound == "mfma" else tbps * 1e3 / HBM_PEAK_GBS
        out[name] = {"T": c.T, "H": c.H, "I": c.I, "E": c.E, "k": c.k, "local": c.n_local,
                     "shared": bool(c.shared), "weights": "MXFP4" if fp4 else "MXFP8",
                     "latency_us": round(us, 2), **spread(each), "TBps": round(tbps, 3),
                     "TFLOPs": round(tflops, 1), "bound": bound, "roofline_frac": round(frac, 4),
                     "active_groups": [a for a, _ in stats], "rows": [R for _, R in stats]}
        log(f"{name}: {out[name]}")
        del dw, copies, w1, w2, ws, hT, res, g
        torch.cuda.empty_cache()
    return out


def backward_workload(torch, moe, synth, device, reps=8):
    """The backward of the fused W1 epilogue at the 16K-token prefill shape:
    the forward layer runs once with the BF16 pre-activation saved, then the
    backward (dh = dy . W2^T on MFMA, the SwiGLU derivative with the routing
    weight, MX-E4M3 rows and 32-row transposed blocks of [dg | du], dw) on
    that grouping, with W2^T quantised along H and prepacked, and dy a seeded
    N(0, 1) gradient quantised to MXFP8. Timed with HIP events between
    `reps` back-to-back calls after one untimed call (the mean, and the
    spread of the single calls); FLOPs 2 R H I."""
    import numpy as np
    c = synth.config("prefill")
    fmt = moe.MOE_FMT_MXFP8
    dw = device.build_weights(c)
    w2t = moe.PackedWeights.empty(c.n_local, c.I, c.H, fmt, False)
    for g in range(c.n_local):
        q, sc = moe.moe_quantize_mx(torch.from_numpy(np.ascontiguousarray(synth.w2(c, g).T)).cuda(), fmt)
        w2t.fill_group(g, q, sc)
    logits, xq, xs = device.build_inputs(c)
    flags = moe.MOE_W1_WRITE_TRANSPOSE
    ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I, False, flags)
    ld = moe.moe_transposed_ld(c.R_max, c.G)
    hT = (torch.empty((c.I, ld), dtype=torch.uint8, device="cuda"),
          torch.empty((c.I, ld // 32), dtype=torch.uint8, device="cuda"))
    pre = torch.empty((c.R_max, 2 * c.I), dtype=torch.uint16, device="cuda")
    moe.moe_layer(logits, xq, xs, dw.w1, dw.w2, c.k, c.e0, c.n_local, None, flags, ws=ws, hTq=hT[0], hTs=hT[1],
                  epi=moe.Epilogue(save_pre=pre))
    g32 = torch.Generator(device="cpu").manual_seed(c.seed + 77)
    dyq, dys = moe.moe_quantize_mx(torch.randn((c.T, c.H), generator=g32).cuda(), fmt)
    R = int(ws.view("counts").sum().item())

    def call():
        return moe.moe_grouped_w1_backward(w2t, ws.view("counts"), ws.view("offsets"), ws.view("row_w"), dyq, dys,
                                           ws.view("row_src"), pre, c.I, flags=moe.MOE_W1_WRITE_TRANSPOSE,
                                           offsets32=ws.view("offsets32"))
    call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    keep = []
    for i in range(reps):
        keep.append(call())
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    del keep
    us = ev[0].elapsed_time(ev[reps]) * 1e3 / reps
    each = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)]
    flops = 2.0 * R * c.H * c.I
    res = {"T": c.T, "H": c.H, "I": c.I, "E": c.E, "k": c.k, "rows": R, "weights": "MXFP8 (W2 transposed)",
           "latency_us": round(us, 2), **spread(each), "TFLOPs": round(flops / us / 1e6, 1), "bound": "mfma",
           "roofline_frac": round(flops / us / 1e6 / MFMA_FP8_PEAK_TFLOPS, 4),
           "work": "dh = dy . W2^T, SwiGLU derivative, MX-E4M3 rows + 32-row transposed blocks, dw"}
    log(f"prefill_backward: {res}")
    del dw, w2t, ws, hT, pre
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=160)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated between calls")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="also time the oracle on every whole workload (median of 3; minutes of CPU work)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the latency lines of the tiny, full-expert, prefill and shared-expert workloads")
    ap.add_argument("--only", choices=["tiny", "full", "prefill", "shared", "prefill_token_ring",
                                       "prefill_backward"],
                    help="time only this workload's layer (no decode bench, no oracle) and print its line; "
                         "for profiling one workload")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the expert-parallel layer on one MI355X; "
              "it has no multi-GPU mode (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import routed_grouped_gemm_amd as moe
    import synth
    from synth import device

    torch.cuda.set_device(0)
    if args.only:
        if args.only == "prefill_backward":
            print(json.dumps({"prefill_backward": backward_workload(torch, moe, synth, device)}), flush=True)
        else:
            print(json.dumps(other_workloads(torch, moe, synth, device, [args.only])), flush=True)
        return
    c = synth.config("decode", 128)
    fp4 = c.w_fmt == "e2m1"
    t_setup = time.perf_counter()
    dw = device.build_weights(c)
    copies = [dw]
    for _ in range(args.copies - 1):
        w1 = moe.PackedWeights.empty(c.n_local, 2 * c.I, c.H, dw.w1.fmt, True)
        w2 = moe.PackedWeights.empty(c.n_local, c.H, c.I, dw.w2.fmt, False)
        w1.buf.copy_(dw.w1.buf)
        w2.buf.copy_(dw.w2.buf)
        copies.append(device.DeviceWeights(w1, w2, None))
    cfg = {T: synth.config("decode", T) for T in DECODE_T}
    inputs = {T: [device.build_inputs(cfg[T], v) for v in range(N_VARIANTS)] for T in DECODE_T}
    wss = {T: moe.LayerWorkspace(T, c.E, c.k, c.n_local, c.H, c.I) for T in DECODE_T}
    outs = {T: torch.empty((T, c.H), dtype=torch.uint16, device="cuda") for T in DECODE_T}
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s on {torch.cuda.get_device_name(0)}")

    # active experts and rows of every (T, draw): one untimed pass
    active, rows = {}, {}
    for T in DECODE_T:
        for v in range(N_VARIANTS):
            lg, xq, xs = inputs[T][v]
            moe.moe_layer(lg, xq, xs, dw.w1, dw.w2, c.k, c.e0, c.n_local, None, 0, out=outs[T], ws=wss[T])
            cnt = wss[T].view("counts").cpu()
            active[T, v] = int((cnt > 0).sum())
            rows[T, v] = int(cnt.sum())

    def call(T, v, w):
        lg, xq, xs = inputs[T][v]
        moe.moe_layer(lg, xq, xs, w.w1, w.w2, c.k, c.e0, c.n_local, None, 0, out=outs[T], ws=wss[T])

    def step(i):
        # call j of step i takes weight copy (i + j) % copies: consecutive
        # calls never share a copy, and every T cycles through all of them
        for j, T in enumerate(DECODE_T):
            call(T, i % N_VARIANTS, copies[(i + j) % len(copies)])

    def step_bytes(i):
        return sum(layer_bytes(T, c.E, c.H, c.I, active[T, i % N_VARIANTS], fp4) for T in DECODE_T)

    # The launch sequence of exactly the warm-up steps and of exactly the
    # timed steps is captured into one HIP graph each and replayed once, so
    # the host never paces the GPU and the measured work is the same
    # whatever --steps and --warmup are.
    def capture(first, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(first, first + n):
                step(i)
        return g

    torch.cuda.synchronize()
    warm_graph = capture(0, args.warmup) if args.warmup > 0 else None
    timed_graph = capture(args.warmup, args.steps)
    torch.cuda.synchronize()
    # The measured HBM read rate: the library's plain streaming read of 2 GiB
    # (one pass per launch), 20 launches between HIP events. It runs here,
    # after the host-side graph captures (during which the GPU idles) and
    # right before the warm-up steps, so that the timed steps start on a GPU
    # that has been busy for several milliseconds (with 5 warm-up steps the
    # step rate was still rising over the first 20-60 steps otherwise).
    stream = torch.cuda.current_stream()
    nb = 1 << 31
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    sink = torch.empty(moe.MOE_HBM_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    for _ in range(3):
        moe.moe_hbm_read_probe(buf, sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(20):
        moe.moe_hbm_read_probe(buf, sink)
    b.record(stream)
    torch.cuda.synchronize()
    read_tbps = nb * 20 / (a.elapsed_time(b) * 1e-3) / 1e12
    del buf, sink
    if warm_graph is not None:
        warm_graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timed_graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del warm_graph, timed_graph
    total_bytes = sum(step_bytes(i) for i in range(args.warmup, args.warmup + args.steps))
    value = total_bytes / wall / 1e12
    ms_per_step = wall / args.steps * 1e3

    # the same steps launched eagerly (one host call per layer), for reference
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    eager_tbps = sum(step_bytes(i) for i in range(args.steps)) / (time.perf_counter() - t0) / 1e12

    # a plain copy of known size (1 GiB), so hardware byte counters collected
    # on this run can be calibrated against it
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    # per-T layer latency: a graph of 16 consecutive calls (one per routing
    # draw, rotating weight copies), timed with HIP events on the replay stream
    stream = torch.cuda.current_stream()

    def graph_latency(T, weight_copies, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for v in range(N_VARIANTS):
                call(T, v, weight_copies[v % len(weight_copies)])
        g.replay()
        torch.cuda.synchronize()
        # back-to-back replays, each between its own pair of events: the mean
        # over all of them, and the per-replay means (each over the 16 draws)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            g.replay()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[reps]) * 1e3 / (reps * N_VARIANTS)
        each = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 / N_VARIANTS for i in range(reps))
        return us, each

    per_t = {}
    for T in DECODE_T:
        # 20 replays: min / p10 / median / p90 / max of the per-replay means
        us, each = graph_latency(T, copies, 20)
        b = sum(layer_bytes(T, c.E, c.H, c.I, active[T, v], fp4) for v in range(N_VARIANTS)) / N_VARIANTS
        # warm cache, labelled as such: every call on the same weight copy, so
        # the weights of the smaller T stay in the 256 MB MALL between calls
        wus, _ = graph_latency(T, copies[:1], 4)
        per_t[str(T)] = {"latency_us": round(us, 2), "TBps": round(b / us / 1e6, 3), **spread(each),
                         "warm_cache_latency_us": round(wus, 2),
                         "active_experts": round(sum(active[T, v] for v in range(N_VARIANTS)) / N_VARIANTS, 2)}

    # dominant kernel: grouped W1, launched through its own entry point on
    # the grouping each layer call of the step sequence produced (saved per
    # routing draw and T), with R_max = that call's row count, so the library
    # picks the configuration moe_layer picks. One graph holds the W1
    # launches of 16 steps in step order (T = 1, 8, 32, 128 per draw, weight
    # copies rotating as in the steps), so, as in the steps, each launch
    # streams its weights from HBM; HIP events on the replay stream bracket
    # the replays, and the average launch duration is their time over the
    # launches (the short gaps between graph nodes included).
    grouping = {}
    for T in DECODE_T:
        for v in range(N_VARIANTS):
            call(T, v, dw)
            ws = wss[T]
            grouping[T, v] = {n: ws.view(n).clone() for n in ("counts", "offsets", "offsets32", "row_src",
                                                               "row_w")}
    torch.cuda.synchronize()

    def w1_launch(T, v, w):
        gsv = grouping[T, v]
        lg, xq, xs = inputs[T][v]
        ws = wss[T]
        moe.moe_grouped_w1(w.w1, gsv["counts"], gsv["offsets"], gsv["row_w"], xq, xs, c.I, 0,
                           offsets32=gsv["offsets32"], hq=ws.view("hq"), hs=ws.view("hs"),
                           row_src=gsv["row_src"], R_max=max(rows[T, v], 1))

    w1_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(w1_graph):
        for v in range(N_VARIANTS):
            for j, T in enumerate(DECODE_T):
                w1_launch(T, v, copies[(v + j) % len(copies)])
    w1_graph.replay()
    torch.cuda.synchronize()
    w1_reps = 5
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(w1_reps):
        w1_graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    w1_ms = a.elapsed_time(b)
    nlaunch = w1_reps * N_VARIANTS * len(DECODE_T)
    w1_b = w1_reps * sum(w1_bytes(rows[T, v], c.H, c.I, active[T, v], fp4)
                         for v in range(N_VARIANTS) for T in DECODE_T)
    del w1_graph
    w1_gbs = w1_b / (w1_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(w1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(w1_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "kernel": "grouped_gemm_kernel (W1, MXFP4)",
                "avg_launch_us": round(w1_ms * 1e3 / nlaunch, 2), "launches": nlaunch,
                "bytes_per_launch": round(w1_b / nlaunch)}

    hbm_read = {"kernel": "hbm_read_kernel: one streaming read of 2 GiB per launch",
                "TBps": round(read_tbps, 3), "frac_of_peak": round(read_tbps * 1e3 / HBM_PEAK_GBS, 4),
                "value_over_measured": round(value / read_tbps, 4),
                "roofline_over_measured": round(w1_gbs / 1e3 / read_tbps, 4)}
    log(f"measured HBM read rate: {hbm_read}")

    others = None
    if not args.no_other_workloads:
        others = other_workloads(torch, moe, synth, device, ["tiny", "full", "prefill", "shared",
                                                            "prefill_token_ring"])
        others["prefill_backward"] = backward_workload(torch, moe, synth, device)

    cpu = None
    if not args.no_cpu_baseline:
        cpu, _ = cpu_baseline(cfg, lambda T, act: layer_bytes(T, c.E, c.H, c.I, act, fp4))
        if others is not None:
            import numpy  # noqa: F401  (loads BLAS so its thread count is visible)
            threads = oracle_threads()
            for name, ntok in ORACLE_SAMPLE_TOKENS.items():
                others[name]["cpu_oracle"] = cpu_oracle_sample(name, ntok, threads)
                log(f"{name} oracle: {others[name]['cpu_oracle']}")

    cpu_full = None
    if args.cpu_full:
        import numpy  # noqa: F401
        cpu_full = cpu_oracle_full([("tiny", None), ("decode", 1), ("decode", 8), ("decode", 32),
                                    ("decode", 128), ("shared", None), ("full", None), ("prefill", None)],
                                   oracle_threads())

    line = {
        "metric": "MoE layer latency µs + achieved HBM TB/s (decode), MFMA TFLOPS (prefill)",
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1 (MX), fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "decode share: T in {1,8,32,128} per step, H=7168, I=2048, "
                               "top-8 of 256 experts, experts 0-31 local, MXFP4 weights",
                   "weight_copies": args.copies, "routing_draws": N_VARIANTS},
        "per_T": per_t,
        "eager_TBps": round(eager_tbps, 4),
        "roofline": roofline,
        "hbm_read_measured": hbm_read,
        "cpu_baseline": cpu,
        "other_workloads": others,
    }
    if cpu_full is not None:
        line["cpu_oracle_full"] = cpu_full
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
