#!/usr/bin/env python3
"""Benchmark of the RG-LRU scan hot path on one MI355X.

One step = rglru_fwd (training mode: writes the float32 checkpoint) followed by
rglru_bwd (reverse scan, pointwise gradients and the lambda-gradient
reduction) over one batch of the workload, inputs already resident in HBM.
The default workload is the pages' measured shape, B=4, L=2048, W=2048, bf16
io with a float32 carry, zero initial state and no resets.

Cache honesty: the step's working set (about 270 MB) would otherwise sit in
the 256 MB Infinity Cache between steps, so the benchmark rotates through
several copies of every buffer (more than twice the cache in total) and each
step reads data last touched two steps earlier.

Two timed passes of the same steps: `value` is the wall time of the first,
which has nothing on the stream but the work; the per-call durations behind
the roofline figures come from the second, whose library calls are bracketed
by HIP events on the launch stream.

Prints one JSON line (see the "fields" list in the docstring of main()).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (the published figure counts packed FMA)
METRIC = "RG-LRU fwd & fwd+bwd ms + % HBM peak, B=4 L=2048 W=2048 bf16"
FWD_BYTES_PER_ELEM = {"bf16": 8, "f32": 16}    # read x, gate_x, gate_a; write h
BWD_BYTES_PER_ELEM = {"bf16": 14, "f32": 28}   # read x, gate_x, gate_a, dh; write dx, dgate_x, dgate_a


_CPU_INPUT = None


def _cpu_worker(task):
    """One worker's share of the oracle: channels [lo, hi) for `reps` fwd+bwd passes."""
    import oracle

    lo, hi, reps = task
    x, gx, ga, dh, lam, reset, h0 = _CPU_INPUT
    sl = slice(lo, hi)
    h0s = None if h0 is None else h0[:, sl]
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.rglru_forward(x[:, :, sl], gx[:, :, sl], ga[:, :, sl], lam[sl], reset, h0s)
        oracle.rglru_backward(x[:, :, sl], gx[:, :, sl], ga[:, :, sl], lam[sl], dh[:, :, sl], reset, h0s)
    return time.perf_counter() - t0


def cpu_cores() -> int:
    """Host threads for the oracle: the cores this process may run on, at most 16
    (one GPU's share of a shared 8-GPU host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, inp, seconds_target=12.0):
    """The float64 oracle (untuned) on the same workload, channels split over a process pool.

    Channels are independent, so each worker runs the oracle's forward and
    backward on its own contiguous channel range; the pool covers the whole
    width. Must run before anything in this process touches the GPU: the
    workers are forked.
    """
    import multiprocessing as mp

    import numpy as np

    global _CPU_INPUT
    cores = cpu_cores()
    _CPU_INPUT = (inp.x.value, inp.gx.value, inp.ga.value, inp.dh.value, inp.lam.astype(np.float64),
                  inp.reset, None if inp.h0 is None else inp.h0.astype(np.float64))
    W = wl.width
    bounds = np.linspace(0, W, cores + 1).astype(int)
    ranges = [(int(bounds[k]), int(bounds[k + 1])) for k in range(cores) if bounds[k + 1] > bounds[k]]
    with mp.get_context("fork").Pool(processes=len(ranges)) as pool:
        t0 = time.perf_counter()
        pool.map(_cpu_worker, [(lo, hi, 1) for lo, hi in ranges])
        first = time.perf_counter() - t0
        reps = int(max(1, min(20, (seconds_target - first) // max(first, 1e-3))))
        t0 = time.perf_counter()
        pool.map(_cpu_worker, [(lo, hi, reps) for lo, hi in ranges])
        el = time.perf_counter() - t0
    _CPU_INPUT = None
    return {
        "value": el / reps * 1e3,
        "unit": "ms",
        "cores": len(ranges),
        "kind": "oracle",
        "sample": f"the whole workload (B={wl.batch} L={wl.length} W={W}), fwd+bwd, width split over "
                  f"{len(ranges)} worker processes, {reps} timed passes ({el:.1f} s) after one untimed",
    }


DECODE_SHAPES = ((1, 1, 2048), (4, 1, 2048), (16, 1, 4096), (4, 8, 2048))


def decode(args):
    """Decode-step latency: B rows, L = 1 (or up to 8) new tokens, h0 in, h_last out.

    Each shape runs `steps` calls of rglru_fwd_scratch (no workspace, nothing
    allocated) back to back, first eagerly (host launch rate included), then
    captured once into a HIP graph and replayed, which leaves the GPU time per
    step; the graph's result is checked bitwise against the eager call.
    """
    import numpy as np
    import torch

    import gated_linear_recurrence_amd as glr
    import synth

    glr.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps = max(args.steps, 20)
    rows = []
    for B, L, W in DECODE_SHAPES:
        wl = synth.dataclasses.replace(synth.WORKLOADS[2].resized(batch=B, length=L, width=W), doc_mean=None)
        inp = synth.make_inputs(wl)

        def io(st):
            return torch.from_numpy(np.ascontiguousarray(st.raw).view(np.int16)).view(torch.bfloat16).to(dev)

        x, gx, ga = io(inp.x), io(inp.gx), io(inp.ga)
        lam = torch.from_numpy(inp.lam).to(dev)
        h0 = torch.from_numpy(inp.h0).to(dev)
        h = torch.empty_like(x)
        h_last = torch.empty((B, W), dtype=torch.float32, device=dev)

        def call():
            glr.rglru_fwd_scratch(x, gx, ga, lam, None, h0, h=h, h_last=h_last)

        for _ in range(args.warmup + 5):
            call()
        torch.cuda.synchronize()
        ref_h, ref_hl = h.clone(), h_last.clone()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / steps
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                for _ in range(steps):
                    call()
        torch.cuda.synchronize()
        h.zero_()
        h_last.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not (torch.equal(h, ref_h) and torch.equal(h_last, ref_hl)):
            print(f"graph replay differs from the eager call at B={B} L={L} W={W}", file=sys.stderr)
            sys.exit(3)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / steps
        if not (torch.equal(h, ref_h) and torch.equal(h_last, ref_hl)):
            print(f"second graph replay differs at B={B} L={L} W={W}", file=sys.stderr)
            sys.exit(3)
        del graph
        rows.append({"batch": B, "length": L, "width": W, "eager_us_per_step": round(eager_us, 2),
                     "graph_us_per_step": round(graph_us, 2),
                     "bytes_per_step": B * L * W * 2 * 4 + B * W * 4 * 2})
    print(json.dumps({"metric": "RG-LRU decode step latency (graph replay)", "unit": "us",
                      "higher_is_better": False, "n_gpus": 1, "steps": steps, "dtype": "bf16",
                      "data": "synthetic", "entry_point": "rglru_fwd_scratch", "shapes": rows}), flush=True)


def main():
    """Fields: metric, value (fwd+bwd ms per step), unit, n_gpus, steps, warmup, ms_per_step,
    higher_is_better, scaling, vs_baseline, dtype, data, config, fwd_ms, bwd_ms, elements_per_s,
    hbm_frac_fwd, hbm_frac_fwd_bwd, roofline, roofline_fwd, cpu_baseline; with the projections
    (workloads 4 and 5) also projection and fused_forward."""
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1, help="synth workload id (1 = pages' shape)")
    ap.add_argument("--chunk", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sets", type=int, default=3, help="rotating buffer copies (cache honesty)")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a known-size "
                         "reference for hardware traffic counters)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="with the default workload, skip the long-sequence and projection workloads "
                         "measured after it")
    ap.add_argument("--decode", action="store_true",
                    help="instead: decode-step latency (L = 1, h0 in, h_last out) through the "
                         "allocation-free forward, eager and replayed from a HIP graph")
    ap.add_argument("--delta-only", action="store_true",
                    help="instead: only the gated delta rule workloads (one JSON object per workload)")
    ap.add_argument("--delta-workload", type=int, default=None, choices=(10, 11, 12),
                    help="with --delta-only: that delta-rule workload alone")
    ap.add_argument("--delta-no-backward", action="store_true",
                    help="with --delta-only: skip the delta rule's training step (forward with "
                         "checkpoint + backward), so the forward kernels run in one configuration")
    args = ap.parse_args()

    if args.delta_only:
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        if args.calibration_copy_mb > 0:
            calibration_copy(args.calibration_copy_mb)
        for w in ((10, 11, 12) if args.delta_workload is None else (args.delta_workload,)):
            print(json.dumps(run_delta(args, w, args.steps, args.warmup)), flush=True)
        return

    if args.decode:
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        decode(args)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the scan shards by channel or batch with no exchange in the forward)",
              file=sys.stderr)
        sys.exit(2)

    out = run_workload(args, args.workload, args.steps, args.warmup, True)
    if args.workload == 1 and not args.no_other_workloads:
        # The long-sequence shape and the pages' measured scope (projections
        # in the step, and the fused forward), measured in the same run;
        # reported beside the headline, which they do not change.
        import torch
        other = {}
        for wid in (3, 5):
            torch.cuda.empty_cache()
            o = run_workload(args, wid, 20, 3, False)
            keep = ("config", "value", "fwd_ms", "bwd_ms", "hbm_frac_fwd", "hbm_frac_fwd_bwd", "projection",
                    "fused_forward")
            other[o["config"]["workload"]] = {k: o[k] for k in keep if k in o}
            other[o["config"]["workload"]]["roofline_frac_bwd"] = o["roofline"]["frac"]
            other[o["config"]["workload"]]["roofline_frac_fwd"] = o["roofline_fwd"]["frac"]
        out["other_workloads"] = other
        torch.cuda.empty_cache()
        out["delta_rule"] = {str(w): run_delta(args, w, 20, 3) for w in (10, 11, 12)}
    print(json.dumps(out), flush=True)


def calibration_copy(mib):
    """One device-to-device copy of `mib` MiB: a known-size reference for the hardware traffic counters."""
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def measured_traffic(key):
    """Per-call HBM bytes of a library call from profiles/traffic.json (None when not measured)."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            return (json.load(f).get(key) or {}).get("bytes")
    except (OSError, ValueError):
        return None


def delta_cpu_baseline(inp, seconds_target=2.0):
    """The float64 oracle (untuned, one thread) on a bounded sample of a delta-rule workload:
    one (batch row, value head) pair over up to 256 tokens, repeated for about
    seconds_target, scaled to the whole workload's (row, head, token) count."""
    import numpy as np

    import oracle

    wl = inp.wl
    T = min(wl.length, 256)
    kh = 0
    sl = lambda st: st.value[:1, :T, kh:kh + 1]
    g = inp.g[:1, :T, :1].astype(np.float64)
    beta = inp.beta[:1, :T, :1].astype(np.float64)
    h0 = None if inp.h0 is None else inp.h0[:1, :1]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.recurrent_delta_rule(sl(inp.q), sl(inp.k), inp.v.value[:1, :T, :1], g, beta, initial_state=h0)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds_target:
            break
    per_token_head = el / reps / T
    total = per_token_head * wl.batch * wl.length * wl.v_heads
    return {
        "value": round(total * 1e3, 3), "unit": "ms", "cores": 1, "kind": "oracle",
        "sample": f"one (row, head) pair over {T} tokens, {reps} passes in {el:.1f} s, scaled to "
                  f"{wl.batch} x {wl.length} x {wl.v_heads} (row, token, head) steps",
    }


def run_delta(args, wid, steps, warmup):
    """Gated delta rule forward (rglru_delta_rule_fwd) on one delta workload: its JSON object.

    Rotates through enough copies of the inputs and outputs to exceed the
    Infinity Cache; the events bracket `steps` back-to-back calls on the
    launch stream (one kernel launch per call)."""
    import numpy as np
    import torch

    import gated_linear_recurrence_amd as glr
    from synth import delta as sd

    wl = sd.DELTA_WORKLOADS[wid]
    inp = sd.make_delta_inputs(wl)
    cpu = None if args.no_cpu_baseline else delta_cpu_baseline(inp)
    glr.load_library()
    dev = torch.device("cuda:0")

    def io(st):
        t = torch.from_numpy(np.ascontiguousarray(st.raw)).to(dev)
        return t.view(torch.bfloat16) if st.io == "bf16" else t

    base = dict(q=io(inp.q), k=io(inp.k), v=io(inp.v), g=torch.from_numpy(inp.g).to(dev),
                beta=torch.from_numpy(inp.beta).to(dev))
    h0 = None if inp.h0 is None else torch.from_numpy(inp.h0).to(dev)
    B, T, Hv, Dk, Dv = wl.batch, wl.length, wl.v_heads, wl.k_dim, wl.v_dim
    es = 2 if wl.io == "bf16" else 4
    state_bytes = B * Hv * Dk * Dv * 4
    nbytes = (B * T * wl.k_heads * Dk * 2 * es + B * T * Hv * Dv * 2 * es
              + B * T * Hv * (Dk if wl.kda else 1) * 4 + B * T * Hv * 4
              + state_bytes * (2 if h0 is not None else 1))
    n_sets = max(2, int(np.ceil(600e6 / max(nbytes, 1))))
    n_sets = min(n_sets, 8)
    sets = []
    for _ in range(n_sets):
        d = {kk: vv.clone() for kk, vv in base.items()}
        d["o"] = torch.empty_like(d["v"])
        d["fs"] = torch.empty((B, Hv, Dk, Dv), dtype=torch.float32, device=dev)
        d["h0"] = None if h0 is None else h0.clone()
        sets.append(d)
    del base

    def call(d):
        glr.rglru_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"],
                                 o=d["o"], final_state=d["fs"])

    def timed(fn):
        for i in range(warmup):
            fn(sets[i % n_sets])
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(sets[i % n_sets])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(call)
    flops = 7 * B * T * Hv * Dk * Dv   # per state element and token: decay, two dot-product FMAs, one write FMA
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    chunk = None
    shape = glr.ops._lib.rglru_delta_shape_t(B, T, wl.k_heads, Hv, Dk, Dv, 1 if wl.io == "bf16" else 0,
                                             1 if wl.kda else 0, 0, 1.0)
    ws_bytes = glr.rglru_delta_chunk_workspace_bytes(shape, 0)
    if ws_bytes > 0 and T >= 64:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def chunk_call(d):
            glr.rglru_delta_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"],
                                      o=d["o"], final_state=d["fs"], workspace=ws)

        cms = timed(chunk_call)
        # dense products of the chunk form per (64-token chunk, head), as multiply-adds:
        # K K^T, Q K^T and W (64 x 64 x Dk each), U~ and P U (64 x 64 x Dv each), and
        # U = U~ - W S, Q S and the state update (64 x Dk x Dv each)
        n_chunks = B * Hv * ((T + 63) // 64)
        cflops = 2 * n_chunks * (3 * 64 * 64 * Dk + 2 * 64 * 64 * Dv + 3 * 64 * Dk * Dv)
        ctf = cflops / (cms * 1e-3) / 1e12
        chunk = {
            "call": "rglru_delta_chunk_fwd (64-token chunks, bf16 MFMA)", "ms": round(cms, 5),
            "tokens_per_s": B * T / (cms * 1e-3),
            "roofline": {"kernel": "gdn_chunk_prep + gdn_chunk_state", "bound": "mfma", "achieved": round(ctf, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ctf / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(f"{wl.name}:delta_chunk"),
                         "algorithmic_flops_per_launch": cflops, "launch_ms": round(cms, 5)},
            "speedup_vs_token_recurrence": round(ms / cms, 3),
        }
    backward = None
    if T >= 16 and not getattr(args, "delta_no_backward", False):
        # training step of the token form: the forward writing its checkpoint, then the backward
        n_ck = glr.rglru_delta_ckpt_elems(shape, 0)
        for d in sets:
            d["ck"] = torch.empty(n_ck, dtype=torch.float32, device=dev)
            d["do"] = torch.randn_like(d["v"], dtype=torch.float32).to(d["v"].dtype)
        bws = torch.empty(max(glr.rglru_delta_bwd_workspace_bytes(shape, 0), 1), dtype=torch.uint8, device=dev)

        def fwd_train(d):
            glr.rglru_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"],
                                     o=d["o"], final_state=d["fs"], ckpt=d["ck"])

        def bwd(d):
            glr.rglru_delta_rule_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["ck"], d["do"], d["fs"],
                                     workspace=bws)

        ftm = timed(fwd_train)
        for d in sets:
            fwd_train(d)
        btm = timed(bwd)
        # per state element and token: recomputing the step (5 flops) and the reverse step
        # (17: the read-out's gradient, dq, du, dk, the decayed gradient, dg and its decay)
        bflops = 22 * B * T * Hv * Dk * Dv
        btf = bflops / (btm * 1e-3) / 1e12
        backward = {
            "call": "rglru_delta_rule_fwd with its checkpoint + rglru_delta_rule_bwd (token form)",
            "fwd_train_ms": round(ftm, 5), "bwd_ms": round(btm, 5), "step_ms": round(ftm + btm, 5),
            "roofline": {"kernel": "delta_bwd_kernel + delta_bwd_reduce", "bound": "alu", "achieved": round(btf, 2),
                         "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(btf / FP32_VECTOR_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(f"{wl.name}:delta_bwd"),
                         "algorithmic_flops_per_launch": bflops, "launch_ms": round(btm, 5)},
        }
    del sets
    torch.cuda.empty_cache()
    return {
        "backward": backward,
        "call": "rglru_delta_rule_fwd (token recurrence)",
        "config": {"workload": wl.name, "batch": B, "length": T, "k_heads": wl.k_heads, "v_heads": Hv,
                   "k_dim": Dk, "v_dim": Dv, "io": wl.io, "decay": "KDA" if wl.kda else "GDN",
                   "h0": inp.h0 is not None},
        "ms": round(ms, 5),
        "tokens_per_s": B * T / (ms * 1e-3),
        "roofline": {"kernel": "delta_fwd_kernel", "bound": "alu", "achieved": round(tf, 2),
                     "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(f"{wl.name}:delta_token"),
                     "algorithmic_flops_per_launch": flops, "launch_ms": round(ms, 5)},
        "hbm": {"algorithmic_bytes": nbytes, "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)},
        "chunk_form": chunk,
        "cpu_baseline": cpu,
    }


def run_workload(args, wid, steps, warmup, with_cpu):
    """Measures one synth workload: its bench JSON object."""
    import numpy as np

    import synth

    wl = synth.WORKLOADS[wid]
    chunk = wl.chunk if args.chunk is None else args.chunk
    inp = synth.make_inputs(wl)
    # the oracle's pool is forked, so it runs before the GPU is touched
    cpu = None if (args.no_cpu_baseline or not with_cpu) else cpu_baseline(wl, inp)

    import torch

    import gated_linear_recurrence_amd as glr

    glr.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, L, W = wl.batch, wl.length, wl.width
    N = B * L * W

    def io_tensor(s):
        if s.io == "f32":
            return torch.from_numpy(np.ascontiguousarray(s.raw)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(s.raw).view(np.int16)).view(torch.bfloat16).to(dev)

    base = {k: io_tensor(getattr(inp, k)) for k in ("x", "gx", "ga", "dh")}
    lam = torch.from_numpy(inp.lam).to(dev)
    reset = None if inp.reset is None else torch.from_numpy(inp.reset).to(dev)
    h0 = None if inp.h0 is None else torch.from_numpy(inp.h0).to(dev)
    shape = glr.make_shape(B, L, W, base["x"].dtype, chunk)
    proj = wl.proj_blocks > 0
    if proj:
        wx, wa, bx, ba = (io_tensor(getattr(inp, k)) for k in ("wx", "wa", "bx", "ba"))
    n_ck = glr.rglru_ckpt_elems(shape)
    sets = []
    for s in range(args.sets):
        d = {k: v.clone() for k, v in base.items()}
        d["h"] = torch.empty_like(d["x"])
        d["h_last"] = torch.empty((B, W), dtype=torch.float32, device=dev)
        d["ckpt"] = torch.empty(n_ck, dtype=torch.float32, device=dev)
        for k in ("dx", "dgx", "dga"):
            d[k] = torch.empty_like(d["x"])
        d["dlam"] = torch.empty(W, dtype=torch.float32, device=dev)
        d["dh0"] = torch.empty((B, W), dtype=torch.float32, device=dev) if h0 is not None else None
        d["ws"] = glr.Workspace(dev)
        d["ws"].get(glr.rglru_workspace_bytes(shape))
        if proj:
            d["gxp"] = torch.empty_like(d["x"])
            d["gap"] = torch.empty_like(d["x"])
            d["dxp"] = torch.empty_like(d["x"])
        sets.append(d)
    del base
    stream = torch.cuda.current_stream(dev)

    def step(d, evs=None):
        """One pass of the hot path; evs[k] brackets the k-th launch group."""
        def mark(k):
            if evs is not None:
                evs[k].record(stream)
        mark(0)
        if proj:
            x2 = d["x"].view(B * L, W)
            glr.rglru_blockdiag_gate_proj_fwd(x2, wx, bx, wa, ba, gate_x=d["gxp"].view(B * L, W),
                                              gate_a=d["gap"].view(B * L, W))
            gx, ga = d["gxp"], d["gap"]
        else:
            gx, ga = d["gx"], d["ga"]
        mark(1)
        glr.rglru_fwd(d["x"], gx, ga, lam, reset, h0, chunk=chunk, h=d["h"], h_last=d["h_last"],
                      ckpt=d["ckpt"], workspace=d["ws"])
        mark(2)
        glr.rglru_bwd(d["x"], gx, ga, lam, reset, d["ckpt"], d["dh"], None, chunk=chunk,
                      want_dh0=h0 is not None, dx=d["dx"], dgate_x=d["dgx"], dgate_a=d["dga"], dlam=d["dlam"],
                      dh0=d["dh0"], workspace=d["ws"])
        mark(3)
        if proj:
            glr.rglru_blockdiag_gate_proj_bwd(d["x"].view(B * L, W), wx, wa, d["dgx"].view(B * L, W),
                                              d["dga"].view(B * L, W), d["dx"].view(B * L, W),
                                              dx_out=d["dxp"].view(B * L, W))
        mark(4)

    if args.calibration_copy_mb > 0:
        calibration_copy(args.calibration_copy_mb)
    for i in range(warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # Throughput: exactly `steps` steps with nothing but the work on the
    # stream. A timing event costs about 3 us of GPU time on this part (the
    # stream drains before its timestamp), so the per-call events are kept
    # out of this pass.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Per-call durations (the roofline figures): the same steps again, each
    # library call bracketed by events recorded on the launch stream.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    pfwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    fwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    bwd_ms = [e[2].elapsed_time(e[3]) for e in evs]
    pbwd_ms = [e[3].elapsed_time(e[4]) for e in evs]
    fused = None
    if proj:
        # The fused forward (both projections inside the scan), with and
        # without the logits as outputs, timed the same way. Its result is
        # bitwise that of the projection followed by the scan with 64-step tiles.
        def fused_call(d, gates):
            glr.rglru_blockdiag_fused_fwd(d["x"], wx, bx, wa, ba, lam, reset, h0, h=d["h"], h_last=d["h_last"],
                                          ckpt=d["ckpt"], gate_x=d["gxp"] if gates else None,
                                          gate_a=d["gap"] if gates else None, workspace=d["ws"])
        fused = {}
        for gates in (False, True):
            for i in range(warmup):
                fused_call(sets[i % len(sets)], gates)
            fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps)]
            torch.cuda.synchronize()
            for i in range(steps):
                fev[i][0].record(stream)
                fused_call(sets[i % len(sets)], gates)
                fev[i][1].record(stream)
            torch.cuda.synchronize()
            fused[gates] = float(np.mean([a.elapsed_time(b) for a, b in fev]))
    err = max(d["ws"].error_bits() for d in sets)
    if err:
        print(f"look-back spin limit reported (error bits {err}); timings invalid", file=sys.stderr)
        sys.exit(3)

    ms_per_step = wall * 1e3 / steps
    fwd_avg = float(np.mean(fwd_ms))
    bwd_avg = float(np.mean(bwd_ms))
    fb = FWD_BYTES_PER_ELEM[wl.io] * N
    bb = BWD_BYTES_PER_ELEM[wl.io] * N
    fwd_gbs = fb / (fwd_avg * 1e-3) / 1e9
    bwd_gbs = bb / (bwd_avg * 1e-3) / 1e9
    fb_gbs = (fb + bb) / (ms_per_step * 1e-3) / 1e9
    tr = {}
    prof = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(prof):
        # bytes per call from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE)
        # scaled by a copy of known size; refreshed whenever the kernels change
        with open(prof) as f:
            tr = json.load(f)

    def measured(group):
        return (tr.get(f"{wl.name}:{group}") or {}).get("bytes")

    traffic = measured("bwd")
    fwd_traffic = measured("fwd")
    out = {
        "metric": METRIC,
        "value": round(ms_per_step, 5),
        "unit": "ms",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.io,
        "data": "synthetic (seeded N(0,1) inputs and logits, decay U[0.9,0.999]; no datasets)",
        "config": {"workload": wl.name, "batch": B, "length": L, "width": W, "io": wl.io,
                   "chunk": chunk or "library default (forward 128 steps, backward 64)", "resets": wl.doc_mean is not None, "h0": wl.h0,
                   "step": ("rglru_blockdiag_gate_proj_fwd + rglru_fwd + rglru_bwd + rglru_blockdiag_gate_proj_bwd"
                            if proj else "rglru_fwd + rglru_bwd")},
        "fwd_ms": round(fwd_avg, 5),
        "bwd_ms": round(bwd_avg, 5),
        "fwd_plus_bwd_ms": round(fwd_avg + bwd_avg, 5),
        "elements_per_s": N / (ms_per_step * 1e-3),
        "hbm_frac_fwd": round(fwd_gbs / HBM_PEAK_GBS, 4),
        "hbm_frac_fwd_bwd": round(fb_gbs / HBM_PEAK_GBS, 4),
        # The backward is one library call of two launches (the reverse scan
        # with the pointwise gradients, then the fixed-order lambda-gradient
        # sum); the events bracket both and the bytes are the backward's
        # algorithmic bytes.
        "roofline": {
            "kernel": "rglru_bwd: bwd_kernel + bwd_dlam_kernel",
            "bound": "hbm",
            "achieved": round(bwd_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(bwd_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bb,
            "launch_ms": round(bwd_avg, 5),
        },
        "roofline_fwd": {
            "kernel": "rglru_fwd: fwd_kernel",
            "bound": "hbm",
            "achieved": round(fwd_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(fwd_gbs / HBM_PEAK_GBS, 4),
            "traffic": fwd_traffic,
            "algorithmic_bytes_per_launch": fb,
            "launch_ms": round(fwd_avg, 5),
        },
        "cpu_baseline": None,
    }
    if proj:
        # projection: x read once, both gates written; backward reads x, both gate
        # gradients and the scan's dx, writes dx (weights and their gradients are small)
        T = B * L
        pf_bytes = 3 * 2 * N
        pb_bytes = 5 * 2 * N
        flops = 2 * 2 * T * W * wl.proj_block
        pf = float(np.mean(pfwd_ms))
        pbk = float(np.mean(pbwd_ms))
        fwd_tf = flops / (pf * 1e-3) / 1e12
        bwd_tf = 2 * flops / (pbk * 1e-3) / 1e12
        # the whole step's algorithmic bytes (scan and projections) over its time
        out["hbm_frac_fwd_bwd"] = round((fb + bb + pf_bytes + pb_bytes) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        out["projection"] = {
            "fwd_ms": round(pf, 5), "bwd_ms": round(pbk, 5),
            "fwd_gbs": round(pf_bytes / (pf * 1e-3) / 1e9, 1), "bwd_gbs": round(pb_bytes / (pbk * 1e-3) / 1e9, 1),
            "fwd_hbm_frac": round(pf_bytes / (pf * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bwd_hbm_frac": round(pb_bytes / (pbk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "fwd_tflops": round(fwd_tf, 1), "bwd_tflops": round(bwd_tf, 1),
            "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "fwd_mfma_frac": round(fwd_tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "bwd_mfma_frac": round(bwd_tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "fwd_algorithmic_bytes": pf_bytes, "bwd_algorithmic_bytes": pb_bytes,
            "fwd_traffic": measured("proj_fwd"), "bwd_traffic": measured("proj_bwd"),
        }
        # x read and h written (2 + 2 bytes per element), plus both logits
        # written when they are outputs
        fz = fused[False]
        fzg = fused[True]
        out["fused_forward"] = {
            "call": "rglru_blockdiag_fused_fwd (64-step tiles)",
            "ms": round(fz, 5),
            "with_logits_ms": round(fzg, 5),
            "two_call_ms": round(pf + fwd_avg, 5),
            "algorithmic_bytes": 2 * 2 * N,
            "with_logits_algorithmic_bytes": 4 * 2 * N,
            "hbm_frac": round(2 * 2 * N / (fz * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "with_logits_hbm_frac": round(4 * 2 * N / (fzg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(flops / (fz * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        }
    out["cpu_baseline"] = cpu
    return out




if __name__ == "__main__":
    main()
