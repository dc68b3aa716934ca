#!/usr/bin/env python3
"""Benchmark of the Q4_0 W4A8 MoE expert matmul on one MI355X.

Headline (the JSON `value`): decode weight bandwidth, in GB/s of expert weight
bytes touched, on the largest single-GPU workload: the 40-layer MoE FFN stack
(hidden 2048, 128 experts per layer with gate/up 512x2048 and down 2048x512,
top-8, ~9 GB of resident Q4_0 weights) decoding a batch of 16 tokens, each
layer's input the previous layer's output plus the residual, fresh router
logits per layer.  A step is one pass of the whole path over the batch: for
every layer the pre-norm and Q8_0 quantisation, routing (softmax, top-8,
renormalisation, counting sort), gate/up + SwiGLU + re-quantisation, down and
the weighted combine into the residual stream, as the library's one-launch
batched stack (moe_q4_decode_stack_batch).  The timed steps are captured into
a HIP graph and replayed, each on its own input rows, so the clock sees GPU
work only.

`roofline` covers the persistent kernel of that call (bstack_kernel; the
call's small routing launch is inside the timed duration), timed live with
HIP events on the launch stream; its `traffic` comes from the rocprofv3
FETCH_SIZE / WRITE_SIZE runs summarised in profiles/.  `achievable` holds the
ceilings measured on the same GPU by the library's three probes.  `extra`
reports the other paths and batch sizes of the stack (each with a roofline
object for its one-launch kernel), the one-layer decode at one token, the
single GEMV, the prefill grouped GEMM (int8 TOPS on the 947-token and the
skewed 4096-token workloads, and its W4A16 variant), and the router
projection.  `cpu_baseline` times the CPU oracle on a bounded sample of every
workload, pinned to one core.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, TOP/s
FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, TFLOP/s (the published figure counts packed fp32, not used here)
CAL_COPY_BYTES = 64 << 20  # counter calibration copy
METRIC = "W4A8 MoE decode weight GB/s (% of HBM peak); prefill grouped-GEMM int8 TOPS"


# HBM traffic per launch of a kernel, from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of this
# bench, each scaled by what the same counter reads for the plain 64 MiB copy that main() runs first (the
# summary and its commands are in profiles/).  A figure is valid only for the sources it was measured on
# (their SHA-256, in order), so a kernel edited since then reports null.
TRAFFIC = {
    # kernel@workload: (source files, sha256 over their bytes, HBM bytes per launch)
    "bstack_kernel@stack40_T16": (
        ["quantized_moe_q4_amd/csrc/bstack.hip", "quantized_moe_q4_amd/csrc/rows.h", "quantized_moe_q4_amd/csrc/topk.h",
         "quantized_moe_q4_amd/csrc/device.h"],
        "44d9087690ebb4f5f529e892017f3b678ea314d8f7925fbe420f9c74db97b5ca",
        6276657276,
    ),
    "bstack_kernel@stack40_T4": (
        ["quantized_moe_q4_amd/csrc/bstack.hip", "quantized_moe_q4_amd/csrc/rows.h", "quantized_moe_q4_amd/csrc/topk.h",
         "quantized_moe_q4_amd/csrc/device.h"],
        "44d9087690ebb4f5f529e892017f3b678ea314d8f7925fbe420f9c74db97b5ca",
        2172137094,
    ),
    "bstack_kernel@stack40_T1": (
        ["quantized_moe_q4_amd/csrc/bstack.hip", "quantized_moe_q4_amd/csrc/rows.h", "quantized_moe_q4_amd/csrc/topk.h",
         "quantized_moe_q4_amd/csrc/device.h"],
        "44d9087690ebb4f5f529e892017f3b678ea314d8f7925fbe420f9c74db97b5ca",
        595685436,
    ),
    "decode_stack_kernel@stack40_T1": (
        ["quantized_moe_q4_amd/csrc/stack.hip", "quantized_moe_q4_amd/csrc/fused.h", "quantized_moe_q4_amd/csrc/rows.h",
         "quantized_moe_q4_amd/csrc/topk.h", "quantized_moe_q4_amd/csrc/device.h"],
        "8ddea21d144549fefa204732e603475c28510b013a1cb2df038d96d391bd4806",
        607802787,
    ),
}


def traffic_of(key: str):
    ent = TRAFFIC.get(key)
    if ent is None:
        return None
    import hashlib
    srcs, digest, nbytes = ent
    h = hashlib.sha256()
    try:
        for src in srcs:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except OSError:
        return None
    return nbytes if h.hexdigest() == digest else None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: enough for >= 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the CPU-oracle samples (all workloads)")
    ap.add_argument("--no-stack1-launch", action="store_true",
                    help="leave out the one-launch batch-1 stack (moe_q4_decode_stack); rocprofv3 aborted at exit in "
                         "every profiled run that held it while it was a cooperative launch")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              "(the expert matmul runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_moe_q4_amd as mq
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def experts_dev(es):
        return mq.Experts(to_dev(es.gate_qs), to_dev(es.up_qs), to_dev(es.down_qs), to_dev(es.gate_d),
                          to_dev(es.up_d), to_dev(es.down_d))

    def clone(ex):
        return mq.Experts(*(t.clone() for t in (ex.gate_qs, ex.up_qs, ex.down_qs, ex.gate_d, ex.up_d, ex.down_d)))

    # A plain device copy of known size (64 MiB read + 64 MiB written), run first: in a rocprofv3 --pmc run
    # of this script, its FETCH_SIZE / WRITE_SIZE calibrate the counters for the kernels measured after it.
    cal_src = torch.ones(CAL_COPY_BYTES // 4, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    for _ in range(3):
        cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    ach = achievable(torch, mq, dev)
    log(f"achievable: HBM read {ach['hbm_read_gbs']:.0f} GB/s, int8 MFMA {ach['int8_mfma_tops']:.0f} TOPS, "
        f"W4A8 step {ach['w4a8_step_tops']:.0f} TOPS")

    # ---------------------------------------------------------------- the 40-layer stack (headline at batch 16)
    w4 = synth.WORKLOADS[4]
    t0 = time.time()
    layers = [experts_dev(synth.expert_set(w4.seed, l, w4.E, w4.H, w4.I)) for l in range(w4.layers)]
    log(f"stack setup: {w4.layers} layers x {layers[0].nbytes / 1e6:.1f} MB, {time.time() - t0:.1f} s")
    stack = stack_lines(args, np, torch, mq, synth, to_dev, layers, ach)
    head = stack["T16"]
    one = head["by_path"]["decode_stack_batch (one launch)"]
    result = {
        "metric": METRIC,
        "value": one["weight_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": one["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": w4.name + "_T16", "tokens": 16, "layers": w4.layers, "hidden": w4.H, "inter": w4.I,
                   "experts": w4.E, "top_k": w4.k, "experts_touched_per_step": head["experts_touched"],
                   "bytes_per_expert": layers[0].expert_bytes(),
                   "step": "moe_q4_decode_stack_batch: 40 x (pre-norm + Q8_0 + route + gate/up + SwiGLU + requant + "
                           "down + combine into the residual), one routing launch and one persistent launch"},
        "pct_of_hbm_peak": round(100.0 * one["weight_gbs"] / HBM_PEAK_GBS, 3),
        "step_ms_by_path": head["step_ms_by_path"],
        "roofline": one["roofline"],
        "achievable": ach,
    }
    extra = {w4.name: stack}
    del layers

    if not args.no_extra:
        extra.update(extras(args, np, torch, mq, synth, to_dev, experts_dev, clone, ach))
    result["extra"] = extra

    # ---------------------------------------------------------------- CPU oracle beside it
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baselines(args, np, synth)

    print(json.dumps(result), flush=True)


def graph_ms(torch, fn, n, reps=1):
    """Average ms of fn() over n calls captured in one HIP graph (best of `reps` replays), timed by events on the
    stream the graph replays on."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        best = ms if best is None else min(best, ms)
    del g
    return best


def roofline_hbm(kernel, workload, ms, nbytes, ach, note):
    """Roofline object of a one-launch HBM-bound kernel: algorithmic bytes per launch over its average duration;
    traffic: HBM bytes per launch from the counter runs (null when none matches the current sources)."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 5), "traffic": traffic_of(f"{kernel}@{workload}"),
            "avg_launch_us": round(ms * 1e3, 3),
            "algorithmic_bytes_per_launch": float(nbytes), "achievable": ach["hbm_read_gbs"],
            "frac_of_achievable": round(gbs / ach["hbm_read_gbs"], 5), "timed": note}


def stack_lines(args, np, torch, mq, synth, to_dev, layers, ach):
    """The 40-layer stack at batch 1, 4 and 16 by every path the library offers; each one-launch path carries a
    roofline object (its kernel, timed per step)."""
    dev = torch.device("cuda:0")
    w4 = synth.WORKLOADS[4]
    eb = layers[0].expert_bytes()
    k = w4.k
    flags = mq.QUANT_RMSNORM | mq.ACCUMULATE
    stl = mq.StackLayers(layers)  # pointers checked and packed once
    out = {}
    for T in synth.STACK_BATCHES:
        n = args.steps if T == 16 else max(20, args.steps // 4)
        h0 = to_dev(synth.normal(w4.seed, synth.x_tid(T), (T, w4.H)))
        lgs = [to_dev(synth.normal(w4.seed, synth.logits_tid(l, T), (T, w4.E))) for l in range(w4.layers)]
        lg_all = torch.stack(lgs)
        hs = h0.unsqueeze(0).repeat(n + 1, 1, 1)  # every step decodes its own rows (no reset inside the step)
        routes = [mq.route(lgs[l], k) for l in range(w4.layers)]
        touched = sum(int((np.diff(r[2].cpu().numpy()) > 0).sum()) for r in routes)
        nbytes = touched * eb
        timed, roof = {}, {}

        # one launch: moe_q4_decode_stack_batch (T <= 16)
        bws = mq.new_stack_batch_workspace(w4.layers, T, w4.E, k, w4.H, w4.I, dev)
        for i in range(args.warmup):
            mq.decode_stack_batch(stl, hs[n], lg_all, k, flags=flags, ws=bws)
        ms = graph_ms(torch, lambda i=n: mq.decode_stack_batch(stl, hs[i], lg_all, k, flags=flags, ws=bws), n, 2)
        if mq.workspace_error(bws):
            raise RuntimeError("decode_stack_batch: a bounded wait gave up (workspace error word set)")
        name = "decode_stack_batch (one launch)"
        timed[name] = ms
        roof[name] = roofline_hbm("bstack_kernel", f"stack40_T{T}", ms, nbytes, ach,
                                  "HIP events around a graph of steps; a step is the routing launch and the "
                                  "persistent launch")
        del bws

        # one launch per stack at T = 1: moe_q4_decode_stack
        if T == 1 and not args.no_stack1_launch:
            sws = mq.new_stack_workspace(w4.H, dev)
            lg1 = lg_all.reshape(w4.layers, w4.E)
            for i in range(args.warmup):
                mq.decode_stack(stl, hs[n].reshape(-1), lg1, k, flags=flags, ws=sws)
            ms = graph_ms(torch, lambda i=n: mq.decode_stack(stl, hs[i].reshape(-1), lg1, k, flags=flags, ws=sws),
                          n, 2)
            if mq.workspace_error(sws):
                raise RuntimeError("decode_stack: a bounded wait gave up (workspace error word set)")
            name = "decode_stack (one launch)"
            timed[name] = ms
            roof[name] = roofline_hbm("decode_stack_kernel", "stack40_T1", ms, nbytes, ach,
                                      "HIP events around a graph of steps; a step is the routing launch and the "
                                      "persistent launch")
            del sws

        # per layer: one fused launch (T <= 8), or quantize_act + route + decode
        ws = mq.new_workspace(T, w4.E, k, w4.H, w4.I, dev)
        xq = torch.empty((T, w4.H), dtype=torch.int8, device=dev)
        xd = torch.empty((T, w4.H // 32), dtype=torch.float32, device=dev)

        def per_layer(i, fused):
            h = hs[i]
            for l in range(w4.layers):
                if fused:
                    mq.decode_fused(layers[l], h, lgs[l], k, flags=flags, out=routes[l], y=h, ws=ws)
                else:
                    mq.quantize_act(h, flags=mq.QUANT_RMSNORM, xq=xq, xd=xd)
                    r = mq.route(lgs[l], k, out=routes[l])
                    mq.decode(layers[l], xq, xd, *r, flags=mq.ACCUMULATE, y=h, ws=ws)

        nl = max(5, n // 8)
        for fused in ([True, False] if T <= mq.MAX_FUSED_TOKENS else [False]):
            name = "decode_fused per layer" if fused else "quantize_act + route + decode per layer"
            timed[name] = graph_ms(torch, lambda i=n, f=fused: per_layer(i, f), nl, 1)
        del ws
        best = min(timed, key=timed.get)
        line = {"experts_touched": touched, "bytes_per_step": nbytes,
                "step_ms_by_path": {p: round(v, 4) for p, v in timed.items()}, "best_path": best, "by_path": {}}
        for p, ms in timed.items():
            gbs = nbytes / (ms * 1e-3) / 1e9
            e = {"step_ms": round(ms, 4), "weight_gbs": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                 "pct_of_achievable_hbm": round(100 * gbs / ach["hbm_read_gbs"], 2)}
            if p in roof:
                e["roofline"] = roof[p]
            line["by_path"][p] = e
        out[f"T{T}"] = line
        log(f"stack T={T}: " + ", ".join(f"{p} {v:.3f} ms" for p, v in timed.items()))
        del hs
    return out


def achievable(torch, mq, dev, read_bytes=1 << 30, reps=5):
    """Ceilings measured on this GPU: a plain streaming read of a buffer larger
    than every cache (best of `reps` calls) and back-to-back int8 MFMA on
    registers, eight workgroups of four waves per CU (best of `reps`)."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    buf = torch.empty(read_bytes, dtype=torch.uint8, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def best_ms(fn):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            t.append(ev[0].elapsed_time(ev[1]))
        return min(t)

    ms_read = best_ms(lambda: mq.probe_read(buf, sink))
    iters, wgs = 256, 8 * cus
    ops = 262144 * iters * 4 * wgs
    ms_mfma = best_ms(lambda: mq.probe_mfma_i8(iters, wgs, sink))
    fsink = torch.zeros(1, dtype=torch.float32, device=dev)
    st_iters, st_wgs = 2048, 2 * cus
    st_ops = 131072 * st_iters * 4 * st_wgs
    ms_step = best_ms(lambda: mq.probe_w4a8_step(st_iters, st_wgs, fsink))
    del buf
    return {"hbm_read_gbs": round(read_bytes / (ms_read * 1e-3) / 1e9, 1),
            "int8_mfma_tops": round(ops / (ms_mfma * 1e-3) / 1e12, 1),
            "w4a8_step_tops": round(st_ops / (ms_step * 1e-3) / 1e12, 1),
            "probe": f"moe_q4_probe_read over {read_bytes >> 20} MiB; moe_q4_probe_mfma_i8 {iters} x 4 MFMA "
                     f"32x32x32 per wave, {wgs} workgroups of 4 waves; moe_q4_probe_w4a8_step {st_iters} steps "
                     f"(2 MFMA + 2 scale FMAs per output) per wave, {st_wgs} workgroups of 4 waves; best of {reps}"}


def extras(args, np, torch, mq, synth, to_dev, experts_dev, clone, ach):
    out = {}
    dev = torch.device("cuda:0")
    reps = 20
    for wi in (2, 3):
        w = synth.WORKLOADS[wi]
        t0 = time.time()
        es = synth.expert_set(w.seed, 0, w.E, w.H, w.I)
        base = experts_dev(es)
        R = max(2, math.ceil((1 << 30) / base.nbytes) + 1)
        copies = [base] + [clone(base) for _ in range(R - 1)]
        x = to_dev(synth.activations(w))
        lg = to_dev(synth.logits(w))
        xq, xd = mq.quantize_act(x)
        ids, wts, off, sp = mq.route(lg, w.k)
        y = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
        ws = torch.empty(mq.workspace_size(w.T, w.E, w.k, w.H, w.I), dtype=torch.uint8, device=dev)
        for i in range(3):
            mq.prefill(copies[i % R], xq, xd, ids, wts, off, sp, y=y, ws=ws)
        torch.cuda.synchronize()
        g_pf, g_st = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_pf):
            for i in range(reps):
                mq.prefill(copies[i % R], xq, xd, ids, wts, off, sp, y=y, ws=ws)
        with torch.cuda.graph(g_st):
            for i in range(reps):
                mq.quantize_act(x, xq=xq, xd=xd)
                mq.route(lg, w.k, out=(ids, wts, off, sp))
                mq.prefill(copies[i % R], xq, xd, ids, wts, off, sp, y=y, ws=ws)
        g_pf.replay()
        g_st.replay()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        g_pf.replay()
        e[1].record()
        g_st.replay()
        e[2].record()
        torch.cuda.synchronize()
        pf_ms = e[0].elapsed_time(e[1]) / reps
        step_ms = e[1].elapsed_time(e[2]) / reps
        # the W4A16 variant of the same layer (fp16 activations, fp16 MFMA) on the same routing
        ws16 = torch.empty(mq.prefill_a16_workspace_size(w.T, w.k, w.H, w.I), dtype=torch.uint8, device=dev)
        for i in range(3):
            mq.prefill_a16(copies[i % R], x, ids, wts, off, sp, y=y, ws=ws16)
        torch.cuda.synchronize()
        g16 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g16):
            for i in range(reps):
                mq.prefill_a16(copies[i % R], x, ids, wts, off, sp, y=y, ws=ws16)
        g16.replay()
        torch.cuda.synchronize()
        e[0].record()
        g16.replay()
        e[1].record()
        torch.cuda.synchronize()
        a16_ms = e[0].elapsed_time(e[1]) / reps
        del g_pf, g_st, g16, ws16
        cnt = np.diff(off.cpu().numpy())
        ops = 2.0 * float(cnt.sum()) * 3 * w.H * w.I
        # what the MFMA tiles execute: every touched expert's rows padded to whole 32-row m-tiles (a row tile
        # runs as many m-tiles as its live rows need)
        padded_ops = 2.0 * float(((cnt + 31) // 32 * 32).sum()) * 3 * w.H * w.I
        touched = int((cnt > 0).sum())
        wbytes = touched * base.expert_bytes()
        tops = ops / (pf_ms * 1e-3) / 1e12
        out[w.name] = {"prefill_call_us": round(pf_ms * 1e3, 2), "step_us": round(step_ms * 1e3, 2),
                       "int8_tops": round(tops, 2), "pct_of_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2),
                       "pct_of_achievable_int8": round(100 * tops / ach["int8_mfma_tops"], 2),
                       "pct_of_w4a8_step_ceiling": round(100 * tops / ach["w4a8_step_tops"], 2),
                       "weight_gbs": round(wbytes / (pf_ms * 1e-3) / 1e9, 1),
                       "pct_of_hbm_peak": round(100 * wbytes / (pf_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                       "algorithmic_ops": ops, "padded_ops": padded_ops,
                       "w4a16": {"prefill_call_us": round(a16_ms * 1e3, 2),
                                 "fp16_tflops": round(ops / (a16_ms * 1e-3) / 1e12, 2),
                                 "pct_of_fp16_peak": round(100 * ops / (a16_ms * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 2),
                                 "weight_gbs": round(wbytes / (a16_ms * 1e-3) / 1e9, 1),
                                 "pct_of_hbm_peak": round(100 * wbytes / (a16_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)},
                       "experts_touched": touched, "max_tokens_per_expert": int(cnt.max()),
                       "weight_copies_rotated": R}
        log(f"prefill {w.name}: {pf_ms * 1e3:.1f} us, {tops:.1f} TOPS; W4A16 {a16_ms * 1e3:.1f} us; "
            f"setup {time.time() - t0:.1f} s")
        del copies, base

    # router projection (the step in front of the routing) at the decode and prefill shapes
    rl = {}
    for T, E in ((1, 128), (947, 128), (4096, 256)):
        H = 2048
        xr = to_dev(synth.normal(3, synth.x_tid(T), (T, H)))
        wrs = [to_dev(synth.router_weights(3, l, E, H)) for l in range(8)]  # 8 layers' weights rotate
        lo = torch.empty((T, E), dtype=torch.float32, device=dev)
        for i in range(3):
            mq.router_logits(xr, wrs[i % 8], flags=mq.QUANT_RMSNORM, out=lo)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        n = 40
        with torch.cuda.graph(g):
            for i in range(n):
                mq.router_logits(xr, wrs[i % 8], flags=mq.QUANT_RMSNORM, out=lo)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / n * 1e3
        flops = 2.0 * T * E * H
        nbytes = 4.0 * (E * H + T * H + T * E)
        rl[f"T{T}_E{E}_H{H}"] = {"us": round(us, 2), "gflops": round(flops / (us * 1e-6) / 1e9, 1),
                                 "pct_of_fp32_vector_peak": round(100 * flops / (us * 1e-6) / 1e12 / FP32_PEAK_TFLOPS, 2),
                                 "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}
        log(f"router logits T={T} E={E}: {us:.2f} us")
        del g, wrs
    out["router_logits_fp32"] = rl

    out[synth.WORKLOADS[1].name] = decode_t1(args, np, torch, mq, synth, to_dev, experts_dev, clone, ach)
    out[synth.WORKLOADS[0].name] = gemv_line(args, np, torch, mq, synth, to_dev, ach)
    return out


def decode_t1(args, np, torch, mq, synth, to_dev, experts_dev, clone, ach):
    """One MoE layer at one token: moe_q4_decode_fused (one launch) and the three calls.  The expert weights
    rotate through R distinct resident copies (>= 1 GiB in total) so that no step finds its weights in the
    256 MB last-level cache."""
    dev = torch.device("cuda:0")
    w1 = synth.WORKLOADS[1]
    t0 = time.time()
    es = synth.expert_set(w1.seed, 0, w1.E, w1.H, w1.I)
    base = experts_dev(es)
    expert_bytes = base.expert_bytes()
    R = args.copies or max(2, math.ceil((1 << 30) / base.nbytes) + 1)
    copies = [base] + [clone(base) for _ in range(R - 1)]
    n = args.steps
    S = args.warmup + n
    X = to_dev(synth.normal(w1.seed, synth.x_tid(1) + (1 << 48), (S, 1, w1.H)))
    Lg = to_dev(synth.normal(w1.seed, synth.logits_tid(0, 1) + (1 << 48), (S, 1, w1.E)))
    k = w1.k
    xq = torch.empty((1, w1.H), dtype=torch.int8, device=dev)
    xd = torch.empty((1, w1.H // 32), dtype=torch.float32, device=dev)
    ids_all = torch.empty((S, 1, k), dtype=torch.int32, device=dev)
    w_all = torch.empty((S, 1, k), dtype=torch.float32, device=dev)
    off = torch.empty(w1.E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(k, dtype=torch.int32, device=dev)
    y = torch.empty((1, w1.H), dtype=torch.float32, device=dev)
    ws = mq.new_workspace(1, w1.E, k, w1.H, w1.I, dev)

    def step(s):  # quantize + route + gate/up + SwiGLU + requant + down + combine in one launch
        mq.decode_fused(copies[s % R], X[s], Lg[s], k, out=(ids_all[s], w_all[s], off, sp), y=y, ws=ws)

    def step3(s):  # the same as three calls (quantize_act, route, decode: four kernels)
        mq.quantize_act(X[s], xq=xq, xd=xd)
        mq.route(Lg[s], k, out=(ids_all[s], w_all[s], off, sp))
        mq.decode(copies[s % R], xq, xd, ids_all[s], w_all[s], off, sp, y=y, ws=ws)

    for s in range(args.warmup):
        step(s)
        step3(s)
    ms3 = graph_ms(torch, lambda i=0: step3(args.warmup + i), n, 1)
    ms = graph_ms(torch, lambda i=0: step(args.warmup + i), n, 2)
    if mq.workspace_error(ws):
        raise RuntimeError("fused decode: a bounded wait gave up (workspace error word set)")
    ids_np = ids_all[args.warmup:].cpu().numpy()
    touched = np.array([len(np.unique(ids_np[i])) for i in range(n)])
    nbytes = float(touched.mean() * expert_bytes)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"decode T=1: {ms * 1e3:.2f} us/step fused ({gbs:.0f} GB/s); three calls {ms3 * 1e3:.2f} us/step; "
        f"setup {time.time() - t0:.1f} s")
    del copies, base
    return {"step_us": round(ms * 1e3, 3), "weight_gbs": round(gbs, 2), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 3),
            "three_call_us_per_step": round(ms3 * 1e3, 3), "weight_copies_rotated": R, "bytes_per_expert": expert_bytes,
            "step": "moe_q4_decode_fused (quantize + route + gate/up + SwiGLU + requant + down + combine)",
            "roofline": roofline_hbm("decode_fused_kernel", "decode_T1", ms, nbytes, ach,
                                     "HIP events around a graph of steps; one launch per step")}


def gemv_line(args, np, torch, mq, synth, to_dev, ach):
    """One Q4_0 matrix (512 x 2048) times one Q8_0 row: a latency line (the matrix is 576 KB, so the call is
    launch- and latency-bound, not bandwidth-bound); 16 matrix copies rotate."""
    dev = torch.device("cuda:0")
    w0 = synth.WORKLOADS[0]
    qs, d = synth.gemv_matrix(w0)
    copies = [(to_dev(qs).clone(), to_dev(d).clone()) for _ in range(16)]
    x = to_dev(synth.normal(w0.seed, synth.x_tid(1), (1, 2048)))
    xq, xd = mq.quantize_act(x)
    y = torch.empty((1, 512), dtype=torch.float32, device=dev)
    n = max(50, args.steps)
    ms = graph_ms(torch, lambda i=0: mq.gemv(copies[i % 16][0], copies[i % 16][1], xq, xd, y=y), n, 2)
    nbytes = qs.nbytes + d.nbytes
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"gemv 512x2048: {ms * 1e3:.2f} us")
    return {"call_us": round(ms * 1e3, 3), "weight_gbs": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 3),
            "bytes_per_call": int(nbytes), "timed": "HIP events around a graph of calls (one launch each)"}


def host_cores():
    """(physical cores, logical CPUs) of the host, from /proc/cpuinfo's (physical id, core id) pairs."""
    logical = os.cpu_count() or 1
    pairs, phys = set(), None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("physical id"):
                    phys = line.split(":", 1)[1].strip()
                elif line.startswith("core id"):
                    pairs.add((phys, line.split(":", 1)[1].strip()))
    except OSError:
        pass
    return (len(pairs) or logical), logical


def cpu_baselines(args, np, synth):
    """The CPU oracle, as it stands, on a bounded sample of every workload, one host thread pinned to one core
    (os.sched_setaffinity on this process for the duration; restored afterwards).  The headline figure is the
    stack at batch 16 in the headline's unit."""
    import oracle

    budget = args.cpu_seconds / 5.0  # seconds per workload
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[-1]
    os.sched_setaffinity(0, {core})
    per = {}
    try:
        # workload 0: the single GEMV
        w0 = synth.WORKLOADS[0]
        qs, d = synth.gemv_matrix(w0)
        x = synth.normal(w0.seed, synth.x_tid(1), (1, 2048))
        xq, xd = oracle.q8_quantize(x)
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget:
            oracle.gemv(qs, d, xq, xd)
            n += 1
        dt = time.perf_counter() - t0
        per[w0.name] = {"value": round((qs.nbytes + d.nbytes) * n / dt / 1e9, 4), "unit": "GB/s",
                        "us_per_call": round(dt / n * 1e6, 2), "sample": f"{n} calls, {dt:.1f} s"}
        # workload 1: one layer at one token (quantize + route + layer)
        w1 = synth.WORKLOADS[1]
        es = synth.expert_set(w1.seed, 0, w1.E, w1.H, w1.I)
        n, nbytes, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 < budget:
            x = synth.normal(w1.seed, synth.x_tid(1) + (1 << 48), (1, w1.H), start=n * w1.H)
            lg = synth.normal(w1.seed, synth.logits_tid(0, 1) + (1 << 48), (1, w1.E), start=n * w1.E)
            xq, xd = oracle.q8_quantize(x)
            ids, w, off, sp = oracle.route(lg, w1.k)
            oracle.moe_layer(es, xq, xd, ids, w)
            nbytes += len(np.unique(ids)) * expert_bytes_of(es)
            n += 1
        dt = time.perf_counter() - t0
        per[w1.name] = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "ms_per_step": round(dt / n * 1e3, 2),
                        "sample": f"{n} decode steps (quantize + route + layer, one token each), {dt:.1f} s"}
        del es
        # workloads 2 and 3: the prefill layer on a sample of its tokens (full routing, layer on the sample)
        for wi in (2, 3):
            w = synth.WORKLOADS[wi]
            es = synth.expert_set(w.seed, 0, w.E, w.H, w.I)
            x = synth.activations(w)
            lg = synth.logits(w)
            xq, xd = oracle.q8_quantize(x)
            ids, wt, off, sp = oracle.route(lg, w.k)
            n, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < budget and n < w.T:
                toks = np.arange(n, min(n + 8, w.T), dtype=np.int32)
                oracle.moe_layer(es, xq, xd, ids, wt, tokens=toks)
                n += len(toks)
            dt = time.perf_counter() - t0
            ops = 2.0 * n * w.k * 3 * w.H * w.I
            per[w.name] = {"value": round(ops / dt / 1e12, 6), "unit": "int8 TOPS", "ms_per_token": round(dt / n * 1e3, 2),
                           "sample": f"{n} of {w.T} tokens through the layer (routing of all), {dt:.1f} s"}
            del es, x
        # workload 4: the stack at batch 16, layer after layer (quantize with the pre-norm + route + layer + residual)
        w4 = synth.WORKLOADS[4]
        T = 16
        h = synth.normal(w4.seed, synth.x_tid(T), (T, w4.H))
        n, nbytes, dt = 0, 0, 0.0
        while dt < budget and n < w4.layers:
            es = synth.expert_set(w4.seed, n, w4.E, w4.H, w4.I)  # generating the weights is not timed
            lg = synth.normal(w4.seed, synth.logits_tid(n, T), (T, w4.E))
            t1 = time.perf_counter()
            xq, xd = oracle.q8_quantize(h, oracle.FLAG_RMSNORM)
            ids, wt, off, sp = oracle.route(lg, w4.k)
            h = h + oracle.moe_layer(es, xq, xd, ids, wt)
            dt += time.perf_counter() - t1
            nbytes += len(np.unique(ids)) * expert_bytes_of(es)
            n += 1
        per[w4.name + "_T16"] = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s",
                                 "ms_per_layer": round(dt / n * 1e3, 1),
                                 "sample": f"{n} of {w4.layers} layers at batch 16, {dt:.1f} s"}
    finally:
        os.sched_setaffinity(0, set(allowed))
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    phys, logical = host_cores()
    head = per[synth.WORKLOADS[4].name + "_T16"]
    return {"value": head["value"], "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": head["sample"] + " (the headline workload)", "pinned_cpu": core, "host_cpu": cpu,
            "host_physical_cores": phys, "host_logical_cpus": logical, "per_workload": per}


def expert_bytes_of(es) -> int:
    """Bytes of one expert's Q4_0 gate, up and down matrices (nibbles and fp16 scales)."""
    return int((es.gate_qs[0].nbytes + es.up_qs[0].nbytes + es.down_qs[0].nbytes + es.gate_d[0].nbytes
                + es.up_d[0].nbytes + es.down_d[0].nbytes))


if __name__ == "__main__":
    main()
