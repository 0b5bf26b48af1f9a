#!/usr/bin/env python3
"""Benchmark of the quantize-once convolution hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input, for the ResNet-style
3x3 layer (N=32, Cin=Cout=64, 56x56, stride 1, pad 1, NVFP4): relayout X (NCHW -> channel-batch
first) and W (OIHW -> tap-major), quantize X and W (round-to-nearest) and G_Y (stochastic, a new
seed every step), then the forward, weight-gradient and input-gradient GEMMs. Inputs are resident
in HBM before the timed region starts.

Prints one JSON line. `value` is the step's conv throughput (3 GEMMs' algorithmic flops / step
time); `per_op` holds each op's time, GB/s or TFLOP/s and roofline fraction; `roofline` covers the
op that takes the most time in the step, timed with HIP events around each of its launches
inside the timed steps; `cpu_baseline` times the CPU oracle on a bounded sample (rank 0, N=1).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6    # MI355X dense bf16 MFMA, TFLOP/s (256 CU x 2.4 GHz x 4096)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--op-reps", type=int, default=50, help="reps per op for the breakdown")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-n", type=int, default=32,
                    help="batch elements of the layer the CPU oracle runs on")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path here is single-device; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import microscaling_quantized_convolution_amd as mq
    import workloads

    layer = workloads.config2()[0]
    N, Ci, H, W, Co, Kh, Kw = (layer.N, layer.Cin, layer.H, layer.W, layer.Cout, layer.Kh,
                               layer.Kw)
    Ho, Wo = layer.Ho, layer.Wo
    p = layer.conv_tuple()
    fmt = layer.fmt
    dev = "cuda:0"
    torch.cuda.set_device(0)

    x, w, g = workloads.make_tensors(layer)
    xt = torch.from_numpy(x).to(dev)
    wt = torch.from_numpy(w).to(dev)
    gc = torch.empty(g.size, dtype=torch.float32, device=dev)
    # G_Y arrives channel-batch-first (it is the next layer's input-gradient output)
    mq.mq_relayout_cbf(torch.from_numpy(g).to(dev), gc, N, Co, Ho, Wo, 0)
    xc = torch.empty(x.size, dtype=torch.float32, device=dev)
    wc = torch.empty(w.size, dtype=torch.float32, device=dev)
    amax = torch.empty(4, dtype=torch.int32, device=dev)
    qx = mq.QTensor(H, W, Ci, N, fmt, mq.MQ_ROLE_ACT, dev)
    qw = mq.QTensor(Kh, Kw, Co, Ci, fmt, mq.MQ_ROLE_WEIGHT, dev)
    qg = mq.QTensor(Ho, Wo, Co, N, fmt, mq.MQ_ROLE_GRAD, dev)
    y = torch.empty(Ho * Wo * Co * N, dtype=torch.float32, device=dev)
    gw = torch.empty(Kh * Kw * Co * Ci, dtype=torch.float32, device=dev)
    gx = torch.empty(H * W * Ci * N, dtype=torch.float32, device=dev)
    ws = torch.empty(mq.mq_wgrad_workspace_bytes(p), dtype=torch.uint8, device=dev)
    a0, a1, a2 = amax[0:1], amax[1:2], amax[2:3]

    ops = {
        "relayout_x": lambda s: mq.mq_relayout_cbf(xt, xc, N, Ci, H, W, 0),
        "relayout_w": lambda s: mq.mq_relayout_weight(wt, wc, Co, Ci, Kh, Kw, 0),
        "quantize_x": lambda s: mq.mq_quantize(xc, qx, mq.MQ_RNE, 0, a0),
        "quantize_w": lambda s: mq.mq_quantize(wc, qw, mq.MQ_RNE, 0, a1),
        "quantize_g": lambda s: mq.mq_quantize(gc, qg, mq.MQ_SR, 1 + s, a2),
        "conv_fwd": lambda s: mq.mq_conv_fwd(p, qx, qw, y),
        "conv_wgrad": lambda s: mq.mq_conv_wgrad(p, qg, qx, gw, ws),
        "conv_dgrad": lambda s: mq.mq_conv_dgrad(p, qw, qg, gx),
    }

    flops = layer.gemm_flops()
    sq = lambda o0, o1, r, s_: o0 * o1 * ((r + 3) // 4) * ((s_ + 3) // 4)
    qbytes = lambda shape: sq(*shape) * (8 if fmt == 4 else 12) + sq(*shape)  # codes + scales
    nx, nw, ng = x.size, w.size, g.size
    qx_b, qw_b, qg_b = qbytes((H, W, Ci, N)), qbytes((Kh, Kw, Co, Ci)), qbytes((Ho, Wo, Co, N))
    # algorithmic bytes: quantize = amax read + quantize read + codes/scales written
    alg = {
        "relayout_x": ("hbm", 8 * nx), "relayout_w": ("hbm", 8 * nw),
        "quantize_x": ("hbm", 8 * nx + qx_b), "quantize_w": ("hbm", 8 * nw + qw_b),
        "quantize_g": ("hbm", 8 * ng + qg_b),
        "conv_fwd": ("mfma", flops), "conv_wgrad": ("mfma", flops), "conv_dgrad": ("mfma", flops),
    }
    conv_bytes = {"conv_fwd": qx_b + qw_b + 4 * Ho * Wo * Co * N,
                  "conv_wgrad": qg_b + qx_b + 4 * Kh * Kw * Co * Ci,
                  "conv_dgrad": qw_b + qg_b + 4 * H * W * Ci * N}

    def step(s):
        for f in ops.values():
            f(s)

    # ---- per-op breakdown (each op back to back, events on the launch stream) ----
    for s in range(max(args.warmup, 1)):
        step(s)
    torch.cuda.synchronize()
    per_op = {}
    for name, f in ops.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f(0)
        e0.record()
        for r in range(args.op_reps):
            f(r)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.op_reps
        kind, amount = alg[name]
        if kind == "hbm":
            gbs = amount / (ms * 1e-3) / 1e9
            per_op[name] = {"ms": round(ms, 5), "GB_s": round(gbs, 1),
                            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "alg_bytes": amount}
        else:
            tf = amount / (ms * 1e-3) / 1e12
            gbs = conv_bytes[name] / (ms * 1e-3) / 1e9
            per_op[name] = {"ms": round(ms, 5), "TFLOP_s": round(tf, 1),
                            "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4),
                            "GB_s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                            "alg_flops": amount, "alg_bytes": conv_bytes[name]}
    dominant = max(per_op, key=lambda k: per_op[k]["ms"])

    # ---- timed steps, with events around every launch of the dominant op ----
    torch.cuda.synchronize()
    dom_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for s in range(args.steps):
        for name, f in ops.items():
            if name == dominant:
                dom_ev[s][0].record()
                f(args.warmup + s)
                dom_ev[s][1].record()
            else:
                f(args.warmup + s)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    dom_ms = sum(a.elapsed_time(b) for a, b in dom_ev) / args.steps

    kind, amount = alg[dominant]
    if kind == "hbm":
        ach = amount / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        # the convolution GEMMs at this shape: arithmetic intensity decides the bound
        ai = amount / conv_bytes[dominant]
        ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        if ai >= ridge:
            ach = amount / (dom_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s"}
        else:
            ach = conv_bytes[dominant] / (dom_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = dominant
    roof["ms_per_launch"] = round(dom_ms, 5)

    result = {
        "metric": "quant GB/s (% HBM peak) + conv fwd/wgrad/dgrad TFLOP/s (% bf16 MFMA) per layer",
        "value": round(3 * flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "wall_s_timed": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4-e2m1/e4m3 codes, bf16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded numpy PCG64; X=ReLU(N(0,1)), W Kaiming-normal, G_Y~N(0,1e-3))",
        "config": {"workload": "resnet-3x3-s1p1 N=32 Cin=Cout=64 56x56 NVFP4: relayout + "
                               "quantize x3 + conv fwd/wgrad/dgrad",
                   "N": N, "Cin": Ci, "Cout": Co, "H": H, "W": W, "K": Kh, "stride": 1, "pad": 1,
                   "format": "NVFP4"},
        "per_op": per_op,
        "roofline": roof,
    }

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        result["calib_copy"] = {"bytes_each_way": src.numel() * 4,
                                "ms": round(e0.elapsed_time(e1), 4)}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layer, args.cpu_sample_n)

    print(json.dumps(result), flush=True)


def cpu_baseline(layer, nsample: int):
    """The CPU oracle, as it stands, on the first `nsample` batch elements of the same layer:
    relayout, three quantizations, dequantization and the three explicit-im2col GEMMs in double.
    Reported in the same unit as `value` (conv TFLOP/s of the sample's three GEMMs)."""
    import dataclasses

    import oracle
    import workloads

    sub = dataclasses.replace(layer, N=nsample)
    x, w, g = workloads.make_tensors(layer)
    x, g = x[:nsample].copy(), g[:nsample].copy()
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    p = sub.conv_tuple()
    t = time.perf_counter()
    xc, wc, gc = oracle.nchw_to_cbf(x), oracle.oihw_to_tap_major(w), oracle.nchw_to_cbf(g)
    xh = oracle.quant_dequant(xc, sub.fmt, oracle.RNE)[3]
    wh = oracle.quant_dequant(wc, sub.fmt, oracle.RNE)[3]
    gh = oracle.quant_dequant(gc, sub.fmt, oracle.SR, sub.sr_seed)[3]
    oracle.conv_fwd(p, xh, wh)
    oracle.conv_wgrad(p, gh, xh)
    oracle.conv_dgrad(p, wh, gh)
    sec = time.perf_counter() - t
    tf = 3 * sub.gemm_flops() / sec / 1e12
    return {"value": round(tf, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(sec, 3),
            "sample": f"same layer with N={nsample} of {layer.N} batch elements: relayout, "
                      f"3 quantizations, dequantization, explicit-im2col fwd/wgrad/dgrad in "
                      f"double; flops of the sample's three GEMMs / wall time"}


if __name__ == "__main__":
    main()
