#!/usr/bin/env python3
"""Benchmark of the quantize-once convolution hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input, for the ResNet-style
3x3 layer (N=32, Cin=Cout=64, 56x56, stride 1, pad 1, NVFP4): quantize X from NCHW and W from
OIHW into their squares together, as the forward pass does (round-to-nearest; one batched call:
an amax launch and a quantizing launch over both), quantize G_Y (stochastic, a new seed every
step), then the forward GEMM and the two gradient GEMMs (weight and input gradient in one call,
mq_conv_backward). Inputs are resident in HBM before the timed region starts.

The timed steps call the C ABI back to back on one stream (arguments marshalled once, so the
GPU, not the host, sets the pace), with HIP events on that stream around the op that takes the
longest (`roofline`) in every `--event-every`-th step. `--graph` replays one HIP graph per step instead (split
around that op so the events stay outside the graphs). `per_op` times each op alone as a graph
of back-to-back launches. `cpu_baseline` times the CPU oracle on a bounded sample (rank 0, N=1).

`roofline.traffic` is the HBM traffic of that op per launch from rocprofv3 FETCH_SIZE and
WRITE_SIZE counters (profiles/c2_pmc_traffic.txt), scaled by what the same counters read for a
plain copy of known size; it is null when the kernel sources differ from the ones counted.
`--summarize-pmc FETCH_DB WRITE_DB` writes that file's body from two rocprofv3 --pmc databases.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2516.6    # MI355X dense fp16/bf16 MFMA, TFLOP/s (256 CU x 2.4 GHz x 4096)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "c2_pmc_traffic.txt")
CALIB_ELEMS = 1 << 26        # plain copy for counter calibration: 256 MiB read + 256 MiB written

# which kernels make up each op (rocprofv3 kernel names start with these)
OP_KERNELS = {
    "quantize_xw": ["mq::amax_batch_kernel", "void mq::quantize_batch_kernel"],
    "quantize_x": ["mq::amax_kernel", "void mq::quantize_nchw_kernel"],
    "quantize_w": ["void mq::quantize_weight_small_kernel", "mq::amax_kernel",
                   "void mq::quantize_kernel"],
    "quantize_g": ["mq::amax_kernel", "void mq::quantize_kernel"],
    "conv_fwd": ["void mq::conv_spatial_kernel<4, false"],
    "conv_backward": ["void mq::conv_wgrad_kernel", "void mq::conv_spatial_kernel<4, true",
                      "mq::wgrad_sum_kernel"],
    "conv_wgrad": ["void mq::conv_wgrad_kernel", "mq::wgrad_sum_kernel"],
    "conv_dgrad": ["void mq::conv_spatial_kernel<4, true"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--op-reps", type=int, default=20, help="launches per op for the breakdown")
    ap.add_argument("--event-every", type=int, default=8,
                    help="bracket the dominant op with HIP events in every n-th timed step")
    ap.add_argument("--eager", action="store_true",
                    help="time plain launches (the default; kept for the profiling commands)")
    ap.add_argument("--graph", action="store_true", help="time HIP graph replays of the steps")
    ap.add_argument("--roofline-op", default=None,
                    help="op the roofline covers (default: the one with the longest per-op time)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parts", action="store_true",
                    help="leave out of per_op the timing of conv_wgrad and conv_dgrad as calls of "
                         "their own (they are not part of the step; profiling runs leave them out "
                         "so that every kernel in the trace belongs to one op)")
    ap.add_argument("--cpu-sample-n", type=int, default=32,
                    help="batch elements of the layer the CPU oracle runs on")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (HBM counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="print the traffic summary from two rocprofv3 --pmc databases")
    ap.add_argument("--config", default=None, choices=["c1", "c2", "c3", "c4", "c5"],
                    help="time the hot path of every layer of a workload (one step = every "
                         "layer once) instead of the single 3x3 layer")
    ap.add_argument("--network", default=None, choices=["resnet18"],
                    help="time a full training step of ResNet-18 (19 body convolutions on the "
                         "library, the rest in PyTorch fp32)")
    ap.add_argument("--batch", type=int, default=128, help="batch size of --network")
    ap.add_argument("--inference", action="store_true",
                    help="with --config: the inference path only (quantize X from NCHW, "
                         "conv fwd; the weights are quantized once before timing)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "microscaling_quantized_convolution_amd",
                                           "csrc", "*"))):
        if p.endswith((".hip", ".hpp", ".cpp")):
            h.update(os.path.basename(p).encode())
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(op: str):
    """HBM bytes per launch of `op` from the committed counter summary, or None if there is none
    or it was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#", "|")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_source_hash():
        return None
    v = kv.get(f"traffic_bytes_per_launch.{op}")
    return None if v is None else int(float(v))


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path here is single-device; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.network:
        run_network(args)
        return
    if args.config:
        run_config(args)
        return

    import torch

    import microscaling_quantized_convolution_amd as mq
    from microscaling_quantized_convolution_amd.step import LayerStep
    import workloads

    layer = workloads.config2()[0]
    N, Ci, H, W, Co, Kh, Kw = (layer.N, layer.Cin, layer.H, layer.W, layer.Cout, layer.Kh,
                               layer.Kw)
    Ho, Wo = layer.Ho, layer.Wo
    fmt = layer.fmt
    dev = "cuda:0"
    torch.cuda.set_device(0)

    x, w, g = workloads.make_tensors(layer)
    gc = torch.empty(g.size, dtype=torch.float32, device=dev)
    # G_Y arrives channel-batch-first (it is the next layer's input-gradient output)
    mq.mq_relayout_cbf(torch.from_numpy(g).to(dev), gc, N, Co, Ho, Wo, 0)
    st = LayerStep(layer.conv_tuple(), fmt, torch.from_numpy(x).to(dev),
                   torch.from_numpy(w).to(dev), gc, sr_seed_base=layer.sr_seed)
    ops = st.ops
    stream = torch.cuda.Stream()

    flops = layer.gemm_flops()
    sq = lambda o0, o1, r, s_: o0 * o1 * ((r + 3) // 4) * ((s_ + 3) // 4)
    qbytes = lambda shape: sq(*shape) * (8 if fmt == 4 else 12) + sq(*shape)  # codes + scales
    nx, nw, ng = x.size, w.size, g.size
    qx_b, qw_b, qg_b = qbytes((H, W, Ci, N)), qbytes((Kh, Kw, Co, Ci)), qbytes((Ho, Wo, Co, N))
    # algorithmic bytes: every quantization = amax read + quantize read + codes/scales
    alg = {
        "quantize_xw": ("hbm", 8 * nx + qx_b + 8 * nw + qw_b),
        "quantize_g": ("hbm", 8 * ng + qg_b),
        "conv_fwd": ("gemm", flops), "conv_wgrad": ("gemm", flops), "conv_dgrad": ("gemm", flops),
        "conv_backward": ("gemm", 2 * flops),
    }
    # conv: quantized operands read once + fp32 result written once
    conv_bytes = {"conv_fwd": qx_b + qw_b + 4 * Ho * Wo * Co * N,
                  "conv_wgrad": qg_b + qx_b + 4 * Kh * Kw * Co * Ci,
                  "conv_dgrad": qw_b + qg_b + 4 * H * W * Ci * N}
    conv_bytes["conv_backward"] = conv_bytes["conv_wgrad"] + conv_bytes["conv_dgrad"]
    ridge = MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)

    def capture(fns):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            for f in fns:
                f()
        return gr

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ---- warm-up (eager) ----
    with torch.cuda.stream(stream):
        for s in range(max(args.warmup, 1)):
            st.run(s)
    torch.cuda.synchronize()

    # ---- per-op breakdown: each op alone, `op_reps` launches back to back (the step's ops, and
    # unless --no-parts the two gradients as calls of their own: the per-GEMM rates) ----
    per_op = {}
    for name, f in list(ops.items()) + ([] if args.no_parts else list(st.parts.items())):
        with torch.cuda.stream(stream):
            gr = capture([lambda r=r: f(r) for r in range(args.op_reps)])
            gr.replay()
            e0, e1 = ev(), ev()
            e0.record(stream)
            gr.replay()
            e1.record(stream)
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
                            "frac_mfma": round(tf / MFMA_PEAK_TFLOPS, 4),
                            "GB_s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                            "alg_flops": amount, "alg_bytes": conv_bytes[name],
                            "bound": "mfma" if amount / conv_bytes[name] >= ridge else "hbm"}
    dominant = args.roofline_op or max(ops, key=lambda k: per_op[k]["ms"])
    if dominant not in ops:
        sys.exit(f"--roofline-op {dominant}: not an op of the step ({', '.join(ops)})")
    names = list(ops)
    di = names.index(dominant)

    # ---- timed steps: pre-ops, the dominant op between two events, post-ops ----
    total = args.warmup + args.steps
    calls = st.direct_calls(stream)
    if not args.graph:
        plan = None
    else:
        plan = []
        for s in range(total):
            fs = [lambda f=ops[n], s=s: f(s) for n in names]
            plan.append((capture(fs[:di]) if di > 0 else None, capture([fs[di]]),
                         capture(fs[di + 1:]) if di + 1 < len(fs) else None))
        torch.cuda.synchronize()

    def run_step(s, e_in=None, e_out=None):
        if plan is None:
            for n in names[:di]:
                calls[n](s)
            if e_in is not None:
                e_in.record(stream)
            calls[dominant](s)
            if e_out is not None:
                e_out.record(stream)
            for n in names[di + 1:]:
                calls[n](s)
        else:
            pre, dom, post = plan[s]
            if pre is not None:
                pre.replay()
            if e_in is not None:
                e_in.record(stream)
            dom.replay()
            if e_out is not None:
                e_out.record(stream)
            if post is not None:
                post.replay()

    with torch.cuda.stream(stream):
        for s in range(args.warmup):
            run_step(s)
    torch.cuda.synchronize()
    # events around the dominant op in every args.event_every-th timed step: each pair of event
    # records adds about 5 us to the step it sits in (measured), so they sample the op's launches
    # instead of instrumenting all of them
    dom_ev = [(ev(), ev()) if s_ % args.event_every == 0 else (None, None)
              for s_ in range(args.steps)]
    t0, t1 = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    with torch.cuda.stream(stream):
        t0.record(stream)
        for s in range(args.steps):
            run_step(args.warmup + s, *dom_ev[s])
        t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    sampled = [(a, b) for a, b in dom_ev if a is not None]
    dom_ms = sum(a.elapsed_time(b) for a, b in sampled) / len(sampled)

    kind, amount = alg[dominant]
    if kind == "hbm":
        ach = amount / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    elif amount / conv_bytes[dominant] >= ridge:
        ach = amount / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        ach = conv_bytes[dominant] / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = read_traffic(dominant)
    roof["op"] = dominant
    roof["kernels"] = OP_KERNELS[dominant]
    roof["ms_per_launch"] = round(dom_ms, 5)
    roof["launches_timed"] = len(sampled)
    roof["alg_per_launch"] = amount if roof["bound"] != "hbm" or kind == "hbm" \
        else conv_bytes[dominant]

    result = {
        "metric": "quant GB/s (% HBM peak) + conv fwd/wgrad/dgrad TFLOP/s (% bf16 MFMA) per layer",
        "value": round(3 * flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "wall_s_timed": round(wall, 4),
        "timing": "HIP graph replay per step" if args.graph else "back-to-back launches",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded numpy PCG64; X=ReLU(N(0,1)), W Kaiming-normal, G_Y~N(0,1e-3))",
        "config": {"workload": "resnet-3x3-s1p1 N=32 Cin=Cout=64 56x56 NVFP4: quantize X "
                               "(from NCHW) and W (from OIHW) in one batched call (RNE), G_Y "
                               "(SR), conv fwd, conv backward (wgrad + dgrad in one call)",
                   "N": N, "Cin": Ci, "Cout": Co, "H": H, "W": W, "K": Kh, "stride": 1, "pad": 1,
                   "format": "NVFP4 (E2M1 codes, E4M3 4x4-square scales, fp32 tensor scale)",
                   "mfma": "fp16 operands decoded exactly, fp32 accumulate"},
        "per_op": per_op,
        "roofline": roof,
    }

    if args.calib_copy:
        import torch as _t
        src = _t.full((CALIB_ELEMS,), 1.0, dtype=_t.float32, device=dev)
        dst = _t.empty_like(src)
        _t.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        _t.neg(src, out=dst)
        e1.record()
        _t.cuda.synchronize()
        result["calib_copy"] = {"bytes_read": CALIB_ELEMS * 4, "bytes_written": CALIB_ELEMS * 4,
                                "ms": round(e0.elapsed_time(e1), 4)}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layer, args.cpu_sample_n)

    print(json.dumps(result), flush=True)


def _time_graph(fns, reps: int, stream) -> float:
    """Milliseconds per pass of `fns` (called in order), from one HIP graph of `reps` passes."""
    import torch
    with torch.cuda.stream(stream):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            for r in range(reps):
                for f in fns:
                    f(r)
        gr.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gr.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_config(args):
    """Every layer of a workload through the hot path: one step = each layer's three
    quantizations and three GEMMs once (layers that repeat a shape are timed once and counted
    with their multiplicity). Per layer and op: time, rate and fraction of the bound."""
    import collections

    import numpy as np
    import torch

    from microscaling_quantized_convolution_amd.step import LayerStep
    import workloads

    torch.cuda.set_device(0)
    dev = "cuda:0"
    layers = workloads.CONFIGS[args.config]()
    groups = collections.OrderedDict()
    for l in layers:
        groups.setdefault(l.conv_tuple() + (l.fmt,), []).append(l)
    stream = torch.cuda.Stream()
    ridge = MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    per_layer, step_ms, flops_total = [], 0.0, 0
    for key, ls in groups.items():
        l = ls[0]
        x, w, g = workloads.make_tensors(l)
        gc = torch.empty(g.size, dtype=torch.float32, device=dev)
        import microscaling_quantized_convolution_amd as mq
        mq.mq_relayout_cbf(torch.from_numpy(g).to(dev), gc, l.N, l.Cout, l.Ho, l.Wo, 0)
        st = LayerStep(l.conv_tuple(), l.fmt, torch.from_numpy(x).to(dev),
                       torch.from_numpy(w).to(dev), gc, sr_seed_base=l.sr_seed)
        del x, w, g
        calls = st.direct_calls(stream)
        for s_ in range(max(args.warmup, 1)):
            for f in calls.values():
                f(s_)
        torch.cuda.synchronize()
        if args.inference:  # W stays quantized from the warm-up: activations only
            calls = st.inference_calls(stream)
        eb = 0.5625 if l.fmt == 4 else 0.8125
        nx, nw, ng = l.N * l.Cin * l.H * l.W, l.Cout * l.Cin * l.Kh * l.Kw, l.N * l.Cout * l.Ho * l.Wo
        fl = l.gemm_flops()
        byt = {"quantize_x": 8 * nx + eb * nx, "quantize_xw": 8 * (nx + nw) + eb * (nx + nw),
               "quantize_w": 4 * nw + eb * nw, "quantize_g": 8 * ng + eb * ng,
               "conv_fwd": eb * (nx + nw) + 4 * ng, "conv_wgrad": eb * (nx + ng) + 4 * nw,
               "conv_dgrad": eb * (nw + ng) + 4 * nx}
        byt["conv_backward"] = byt["conv_wgrad"] + byt["conv_dgrad"]
        ops = {}
        for name, f in calls.items():
            ms = _time_graph([f], args.op_reps, stream)
            gbs = byt[name] / (ms * 1e-3) / 1e9
            if name.startswith("conv"):
                fo = 2 * fl if name == "conv_backward" else fl
                tf = fo / (ms * 1e-3) / 1e12
                mfma = fo / byt[name] >= ridge
                ops[name] = {"ms": round(ms, 5), "TFLOP_s": round(tf, 1), "GB_s": round(gbs, 1),
                             "bound": "mfma" if mfma else "hbm",
                             "frac": round(tf / MFMA_PEAK_TFLOPS if mfma else
                                           gbs / HBM_PEAK_GBS, 4)}
            else:
                ops[name] = {"ms": round(ms, 5), "GB_s": round(gbs, 1),
                             "frac": round(gbs / HBM_PEAK_GBS, 4)}
        fns = list(calls.values())
        ms_layer = _time_graph(fns, max(2, args.op_reps // 4), stream)
        step_ms += ms_layer * len(ls)
        flops_total += (1 if args.inference else 3) * fl * len(ls)
        per_layer.append({"layers": [x_.name for x_ in ls], "shape": {
            "N": l.N, "Cin": l.Cin, "Cout": l.Cout, "H": l.H, "W": l.W, "K": l.Kh,
            "stride": l.stride, "pad": l.pad, "format": f"NVFP{l.fmt}"},
            "ms_layer_step": round(ms_layer, 5), "per_op": ops})
        del st, calls, gc
        torch.cuda.empty_cache()
    result = {
        "metric": "quant GB/s (% HBM peak) + conv fwd/wgrad/dgrad TFLOP/s (% bf16 MFMA) per layer",
        "value": round(flops_total / (step_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "ms_per_step": round(step_ms, 5),
        "timing": "per layer: one HIP graph of back-to-back layer steps; the step is the sum "
                  "over the workload's layers with their multiplicity",
        "higher_is_better": True,
        "dtype": "fp16",
        "data": "synthetic (seeded numpy PCG64, the workload's value distributions)",
        "config": {"workload": (f"{args.config} inference: {len(layers)} layers, quantize X "
                                f"(from NCHW), conv fwd each (weights quantized once)")
                   if args.inference else
                   (f"{args.config}: {len(layers)} layers, quantize X and W (one batched call), "
                    f"G_Y, conv fwd and backward (wgrad + dgrad in one call) each")},
        "per_layer": per_layer,
    }
    print(json.dumps(result), flush=True)


def run_network(args):
    """One ResNet-18 training step (forward, cross-entropy on random labels, backward, SGD with
    momentum) at 224x224 on synthetic uniform images: the 19 body convolutions go through the
    library (each of X, W, G_Y quantized once per step), the stem, batch norms, activations,
    residual adds, pooling and classifier stay fp32 PyTorch."""
    import torch

    from microscaling_quantized_convolution_amd.nn import ResNet18MQ
    import workloads

    torch.cuda.set_device(0)
    torch.manual_seed(0)
    B = args.batch
    model = ResNet18MQ(num_classes=1000).cuda()
    opt = torch.optim.SGD(model.parameters(), lr=0.01, momentum=0.9)
    x = torch.rand(B, 3, 224, 224, device="cuda")
    labels = torch.randint(0, 1000, (B,), device="cuda")

    def step():
        opt.zero_grad(set_to_none=True)
        loss = torch.nn.functional.cross_entropy(model(x), labels)
        loss.backward()
        opt.step()
        return loss

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        loss = step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    body_flops = 3 * sum(l.gemm_flops() for l in workloads.config5()) * B // 128
    result = {
        "metric": "ResNet-18 training step with NVFP4 body convolutions",
        "value": round(B / (ms * 1e-3), 1),
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "dtype": "fp16 MFMA on quantized body convs; fp32 elsewhere",
        "data": "synthetic (uniform [0,1) images, random labels)",
        "config": {"workload": f"resnet18 N={B} 224x224: 19 body convs on the library, "
                               f"stem/BN/ReLU/pool/FC fp32 PyTorch, SGD momentum"},
        "body_gemm_flops_per_step": body_flops,
        "body_gemm_tflops_over_step": round(body_flops / (ms * 1e-3) / 1e12, 2),
        "final_loss": round(float(loss.detach()), 4),
    }
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
    # repeat the pass until about 10 s of CPU work (at most 8 passes), report the mean
    secs = []
    while (not secs or sum(secs) < 10.0) and len(secs) < 8:
        t = time.perf_counter()
        xc, wc, gc = oracle.nchw_to_cbf(x), oracle.oihw_to_tap_major(w), oracle.nchw_to_cbf(g)
        xh = oracle.quant_dequant(xc, sub.fmt, oracle.RNE)[3]
        wh = oracle.quant_dequant(wc, sub.fmt, oracle.RNE)[3]
        gh = oracle.quant_dequant(gc, sub.fmt, oracle.SR, sub.sr_seed)[3]
        oracle.conv_fwd(p, xh, wh)
        oracle.conv_wgrad(p, gh, xh)
        oracle.conv_dgrad(p, wh, gh)
        secs.append(time.perf_counter() - t)
    sec = sum(secs) / len(secs)
    tf = 3 * sub.gemm_flops() / sec / 1e12
    return {"value": round(tf, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds_per_pass": round(sec, 3), "passes": len(secs),
            "sample": f"same layer with N={nsample} of {layer.N} batch elements: relayout, "
                      f"3 quantizations, dequantization, explicit-im2col fwd/wgrad/dgrad in "
                      f"double, repeated to about 10 s; flops of the sample's three GEMMs / "
                      f"mean wall time per pass"}


def _short(name: str) -> str:
    """Kernel name without its parameter list."""
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                return name[:i]
    return name


def _pmc_per_kernel(db: str, counter: str):
    """Mean per dispatch of `counter` (summed over its instances) per kernel name."""
    import collections
    import sqlite3
    con = sqlite3.connect(db)
    cols = [r[1] for r in con.execute("pragma table_info(counters_collection)")]
    ki, ci, vi, di = (cols.index(c) for c in ("kernel_name", "counter_name", "value",
                                              "dispatch_id"))
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for row in con.execute("select * from counters_collection"):
        if row[ci] == counter:
            per[_short(row[ki])][row[di]] += row[vi]
    return {k: (sum(d.values()) / len(d), len(d)) for k, d in per.items()}


def summarize_pmc(fetch_db: str, write_db: str):
    """Traffic summary (key: value lines) from a FETCH_SIZE run and a WRITE_SIZE run of
    `bench.py --eager --calib-copy`; the counters are KiB per dispatch."""
    fetch = _pmc_per_kernel(fetch_db, "FETCH_SIZE")
    write = _pmc_per_kernel(write_db, "WRITE_SIZE")
    copy = [k for k in fetch if "neg_kernel" in k]
    if not copy:
        raise SystemExit("no calibration copy kernel in the FETCH_SIZE database")
    ck = copy[0]
    f_cal = fetch[ck][0] * 1024 / (CALIB_ELEMS * 4)
    w_cal = write[ck][0] * 1024 / (CALIB_ELEMS * 4) if ck in write else 1.0
    print(f"kernel_sources_sha256: {kernel_source_hash()}")
    print(f"calibration_kernel: {ck[:90]}")
    print(f"calibration_fetch_factor: {f_cal:.4f}")
    print(f"calibration_write_factor: {w_cal:.4f}")
    print("#")
    print("# kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (calibrated)")
    per_kernel = {}
    for k in sorted(fetch):
        fk = fetch[k][0]
        wk = write.get(k, (0.0, 0))[0]
        b = fk * 1024 / f_cal + wk * 1024 / w_cal
        per_kernel[k] = b
        print(f"| {k[:90]} | {fetch[k][1]} | {fk:.1f} | {wk:.1f} | {b:.0f} |")
    # per op (quantize_x/w/g share kernel names with different sizes, so only
    # the convolutions, whose kernels are distinct, get a per-op figure)
    for op in ("conv_fwd", "conv_backward", "conv_wgrad", "conv_dgrad"):
        tot = sum(b for k, b in per_kernel.items()
                  if any(k.replace("(anonymous namespace)::", "").startswith(p)
                         for p in OP_KERNELS[op]))
        print(f"traffic_bytes_per_launch.{op}: {tot:.0f}")


if __name__ == "__main__":
    main()
