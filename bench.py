#!/usr/bin/env python3
"""Benchmark of the quantize-once convolution hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input for every layer of a
workload. The default workload is the ResNet-18 convolution body (19 convolutions, N = 128,
224x224 input, NVFP4; the stem convolution and the classifier stay fp32 and are not part of the
path). For every layer, in order:
  quantize_xw    X from NCHW and W from OIHW into their squares together (round to nearest; one
                 batched call: an amax launch and a quantizing launch over both)
  quantize_g     G_Y (stochastic rounding; seed 1 + layers*step + layer index)
  conv_fwd       Y = W.X'
  conv_backward  G_W = G_Y.X'^T and G_X = W^T.G_Y in one call
Every layer has its own buffers and all inputs are resident in HBM before the timed region
starts. G_Y arrives channel-batch-first (it is the next layer's input-gradient output).

The timed steps call the C ABI back to back on one stream (arguments marshalled once, so the
GPU, not the host, sets the pace). HIP events on that stream bracket every launch of the step's
dominant kernel in every `--event-every`-th step: of the step's calls that launch exactly one
kernel (the forward convolution; the quantizations launch an amax and a quantizing kernel, the
backward call a weight-gradient and an input-gradient kernel), the layer shape with the most time
per step. `roofline` is that kernel's algorithmic work per launch over its mean bracketed
duration.
`per_layer` times each op of each distinct layer shape alone (a HIP graph of back-to-back
launches), also the two gradients as calls of their own. `quantize_cold` times the largest
layer's quantizations with the MALL flushed before each launch. `cpu_baseline` times the CPU
oracle on a bounded sample of the first layer.

`roofline.traffic` is the HBM traffic of the dominant op per launch from rocprofv3 FETCH_SIZE and
WRITE_SIZE counters (profiles/<workload>_<layer>_pmc_traffic.txt), scaled by what the same
counters read for a plain copy of known size; null when the kernel sources differ from the ones
counted. `--summarize-pmc FETCH_DB WRITE_DB` writes that file's body from two rocprofv3 --pmc
databases; `--summarize-trace DB` and `--summarize-mfma DB` turn a kernel-trace database and an
MFMA-counter database into the summaries kept under profiles/.

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
CALIB_ELEMS = 1 << 26        # plain copy for counter calibration: 256 MiB read + 256 MiB written
FLUSH_BYTES = 512 << 20      # read before each cold launch (the MALL holds 256 MB)
METRIC = "quant GB/s (% HBM peak) + conv fwd/wgrad/dgrad TFLOP/s (% bf16 MFMA) per layer"

# which kernels make up each op (rocprofv3 kernel names start with these)
OP_KERNELS = {
    "quantize_xw": ["mq::amax_batch_kernel", "void mq::quantize_batch_kernel"],
    "quantize_x": ["mq::amax_kernel", "void mq::quantize_nchw_kernel"],
    "quantize_g": ["mq::amax_kernel", "void mq::quantize_kernel"],
    "conv_fwd": ["void mq::conv_spatial_kernel<4, false", "void mq::conv_spatial_kernel<6, false",
                 "void mq::conv_gemm_kernel"],
    "conv_backward": ["void mq::conv_wgrad_kernel", "void mq::conv_spatial_kernel<4, true",
                      "void mq::conv_spatial_kernel<6, true", "mq::wgrad_sum_kernel",
                      "void mq::conv_gemm_kernel", "mq::wgrad_reduce_kernel"],
    "conv_wgrad": ["void mq::conv_wgrad_kernel", "mq::wgrad_sum_kernel",
                   "void mq::conv_gemm_kernel", "mq::wgrad_reduce_kernel"],
    "conv_dgrad": ["void mq::conv_spatial_kernel<4, true", "void mq::conv_spatial_kernel<6, true",
                   "void mq::conv_gemm_kernel"],
    "quantize_g_ready": ["void mq::quantize_kernel"],
}
OP_KERNELS["conv_fwd_amax"] = OP_KERNELS["conv_fwd"] + ["mq::amax_kernel"]
OP_KERNELS["conv_backward_amax"] = OP_KERNELS["conv_backward"] + ["mq::amax_kernel"]
STEP_OPS = ["quantize_xw", "quantize_g", "conv_fwd", "conv_backward"]
INFERENCE_OPS = ["quantize_x", "conv_fwd"]
# calls of the step that launch exactly one kernel (the spatial or generic convolution kernel)
ONE_KERNEL_OPS = ("conv_fwd",)
PARTS = ["conv_wgrad", "conv_dgrad", "conv_fwd_amax", "conv_backward_amax", "quantize_g_ready"]


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c5", choices=["c1", "c2", "c3", "c4", "c5"],
                    help="c5: ResNet-18 body at N=128 (default); c2: ResNet 3x3 layer at N=32; "
                         "c3: strided 3x3 at N=64; c4: YOLO-like NVFP6 stack at N=16; c1: tiny")
    ap.add_argument("--layers", default=None,
                    help="comma-separated layer names: time only these layers of the workload "
                         "(per-shape profiles)")
    ap.add_argument("--op-reps", type=int, default=10, help="launches per op for the breakdown")
    ap.add_argument("--event-every", type=int, default=2,
                    help="bracket the dominant op's launches with HIP events in every n-th step")
    ap.add_argument("--roofline-op", default=None,
                    help="op the roofline covers (default: the op with the most time per step)")
    ap.add_argument("--no-per-op", action="store_true",
                    help="skip the per-op breakdown (profiled runs: every kernel in the trace "
                         "then belongs to a step)")
    ap.add_argument("--cold-reps", type=int, default=5,
                    help="cold-MALL launches of each quantization of the largest layer (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-n", type=int, default=0,
                    help="batch elements of the first layer the CPU oracle runs on (0: the "
                         "workload's default sample)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (HBM counter calibration)")
    ap.add_argument("--inference", action="store_true",
                    help="the inference path only: quantize X from NCHW and conv fwd per layer "
                         "(weights quantized once before timing)")
    ap.add_argument("--network", default=None, choices=["resnet18"],
                    help="time a full training step of ResNet-18 (19 body convolutions on the "
                         "library, the rest in PyTorch fp32)")
    ap.add_argument("--batch", type=int, default=128, help="batch size of --network")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="print the traffic summary from two rocprofv3 --pmc databases")
    ap.add_argument("--summarize-trace", metavar="TRACE_DB",
                    help="print a kernel-trace summary (per kernel and launch shape) from a "
                         "rocprofv3 --kernel-trace database")
    ap.add_argument("--summarize-stalls", nargs=3, metavar=("DB_A", "DB_B", "DB_C"),
                    help="print wave waiting, LDS and MFMA shares per convolution kernel from three "
                         "rocprofv3 --pmc databases (the counter sets are in summarize_stalls)")
    ap.add_argument("--summarize-mfma", metavar="DB",
                    help="print MFMA busy and MFMA op counts per kernel from a rocprofv3 --pmc "
                         "database of SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F16, "
                         "SQ_BUSY_CU_CYCLES, GRBM_GUI_ACTIVE")
    return ap.parse_args(argv)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "microscaling_quantized_convolution_amd",
                                           "csrc", "*"))):
        if p.endswith((".hip", ".hpp", ".cpp")):
            h.update(os.path.basename(p).encode())
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(workload: str, layer: str) -> str:
    return os.path.join(ROOT, "profiles", f"{workload}_{layer.replace('.', '_')}_pmc_traffic.txt")


def read_traffic(path: str, op: str):
    """HBM bytes per launch of `op` from a committed counter summary, or None if there is none
    or it was taken on other kernel sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#", "|")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_source_hash():
        return None
    v = kv.get(f"traffic_bytes_per_launch.{op}")
    return None if v is None else int(float(v))


# ---- the work of one layer's ops (algorithmic, as the method defines it) -----------------------

def _squares(o0, o1, r, s):
    return o0 * o1 * ((r + 3) // 4) * ((s + 3) // 4)


def layer_work(l):
    """Per op of one layer: (kind, algorithmic amount, algorithmic bytes). kind 'hbm' amounts
    are bytes; 'gemm' amounts are flops. Quantization reads its fp32 tensor twice (the amax pass
    and the quantizing pass) and writes codes and scales; a GEMM reads both quantized operands
    once and writes its fp32 result once."""
    cb = 8 if l.fmt == 4 else 12
    q = lambda *shape: _squares(*shape) * (cb + 1)
    nx, nw, ng = l.N * l.Cin * l.H * l.W, l.Cout * l.Cin * l.Kh * l.Kw, l.N * l.Cout * l.Ho * l.Wo
    qx, qw, qg = q(l.H, l.W, l.Cin, l.N), q(l.Kh, l.Kw, l.Cout, l.Cin), q(l.Ho, l.Wo, l.Cout, l.N)
    F = l.gemm_flops()
    fwd_b, wg_b, dg_b = qx + qw + 4 * ng, qg + qx + 4 * nw, qw + qg + 4 * nx
    return {
        "quantize_xw": ("hbm", 8 * (nx + nw) + qx + qw, 8 * (nx + nw) + qx + qw),
        "quantize_x": ("hbm", 8 * nx + qx, 8 * nx + qx),
        "quantize_g": ("hbm", 8 * ng + qg, 8 * ng + qg),
        # the amax comes from the producer's epilogue: one read of G_Y
        "quantize_g_ready": ("hbm", 4 * ng + qg, 4 * ng + qg),
        "conv_fwd": ("gemm", F, fwd_b),
        "conv_wgrad": ("gemm", F, wg_b),
        "conv_dgrad": ("gemm", F, dg_b),
        "conv_backward": ("gemm", 2 * F, wg_b + dg_b),
        "conv_fwd_amax": ("gemm", F, fwd_b),
        "conv_backward_amax": ("gemm", 2 * F, wg_b + dg_b),
    }


def rate(kind, amount, nbytes, ms):
    """Rates and roofline fraction of one op launch taking `ms`."""
    ridge = MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    gbs = nbytes / (ms * 1e-3) / 1e9
    if kind == "hbm":
        return {"ms": round(ms, 5), "GB_s": round(gbs, 1), "bound": "hbm",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "alg_bytes": int(nbytes)}
    tf = amount / (ms * 1e-3) / 1e12
    mfma = amount / nbytes >= ridge
    return {"ms": round(ms, 5), "TFLOP_s": round(tf, 1), "GB_s": round(gbs, 1),
            "bound": "mfma" if mfma else "hbm",
            "frac": round(tf / MFMA_PEAK_TFLOPS if mfma else gbs / HBM_PEAK_GBS, 4),
            "alg_flops": int(amount), "alg_bytes": int(nbytes)}


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


def host_cpu():
    """(model name, threads the oracle's OpenMP runs with)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = min(avail, int(omp)) if omp and omp.isdigit() and int(omp) > 0 else avail
    return model, threads


def main(argv=None):
    args = parse(argv)
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.summarize_stalls:
        summarize_stalls(*args.summarize_stalls)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path here is single-device; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.network:
        run_network(args)
        return
    run_workload(args)


def run_workload(args):
    import collections

    import torch

    import microscaling_quantized_convolution_amd as mq
    from microscaling_quantized_convolution_amd.step import LayerStep
    import workloads

    torch.cuda.set_device(0)
    dev = "cuda:0"
    all_layers = workloads.CONFIGS[args.workload]()
    layers = all_layers
    if args.layers:
        want = args.layers.split(",")
        layers = [l for l in all_layers if l.name in want]
        if len(layers) != len(want):
            sys.exit(f"--layers: unknown names in {want} (have {[l.name for l in all_layers]})")
    nl = len(all_layers)
    stream = torch.cuda.Stream()
    ops = INFERENCE_OPS if args.inference else STEP_OPS

    # ---- every layer's inputs resident on the device, its own buffers ----
    steps, calls = [], []
    for l in layers:
        x, w, g = workloads.make_tensors(l)
        gc = torch.empty(g.size, dtype=torch.float32, device=dev)
        mq.mq_relayout_cbf(torch.from_numpy(g).to(dev), gc, l.N, l.Cout, l.Ho, l.Wo, 0)
        st = LayerStep(l.conv_tuple(), l.fmt, torch.from_numpy(x).to(dev),
                       torch.from_numpy(w).to(dev), gc, sr_seed_base=l.sr_seed, seed_stride=nl)
        del x, w, g
        steps.append(st)
        c = st.direct_calls(stream)
        if args.inference:
            for s_ in range(2):  # W quantized once, before timing
                c["quantize_xw"](s_)
            c.update(st.inference_calls(stream))
        calls.append(c)
    torch.cuda.synchronize()

    groups = collections.OrderedDict()  # distinct shape -> indices into layers
    for i, l in enumerate(layers):
        groups.setdefault(l.conv_tuple() + (l.fmt,), []).append(i)

    def run_step(s, brackets=None):
        for i in range(len(layers)):
            for op in ops:
                if brackets is not None and (i, op) in brackets:
                    e0, e1 = brackets[i, op]
                    e0.record(stream)
                    calls[i][op](s)
                    e1.record(stream)
                else:
                    calls[i][op](s)

    with torch.cuda.stream(stream):
        for s in range(max(args.warmup, 1)):
            run_step(s)
    torch.cuda.synchronize()

    # ---- per distinct layer shape: each op alone, `op_reps` launches back to back ----
    per_layer, op_ms = [], {}
    if not args.no_per_op:
        for key, idx in groups.items():
            l, c = layers[idx[0]], calls[idx[0]]
            work = layer_work(l)
            entry = {}
            for op in ops + ([] if args.inference else PARTS):
                ms = _time_graph([c[op]], args.op_reps, stream)
                kind, amount, nbytes = work[op]
                entry[op] = rate(kind, amount, nbytes, ms)
                op_ms[idx[0], op] = ms
            layer_ms = _time_graph([c[op] for op in ops], max(2, args.op_reps // 2), stream)
            per_layer.append({
                "layers": [layers[i].name for i in idx],
                "shape": {"N": l.N, "Cin": l.Cin, "Cout": l.Cout, "H": l.H, "W": l.W,
                          "K": [l.Kh, l.Kw], "stride": [l.stride, l.sw], "pad": [l.pad, l.pw],
                          "format": f"NVFP{l.fmt}"},
                "ms_layer": round(layer_ms, 5), "per_op": entry})

    # ---- the dominant kernel: the (shape, one-kernel op) with the most time per step ----
    if args.roofline_op and args.roofline_op not in ops:
        sys.exit(f"--roofline-op {args.roofline_op}: not an op of the step ({', '.join(ops)})")
    roof_ops = [args.roofline_op] if args.roofline_op else [op for op in ops if op in ONE_KERNEL_OPS]
    if op_ms:
        cand = [(op_ms[idx[0], op] * len(idx), key, op) for key, idx in groups.items()
                for op in roof_ops]
        _, dom_key, dom_op = max(cand)
    else:
        dom_key = next(iter(groups))
        dom_op = roof_ops[0]
    dom_idx = groups[dom_key]

    # ---- timed steps ----
    def ev():
        return torch.cuda.Event(enable_timing=True)

    brackets = [({(i, dom_op): (ev(), ev()) for i in dom_idx}
                 if s_ % args.event_every == 0 else None) for s_ in range(args.steps)]
    t0, t1 = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    with torch.cuda.stream(stream):
        t0.record(stream)
        for s in range(args.steps):
            run_step(args.warmup + s, brackets[s])
        t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    sampled = [p for b in brackets if b is not None for p in b.values()]
    dom_ms = sum(a.elapsed_time(b) for a, b in sampled) / len(sampled)

    dl = layers[dom_idx[0]]
    kind, amount, nbytes = layer_work(dl)[dom_op]
    roof = rate(kind, amount, nbytes, dom_ms)
    if roof["bound"] == "hbm":
        roof = {"bound": "hbm", "achieved": roof["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        alg = nbytes
    else:
        roof = {"bound": "mfma", "achieved": roof["TFLOP_s"], "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
        alg = amount
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = read_traffic(traffic_file(args.workload, dl.name), dom_op)
    roof.update({"op": dom_op, "layers": [layers[i].name for i in dom_idx],
                 "kernels": OP_KERNELS[dom_op], "ms_per_launch": round(dom_ms, 5),
                 "launches_timed": len(sampled), "alg_per_launch": int(alg)})

    flops = sum(l.gemm_flops() for l in layers) * (1 if args.inference else 3)
    result = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "wall_s_timed": round(wall, 4),
        "timing": "back-to-back launches on one stream",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded numpy PCG64: X=ReLU(N(0,1)) / SiLU / 0.5*t3, W Kaiming-normal, "
                "G_Y~N(0,1e-3))",
        "config": {"workload": workload_name(args, layers),
                   "layers": len(layers), "gemm_flops_per_step": int(flops),
                   "format": "NVFP4 (E2M1 codes, E4M3 4x4-square scales, fp32 tensor scale)"
                   if layers[0].fmt == 4 else "NVFP6 (E2M3 codes, E4M3 4x4-square scales, fp32 "
                                               "tensor scale)",
                   "mfma": "fp16 operands decoded exactly, fp32 accumulate"},
        "roofline": roof,
        "per_layer": per_layer,
    }

    if args.cold_reps > 0 and not args.inference:
        result["quantize_cold"] = quantize_cold(layers, calls, args.cold_reps, stream)

    if args.calib_copy:
        src = torch.full((CALIB_ELEMS,), 1.0, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        torch.neg(src, out=dst)
        e1.record()
        torch.cuda.synchronize()
        result["calib_copy"] = {"bytes_read": CALIB_ELEMS * 4, "bytes_written": CALIB_ELEMS * 4,
                                "ms": round(e0.elapsed_time(e1), 4)}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers[0], args.cpu_sample_n)

    print(json.dumps(result), flush=True)


def workload_name(args, layers):
    names = {"c1": "tiny 3x3 conv N=2 16->16 8x8 (NVFP4)",
             "c2": "ResNet 3x3 s1p1 conv N=32 64->64 56x56 (NVFP4)",
             "c3": "strided 3x3 s2p1 conv N=64 128->256 28->14 (NVFP4)",
             "c4": "YOLOv8n-like stack of 8 convs N=16, 160->20, 3 of 8 1x1 (NVFP6)",
             "c5": "ResNet-18 conv body (19 convs) N=128 at 224x224 (NVFP4)"}
    what = ("inference: quantize X (from NCHW), conv fwd per layer (W quantized once)"
            if args.inference else "per layer: quantize X (NCHW) + W (OIHW) in one batched call "
            "(RNE), G_Y (SR), conv fwd, conv backward (wgrad + dgrad in one call)")
    sel = "" if not args.layers else f" [layers {','.join(l.name for l in layers)}]"
    return f"{args.workload}: {names[args.workload]}{sel}; {what}"


def quantize_cold(layers, calls, reps, stream):
    """The largest layer's quantizations, each launch after reading FLUSH_BYTES of scratch (the
    MALL and L2 then hold none of its inputs, and no dirty lines that the launch would have to
    write back), against the same launches back to back (warm)."""
    import torch
    i = max(range(len(layers)), key=lambda k: layers[k].N * layers[k].Cin * layers[k].H * layers[k].W)
    l = layers[i]
    work = layer_work(l)
    scratch = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    out = {"layer": l.name}
    for op in ("quantize_xw", "quantize_g"):
        cold = []
        with torch.cuda.stream(stream):
            for r in range(reps + 1):
                flush = scratch.max()  # a read of every scratch line
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                calls[i][op](r)
                e1.record(stream)
                cold.append((e0, e1))
        torch.cuda.synchronize()
        ms_cold = sum(a.elapsed_time(b) for a, b in cold[1:]) / reps
        ms_warm = _time_graph([calls[i][op]], 10, stream)
        kind, amount, nbytes = work[op]
        out[op] = {"cold": rate(kind, amount, nbytes, ms_cold),
                   "warm": rate(kind, amount, nbytes, ms_warm)}
    # the practical streaming ceiling for the same bytes: a plain device copy of X's size (one
    # read, one write of fp32), cold as above
    n = l.N * l.Cin * l.H * l.W
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    cold = []
    with torch.cuda.stream(stream):
        for r in range(reps + 1):
            flush = scratch.max()  # a read of every scratch line
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            cold.append((e0, e1))
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in cold[1:]) / reps
    out["copy_reference"] = {"bytes": 8 * n, "ms": round(ms, 5),
                             "GB_s": round(8 * n / (ms * 1e-3) / 1e9, 1),
                             "frac": round(8 * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return out


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
    """The CPU oracle, as it stands, on the first `nsample` batch elements of a layer: relayout,
    three quantizations, dequantization and the three explicit-im2col GEMMs in double, repeated
    to about 10 s. Reported in the same unit as `value` (TFLOP/s of the sample's three GEMMs)."""
    import dataclasses

    import oracle
    import workloads

    if nsample <= 0:
        nsample = min(layer.N, 8)
    nsample = min(nsample, layer.N)
    sub = dataclasses.replace(layer, N=nsample)
    x, w, g = workloads.make_tensors(layer)
    x, g = x[:nsample].copy(), g[:nsample].copy()
    model, threads = host_cpu()
    p = sub.conv_tuple()
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
    return {"value": round(tf, 6), "unit": "TFLOP/s", "cores": threads, "cpu": model,
            "kind": "oracle", "seconds_per_pass": round(sec, 3), "passes": len(secs),
            "sample": f"layer {layer.name} ({layer.Cin}->{layer.Cout}, {layer.H}x{layer.W}, "
                      f"{layer.Kh}x{layer.Kw}) with N={nsample} of {layer.N} batch elements: "
                      f"relayout, 3 quantizations, dequantization, explicit-im2col "
                      f"fwd/wgrad/dgrad in double, repeated to about 10 s; flops of the "
                      f"sample's three GEMMs / mean wall time per pass"}


# ---- profile summaries --------------------------------------------------------------------------

def _short(name: str) -> str:
    """Kernel name without its parameter list."""
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                return name[:i]
    return name


def _pmc_per_kernel(db: str, counters, by_grid: bool = False):
    """Mean per dispatch of each counter (summed over its instances) per kernel name, or per kernel
    name and grid (workgroups along x, y, z) with by_grid."""
    import collections
    import sqlite3
    con = sqlite3.connect(db)
    cols = [r[1] for r in con.execute("pragma table_info(counters_collection)")]
    ki, ci, vi, di = (cols.index(c) for c in ("kernel_name", "counter_name", "value",
                                              "dispatch_id"))
    gi = [cols.index(c) for c in ("grid_size_x", "grid_size_y", "grid_size_z", "workgroup_size_x")]
    per = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    for row in con.execute("select * from counters_collection"):
        if row[ci] in counters:
            key = _short(row[ki])
            if by_grid:
                gx, gy, gz, wx = (row[i] for i in gi)
                key = f"{key} ({gx // max(wx, 1)}, {gy}, {gz}) x {wx}"
            d = per[row[ci]][key]
            if row[ci] == "GRBM_GUI_ACTIVE":  # one chip-wide clock: the largest instance
                d[row[di]] = max(d[row[di]], row[vi])
            else:
                d[row[di]] += row[vi]
    return {c: {k: (sum(d.values()) / len(d), len(d)) for k, d in per[c].items()}
            for c in counters}


def summarize_pmc(fetch_db: str, write_db: str):
    """Traffic summary (key: value lines) from a FETCH_SIZE run and a WRITE_SIZE run of
    `bench.py --calib-copy` on one layer; the counters are KiB per dispatch."""
    fetch = _pmc_per_kernel(fetch_db, ["FETCH_SIZE"])["FETCH_SIZE"]
    write = _pmc_per_kernel(write_db, ["WRITE_SIZE"])["WRITE_SIZE"]
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
    # per op of the layer (the quantize ops share kernel names, so only the convolutions, whose
    # kernels are distinct, get a per-op figure)
    for op in ("conv_fwd", "conv_backward", "conv_wgrad", "conv_dgrad"):
        tot = sum(b for k, b in per_kernel.items()
                  if any(k.replace("(anonymous namespace)::", "").startswith(p)
                         for p in OP_KERNELS[op]))
        print(f"traffic_bytes_per_launch.{op}: {tot:.0f}")


def summarize_trace(db: str):
    """Markdown table from a rocprofv3 --kernel-trace database: per kernel and launch shape (grid
    and workgroup size, so the layer shapes of one kernel template stay apart), the dispatches,
    mean / min / max duration, total time and share, registers and LDS."""
    import collections
    import sqlite3
    con = sqlite3.connect(db)
    groups = collections.defaultdict(list)
    info = {}
    for name, dur, gx, gy, gz, wx, vg, ag, lds in con.execute(
            "select name, duration, grid_x, grid_y, grid_z, workgroup_x, vgpr_count, "
            "accum_vgpr_count, lds_size from kernels"):
        key = (_short(name).replace("(anonymous namespace)::", ""), gx // max(wx, 1), gy, gz, wx)
        groups[key].append(dur)
        info[key] = (vg, ag, lds)
    tot = sum(sum(v) for v in groups.values())
    print(f"kernel_sources_sha256: {kernel_source_hash()}")
    print()
    print("| kernel | workgroups (x, y, z) x lanes | dispatches | mean us | min us | max us | "
          "total us | share | VGPR / AGPR | LDS B |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for key, d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        name, bx, gy, gz, wx = key
        vg, ag, lds = info[key]
        print(f"| `{name[:100]}` | ({bx}, {gy}, {gz}) x {wx} | {len(d)} | "
              f"{sum(d) / len(d) / 1e3:.2f} | {min(d) / 1e3:.2f} | {max(d) / 1e3:.2f} | "
              f"{sum(d) / 1e3:.1f} | {sum(d) / tot:.3f} | {vg} / {ag} | {lds} |")


def summarize_mfma(db: str):
    """MFMA utilisation per kernel and grid from one rocprofv3 --pmc run. SQ_VALU_MFMA_BUSY_CYCLES
    counts busy cycles summed over the 1024 SIMDs (a 32x32x16 fp16 MFMA keeps its SIMD busy 32
    cycles); GRBM_GUI_ACTIVE reads the 8 XCDs' active cycles summed. util = busy / (GRBM_GUI_ACTIVE
    / 8 x 1024): the matrix cores' busy fraction at the clock they ran. The fp16 MFMA flops come
    from SQ_INSTS_VALU_MFMA_MOPS_F16 (512 flop each); TFLOP/s divides them by the dispatch's
    duration under the counters, and frac compares that with the 2.5 PFLOP/s dense fp16 peak."""
    import collections
    import sqlite3
    cs = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_BUSY_CU_CYCLES",
          "GRBM_GUI_ACTIVE"]
    per = _pmc_per_kernel(db, cs, by_grid=True)
    con = sqlite3.connect(db)
    dur = collections.defaultdict(dict)
    for name, gx, gy, gz, wx, did, d in con.execute(
            "select kernel_name, grid_size_x, grid_size_y, grid_size_z, workgroup_size_x, "
            "dispatch_id, duration from counters_collection"):
        dur[f"{_short(name)} ({gx // max(wx, 1)}, {gy}, {gz}) x {wx}"][did] = d
    print(f"kernel_sources_sha256: {kernel_source_hash()}")
    print()
    print("| kernel (workgroups x lanes) | dispatches | mean us | MFMA busy SIMD-cycles | "
          "GRBM_GUI_ACTIVE (8 XCDs) | MFMA util | fp16 MFMA GFLOP | TFLOP/s | frac of 2.5 PF |")
    print("|---|---|---|---|---|---|---|---|---|")
    names = sorted(set().union(*[set(per[c]) for c in cs]))
    rows = []
    for k in names:
        busy = per["SQ_VALU_MFMA_BUSY_CYCLES"].get(k, (0.0, 0))
        act = per["GRBM_GUI_ACTIVE"].get(k, (0.0, 0))[0]
        mops = per["SQ_INSTS_VALU_MFMA_MOPS_F16"].get(k, (0.0, 0))[0]
        if mops == 0:
            continue
        us = sum(dur[k].values()) / max(len(dur[k]), 1) / 1e3
        util = busy[0] / (act / 8 * 1024) if act else 0.0
        gf = mops * 512 / 1e9
        tf = gf / us * 1e3 if us else 0.0  # GFLOP per us = PFLOP/s
        rows.append((-gf * busy[1], k, busy[1], us, busy[0], act, util, gf, tf))
    for _, k, n, us, b, act, util, gf, tf in sorted(rows):
        print(f"| `{k.replace('(anonymous namespace)::', '')[:130]}` | {n} | {us:.2f} | {b:.3e} | "
              f"{act:.3e} | {util:.3f} | {gf:.3f} | {tf:.1f} | {tf / MFMA_PEAK_TFLOPS:.3f} |")


# the three counter passes of summarize_stalls (at most 8 SQ counters and GRBM_GUI_ACTIVE each)
STALL_COUNTERS = (
    ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS",
     "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_UNALIGNED_STALL",
     "SQ_LDS_DATA_FIFO_FULL", "GRBM_GUI_ACTIVE"],
    ["SQ_INSTS_LDS_LOAD", "SQ_INSTS_LDS_STORE", "SQ_INSTS_LDS_LOAD_BANDWIDTH",
     "SQ_INSTS_LDS_STORE_BANDWIDTH", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_MISC", "SQ_WAIT_ANY",
     "SQ_LDS_ADDR_CONFLICT", "GRBM_GUI_ACTIVE"],
    ["SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY",
     "SQ_INST_LEVEL_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
)


def summarize_stalls(db_a: str, db_b: str, db_c: str):
    """Per convolution kernel and grid, from three rocprofv3 --pmc runs of STALL_COUNTERS:
    MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs' active cycles, as summarize_mfma);
    the share of wave-cycles spent waiting on any dependency (SQ_WAIT_ANY / SQ_WAVE_CYCLES) and
    waiting to issue an LDS instruction (SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES); LDS bank-conflict
    cycles over LDS indexed-active cycles; and SQ_LDS_IDX_ACTIVE over 256 CUs' active cycles (the
    LDS's busy share per CU, read as a sum over the CUs)."""
    vals = collections_dd()
    for db, cs in zip((db_a, db_b, db_c), STALL_COUNTERS):
        for c, d in _pmc_per_kernel(db, cs, by_grid=True).items():
            for k, (v, n) in d.items():
                vals[k][c if c != "GRBM_GUI_ACTIVE" else c + db] = v
                vals[k]["n"] = n
    print(f"kernel_sources_sha256: {kernel_source_hash()}")
    print()
    print("| kernel (workgroups x lanes) | dispatches | MFMA busy | waves waiting | waiting on LDS "
          "issue | LDS bank conflicts / LDS active | LDS active per CU |")
    print("|---|---|---|---|---|---|---|")
    for k in sorted(vals):
        v = vals[k]
        if "conv_" not in k or not v.get("SQ_WAVE_CYCLES"):
            continue
        act = v.get("GRBM_GUI_ACTIVE" + db_c, 0.0) / 8
        act_a = v.get("GRBM_GUI_ACTIVE" + db_a, 0.0) / 8
        mfma = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (act * 1024) if act else 0.0
        wait = v.get("SQ_WAIT_ANY", 0.0) / v["SQ_WAVE_CYCLES"]
        wlds = v.get("SQ_WAIT_INST_LDS", 0.0) / v["SQ_WAVE_CYCLES"]
        lact = v.get("SQ_LDS_IDX_ACTIVE", 0.0)
        bc = v.get("SQ_LDS_BANK_CONFLICT", 0.0) / lact if lact else 0.0
        lcu = lact / (act_a * 256) if act_a else 0.0
        print(f"| `{k.replace('(anonymous namespace)::', '')[:130]}` | {v['n']} | {mfma:.3f} | "
              f"{wait:.3f} | {wlds:.3f} | {bc:.4f} | {lcu:.3f} |")


def collections_dd():
    import collections
    return collections.defaultdict(dict)


if __name__ == "__main__":
    main()
