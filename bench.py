#!/usr/bin/env python3
"""Benchmark of the int8-weight MoE feed-forward layer on one MI355X.

A step is one forward of the whole layer (router + top-K gate, permutation,
gate/up contraction with SwiGLU, down contraction, weighted combine) over one
batch of synthetic tokens, through the fused C-ABI call moe_forward. Inputs
and int8 weights are resident in HBM before timing starts.

Default workload: Jamba-Mini-shaped decode step, T=32 tokens, d=4096,
f=14336, 16 experts, top-2, bf16 activations, int8 per-output-channel weights
with bf16 scales. The prefill workload that shares the same weights (T=8192)
is measured in the same run and reported under "prefill".

Printed: one JSON line with the throughput (tokens/s), the roofline of the
dominant kernel measured with HIP events on the launch stream, and the CPU
oracle timed on a bounded sample of the same workload (host cores).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

# decode workload -> the prefill workload with the same weights
SIBLING = {"mini-decode": "mini-prefill", "large-decode": "large-prefill-skewed",
           "large-mlp-decode": "large-mlp-prefill", "large-decode-tp8": "large-prefill-skewed-tp8"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mini-decode")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true", help="skip the sibling prefill workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the weight-encoding comparators (the same layer with bf16 or fp8 weights)")
    ap.add_argument("--cpu-sample-experts", type=int, default=4)
    ap.add_argument("--path", choices=["auto", "stream", "tiled"], default="auto")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (reference for HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- setup
def build_layer(w, dev):
    import torch
    import workloads
    from int8_weight_moe_amd import MoeLayer, quantize_experts

    wr, bias = workloads.draw_router(w)
    src = workloads.draw_expert_weights(w, dev)
    sdt = workloads.TORCH_DTYPE[w.scale]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ex = quantize_experts(src["w_gate"], src["w_up"], src["w_down"], sdt)
    torch.cuda.synchronize()
    qms = (time.perf_counter() - t0) * 1e3
    layer = MoeLayer(wr.to(dev), None if bias is None else bias.to(dev), ex, w.K)
    return layer, src, qms


def touched_rows(layer, x, path):
    """Per-expert row counts of this input (one staged route + permute)."""
    from int8_weight_moe_amd import moe_permute, moe_route
    ids, _ = moe_route(x, layer.router_w, layer.bias, layer.K)
    off, _, _ = moe_permute(ids, layer.experts.E)
    o = off.cpu().tolist()
    return [o[i + 1] - o[i] for i in range(len(o) - 1)]


def algorithmic(w, counts, wfmt="int8"):
    """Bytes and flops the layer (and each contraction kernel) must move / compute.

    wfmt: weight encoding -- int8 or fp8 (1 byte per weight plus per-channel
    scales) or bf16 (2 bytes per weight, no scales)."""
    ab = 4 if w.act == "f32" else 2
    wb = 2 if wfmt == "bf16" else 1
    sb = 0 if wfmt == "bf16" else (4 if w.scale == "f32" else 2)
    touched = sum(1 for c in counts if c > 0)
    S = w.T * w.K
    d, f = w.d, w.f
    gate_up_bytes = touched * (2 * d * f * wb + 2 * f * sb) + w.T * d * ab + S * f * 2
    down_bytes = touched * (d * f * wb + d * sb) + S * f * 2 + S * d * 4
    layer_bytes = touched * (3 * d * f * wb + (2 * f + d) * sb) + 2 * w.T * d * ab + w.E * d * ab
    return {
        "touched": touched,
        "gate_up_bytes": gate_up_bytes, "down_bytes": down_bytes, "layer_bytes": layer_bytes,
        "gate_up_flops": 4.0 * S * d * f, "down_flops": 2.0 * S * d * f, "layer_flops": 6.0 * S * d * f,
    }


def ffn_path_used(w, path):
    """Schedule the library runs: it streams weights when T*K <= 64*E rows (decode-sized)."""
    from int8_weight_moe_amd._lib import MOE_PATH_AUTO, MOE_PATH_STREAM
    if path == MOE_PATH_STREAM or (path == MOE_PATH_AUTO and w.T * w.K <= 64 * w.E):
        return "stream"
    return "tiled"


# ----------------------------------------------------------------------------- timing
def time_forward(layer, x, path, steps, warmup, dense=False):
    """Average step time of the fused call: moe_forward, or moe_mlp_forward for a dense MLP layer."""
    import torch
    from int8_weight_moe_amd import moe_mlp_forward
    y = torch.empty_like(x)
    ids = torch.empty((x.shape[0], layer.K), dtype=torch.int32, device=x.device)
    gw = torch.empty((x.shape[0], layer.K), dtype=torch.float32, device=x.device)
    ws = layer.workspace(layer.shape(x, path))

    def step():
        if dense:
            moe_mlp_forward(x, layer.experts, path=path, y=y, workspace=ws)
        else:
            layer.forward(x, path=path, y=y, ids=ids, w=gw)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return start.elapsed_time(end) / steps, wall


def time_stages(layer, x, path, steps, warmup, dense=False):
    """Average duration (us) of each kernel of the step, HIP events on the launch stream.

    A dense MLP layer has no routing: its row layout (every token once, weight
    1) is set up once, outside the timed stages, and only the FFN passes and
    the combine are timed."""
    import torch
    from int8_weight_moe_amd import moe_combine, moe_expert_down, moe_expert_gate_up, moe_permute, moe_route
    from int8_weight_moe_amd.ops import down_workspace_size, make_shape
    ex, K = layer.experts, layer.K
    T = x.shape[0]
    names = ["gate_up", "down", "combine"] if dense else ["route", "permute", "gate_up", "down", "combine"]
    h = torch.empty((T * K, ex.f), dtype=torch.bfloat16, device=x.device)
    rows = torch.empty((T * K, ex.d), dtype=torch.float32, device=x.device)
    dshape = make_shape(T, ex.d, ex.f, ex.E, K, x.dtype, ex.scale_dtype, path, ex.fmt)
    dws = torch.empty(max(down_workspace_size(dshape), 256), dtype=torch.uint8, device=x.device)
    if dense:
        ids0, gw0 = moe_route(x, layer.router_w, layer.bias, K)
        layout = (gw0,) + tuple(moe_permute(ids0, ex.E))

    def step(ev):
        i = 0
        ev[i].record()
        if dense:
            gw, off, ss, s2r = layout
        else:
            ids, gw = moe_route(x, layer.router_w, layer.bias, K)
            i += 1
            ev[i].record()
            off, ss, s2r = moe_permute(ids, ex.E)
            i += 1
            ev[i].record()
        moe_expert_gate_up(x, off, ss, ex, K, path=path, h=h)
        ev[i + 1].record()
        moe_expert_down(h, off, ex, T, K, act=x.dtype, path=path, y_rows=rows, workspace=dws)
        ev[i + 2].record()
        moe_combine(rows, s2r, gw, x.dtype)
        ev[i + 3].record()

    n_ev = len(names) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    for _ in range(warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(n_ev)])
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    out = {}
    for j, n in enumerate(names):
        out[n] = 1e3 * statistics.mean(e[j].elapsed_time(e[j + 1]) for e in evs)
    return out


def _code_only(text):
    """Source text without comments and blank space, so that edits to comments
    do not invalidate the counter measurements tied to the code."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split())


def kernel_hash():
    """Hash of the code of the FFN kernels (comments and spacing excluded)."""
    hsh = hashlib.sha256()
    for f in ("ffn_stream.hip", "ffn_tiled.hip", "device_common.h"):
        with open(os.path.join(ROOT, "int8_weight_moe_amd", "csrc", f)) as fh:
            hsh.update(_code_only(fh.read()).encode())
    return hsh.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def roofline(w, alg, stages, dominant, workload, hbm_bound):
    dur_s = stages[dominant] * 1e-6
    if hbm_bound:  # decode-sized: weight streaming
        ach = alg[f"{dominant}_bytes"] / dur_s / 1e9
        traffic = measured_traffic(workload, dominant)
        return {"kernel": dominant, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "algorithmic_bytes": alg[f"{dominant}_bytes"],
                "avg_us": round(stages[dominant], 2)}
    ach = alg[f"{dominant}_flops"] / dur_s / 1e12
    return {"kernel": dominant, "bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(workload, dominant), "algorithmic_flops": alg[f"{dominant}_flops"],
            "avg_us": round(stages[dominant], 2)}


# ----------------------------------------------------------------------------- CPU oracle baseline
def cpu_baseline(w, x_host, layer, src, n_experts):
    """The oracle (unchanged) on the host cores, on a bounded sample of the step.

    Timed: the router + gate for every token, the SwiGLU experts of `n_experts`
    touched experts (all their rows) and the combine of those rows. The step
    estimate scales the expert time by touched / sampled experts.
    """
    import numpy as np
    import torch
    from oracle import moe as omoe
    from oracle import quant as oquant
    try:
        import threadpoolctl
        cores = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))

    x64 = x_host.double().numpy()
    wr64 = layer.router_w.double().cpu().numpy()
    b64 = None if layer.bias is None else layer.bias.double().cpu().numpy()
    ids, gw, _ = omoe.route(x64, wr64, b64, w.K)
    touched = sorted(set(ids.reshape(-1).tolist()))
    sample = touched[:n_experts]
    W = {k: {} for k in ("q_gate", "s_gate", "q_up", "s_up", "q_down", "s_down")}
    for e in sample:   # load-time quantization by the oracle: not timed
        for k in ("gate", "up", "down"):
            q, s = oquant.quantize_rows(src["w_" + k][e].double().cpu().numpy(), w.scale)
            W["q_" + k][e], W["s_" + k][e] = q, s
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        ids2, gw2, _ = omoe.route(x64, wr64, b64, w.K)
        t1 = time.perf_counter()
        o = omoe.expert_outputs(x64, ids2, W, experts=sample)
        mask = np.isin(ids2, sample)
        y = omoe.combine(np.where(mask[..., None], o, 0.0), np.where(mask, gw2, 0.0))
        t2 = time.perf_counter()
        times.append((t1 - t0, t2 - t1))
    tr = statistics.median(t[0] for t in times)
    te = statistics.median(t[1] for t in times)
    est = tr + te * len(touched) / len(sample)
    del y
    return {"value": round(w.T / est, 2), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"router+gate over all {w.T} tokens; SwiGLU experts + combine for {len(sample)} of "
                      f"{len(touched)} touched experts (all their rows), fp64 NumPy; step time scaled by "
                      f"{len(touched)}/{len(sample)}; median of 3",
            "step_ms_estimate": round(est * 1e3, 1)}


def vendor_gemm_reference(wp, dev, iters=10):
    """Context for the MFMA roofline: the vendor library's plain bf16 GEMM (torch.matmul ->
    hipBLASLt) on the prefill contractions as single dense GEMMs (no grouping, no
    dequantization): [S, d] x [d, 2f] and [S, f] x [f, d]. Returns TFLOP/s of each."""
    import torch
    S = wp.T * wp.K
    out = {}
    for name, (M, N, K) in (("gate_up", (S, 2 * wp.f, wp.d)), ("down", (S, wp.d, wp.f))):
        a = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
        b = torch.randn(N, K, device=dev, dtype=torch.bfloat16)
        c = a @ b.t()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            c = a @ b.t()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        out[name + "_tflops"] = round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)
        del a, b, c
    torch.cuda.empty_cache()
    return out


def measure_prefill(layer, wp, xp, bias, args, dense, wfmt="int8"):
    """Step time, kernel split and roofline of the sibling prefill workload on this layer."""
    from int8_weight_moe_amd._lib import MOE_PATH_AUTO
    orig_bias = layer.bias
    if bias is not None:
        layer.bias = bias
    cp = touched_rows(layer, xp, MOE_PATH_AUTO)
    ap_ = algorithmic(wp, cp, wfmt)
    pms, _ = time_forward(layer, xp, MOE_PATH_AUTO, args.prefill_steps, 2, dense)
    pst = time_stages(layer, xp, MOE_PATH_AUTO, max(3, args.prefill_steps // 2), 1, dense)
    layer.bias = orig_bias
    pdom = max(("gate_up", "down"), key=lambda k: pst[k])
    log(f"prefill {wp.name} ({wfmt} weights): {pms:.3f} ms/step; stages (us): "
        + ", ".join(f"{k}={v:.1f}" for k, v in pst.items()))
    out = {
        "workload": wp.name, "T": wp.T, "ms_per_step": round(pms, 4),
        "tokens_per_s": round(wp.T / (pms * 1e-3), 1),
        "layer_tflops": round(ap_["layer_flops"] / (pms * 1e-3) / 1e12, 1),
        "layer_mfma_frac": round(ap_["layer_flops"] / (pms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernels_us": {k: round(v, 2) for k, v in pst.items()},
    }
    if wfmt == "int8":
        out["roofline"] = roofline(wp, ap_, pst, pdom, wp.name, ffn_path_used(wp, MOE_PATH_AUTO) == "stream")
    return out


# ----------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer's path is built and measured on a single MI355X "
              "(no collectives). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    from int8_weight_moe_amd._lib import MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED

    path = {"auto": MOE_PATH_AUTO, "stream": MOE_PATH_STREAM, "tiled": MOE_PATH_TILED}[args.path]
    w = workloads.ALL_WORKLOADS[args.workload]
    dense = args.workload in workloads.DENSE_WORKLOADS
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: T={w.T} d={w.d} f={w.f} E={w.E} K={w.K}")
    layer, src, qms = build_layer(w, dev)
    log(f"weights drawn and quantized on the GPU ({qms:.1f} ms for {3 * w.E * w.d * w.f / 1e9:.2f} G weights)")
    x_host = workloads.draw_activations(w)
    x = x_host.to(dev)
    counts = touched_rows(layer, x, path)
    alg = algorithmic(w, counts)

    ms, wall_ms = time_forward(layer, x, path, args.steps, args.warmup, dense)
    log(f"forward: {ms * 1e3:.1f} us/step (wall {wall_ms * 1e3:.1f} us)")
    stages = time_stages(layer, x, path, args.steps, args.warmup, dense)
    log("stages (us): " + ", ".join(f"{k}={v:.1f}" for k, v in stages.items()))
    dominant = max(("gate_up", "down"), key=lambda k: stages[k])
    used_path = ffn_path_used(w, path)

    layer_s = ms * 1e-3
    result = {
        "metric": "MLP-layer tokens/s" if dense else "MoE-layer tokens/s",
        "value": round(w.T / layer_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "f": w.f, "E": w.E, "K": w.K,
                   "weights": f"int8 per-output-channel, {w.scale} scales", "activations": w.act,
                   "ffn_path": used_path, "parallelism": "single GPU"},
        "roofline": roofline(w, alg, stages, dominant, w.name, used_path == "stream"),
        "layer": {"algorithmic_GB": round(alg["layer_bytes"] / 1e9, 4),
                  "hbm_GBps": round(alg["layer_bytes"] / layer_s / 1e9, 1),
                  "hbm_frac": round(alg["layer_bytes"] / layer_s / 1e9 / HBM_PEAK_GBPS, 4),
                  "tflops": round(alg["layer_flops"] / layer_s / 1e12, 2),
                  "touched_experts": alg["touched"]},
        "kernels_us": {k: round(v, 2) for k, v in stages.items()},
        "quantize_ms": round(qms, 2),
    }

    # the sibling prefill workload of the same layer (same weights)
    prefill_x, prefill_bias = None, None
    sib = SIBLING.get(w.name)
    if sib and not args.no_prefill:
        wp = workloads.ALL_WORKLOADS[sib]
        if (wp.d, wp.f, wp.E) == (w.d, w.f, w.E):
            prefill_x = workloads.draw_activations(wp).to(dev)
            if wp.has_bias:
                prefill_bias = torch.tensor([wp.hot_bias, wp.hot_bias] + [0.0] * (w.E - 2), device=dev)
            result["prefill"] = measure_prefill(layer, wp, prefill_x, prefill_bias, args, dense)
            result["prefill"]["vendor_bf16_gemm"] = vendor_gemm_reference(wp, dev)
            log(f"vendor bf16 GEMM reference (hipBLASLt, ungrouped): {result['prefill']['vendor_bf16_gemm']}")

    # weight-encoding comparators: the same layer, inputs and schedule choice
    if not args.no_compare and w.act == "bf16" and w.weight_src == "bf16":
        from int8_weight_moe_amd import MoeLayer, pack_bf16_experts, quantize_experts_fp8
        comp = {}
        for name in ("bf16", "fp8"):
            if name == "bf16":
                ex = pack_bf16_experts(src["w_gate"], src["w_up"], src["w_down"])
            else:
                ex = quantize_experts_fp8(src["w_gate"], src["w_up"], src["w_down"], workloads.TORCH_DTYPE[w.scale])
            clayer = MoeLayer(layer.router_w, layer.bias, ex, w.K)
            cms, _ = time_forward(clayer, x, path, args.steps, args.warmup, dense)
            cst = time_stages(clayer, x, path, args.steps, args.warmup, dense)
            calg = algorithmic(w, counts, wfmt=name)
            log(f"{name} weights: {cms * 1e3:.1f} us/step; stages (us): "
                + ", ".join(f"{k}={v:.1f}" for k, v in cst.items()))
            entry = {"weights": "bf16 as stored, no scales" if name == "bf16" else
                     f"fp8 e4m3 per-output-channel, {w.scale} scales",
                     "ms_per_step": round(cms, 4), "tokens_per_s": round(w.T / (cms * 1e-3), 1),
                     "int8_speedup": round(cms / ms, 3),
                     "layer_GB": round(calg["layer_bytes"] / 1e9, 4),
                     "hbm_GBps": round(calg["layer_bytes"] / (cms * 1e-3) / 1e9, 1),
                     "kernels_us": {k: round(v, 2) for k, v in cst.items()}}
            if prefill_x is not None:
                wp = workloads.ALL_WORKLOADS[sib]
                pr = measure_prefill(clayer, wp, prefill_x, prefill_bias, args, dense, wfmt=name)
                entry["prefill"] = {"workload": wp.name, "ms_per_step": pr["ms_per_step"],
                                    "int8_speedup": round(pr["ms_per_step"] / result["prefill"]["ms_per_step"], 3),
                                    "kernels_us": pr["kernels_us"]}
            comp[name + "_weights"] = entry
            del ex, clayer
            torch.cuda.empty_cache()
        result["comparators"] = comp
    del prefill_x

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {args.copy_calibration_mib} MiB device copies")
        del a, b

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w, x_host, layer, src, args.cpu_sample_experts)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
