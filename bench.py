#!/usr/bin/env python3
"""Benchmark of the int8-weight MoE feed-forward layer on one MI355X.

A step is one forward of the whole layer (router + top-K gate, permutation,
gate/up contraction with SwiGLU, down contraction, weighted combine) over one
batch of synthetic tokens, through the fused C-ABI call moe_forward. Inputs
and int8 weights are resident in HBM before timing starts. Each timed region
of K steps follows W warm-up steps, and before those the step runs untimed
for at least PREWARM_MS (the clocks ramp up over tens of milliseconds).

Default (headline) workload: the Jamba-1.5-Large-shaped MoE layer at prefill
with skewed routing, T=16384 tokens, d=8192, f=24576, 16 experts, top-2,
bf16 activations, int8 per-output-channel weights with bf16 scales, router
bias +2.0 on experts 0 and 1 (the largest workload that fits one GPU). The
decode workload on the same weights (T=64) is measured in the same run and
reported under "decode".

Printed: one JSON line with the throughput (tokens/s), the step-time spread,
the roofline of the dominant kernel measured with HIP events on the launch
stream, and the CPU oracle timed on a bounded sample of the same workload
(host cores).

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

# decode and prefill workloads that share one layer's weights
_PAIRS = {"mini-decode": "mini-prefill", "large-decode": "large-prefill-skewed",
          "large-mlp-decode": "large-mlp-prefill", "large-decode-tp8": "large-prefill-skewed-tp8"}
SIBLING = {**_PAIRS, **{v: k for k, v in _PAIRS.items()}}
HEADLINE = "large-prefill-skewed"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--sibling-steps", type=int, default=50,
                    help="timed steps of the sibling workload on the same weights (decode: 50, prefill: 10)")
    ap.add_argument("--no-sibling", action="store_true", help="skip the sibling workload on the same weights")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the weight-encoding comparators (the same layer with bf16 or fp8 weights)")
    ap.add_argument("--no-vendor", action="store_true", help="skip the vendor bf16 GEMM context figures")
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
# Untimed run of the step itself before its warm-up steps, at least this long:
# the GPU's clocks take tens of milliseconds to ramp up from a lighter load,
# which a few warm-up steps of a sub-millisecond decode step do not cover
# (the Large dense MLP at T=64 measured 157, 154, then 140 us per step over
# three back-to-back 20-step regions after 5 warm-up steps, 132 us after 200).
PREWARM_MS = 200.0


def prewarm(step):
    import torch
    t_end = time.perf_counter() + PREWARM_MS * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


def time_forward(layer, x, path, steps, warmup, dense=False):
    """Step time of the fused call: moe_forward, or moe_mlp_forward for a dense MLP layer.

    One timed region of `steps` back-to-back calls bracketed by synchronisations;
    a HIP event after every call also gives each step's own duration. Returns
    (ms per step over the region, wall ms per step, [per-step ms])."""
    import ctypes
    import torch
    from int8_weight_moe_amd import _lib
    from int8_weight_moe_amd.ops import _ptr, _stream
    y = torch.empty_like(x)
    ids = torch.empty((x.shape[0], layer.K), dtype=torch.int32, device=x.device)
    gw = torch.empty((x.shape[0], layer.K), dtype=torch.float32, device=x.device)
    shape = layer.shape(x, path)
    ws = layer.workspace(shape)
    ex = layer.experts
    # the C call with its arguments marshalled once: at decode sizes the
    # per-call Python marshalling would otherwise approach the step's GPU time
    lib = _lib.load()
    weights = (_ptr(ex.q_gate), _ptr(ex.q_up), _ptr(ex.q_down), _ptr(ex.s_gate), _ptr(ex.s_up), _ptr(ex.s_down))
    tail = (_ptr(ws), ctypes.c_size_t(ws.numel()), _stream())
    if dense:
        fn, args = lib.moe_mlp_forward, (ctypes.byref(shape), _ptr(x), *weights, _ptr(y), *tail)
    else:
        fn, args = lib.moe_forward, (ctypes.byref(shape), _ptr(x), _ptr(layer.router_w), _ptr(layer.bias), *weights,
                                     _ptr(y), _ptr(ids), _ptr(gw), *tail)

    def step():
        st = fn(*args)
        if st:
            _lib.check(st)

    prewarm(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[steps]) / steps, wall, per_step


def spread(per_step):
    """p10 / median / p90 of the per-step durations (ms)."""
    v = sorted(per_step)

    def q(p):
        k = (len(v) - 1) * p
        lo = int(k)
        hi = min(lo + 1, len(v) - 1)
        return v[lo] + (v[hi] - v[lo]) * (k - lo)
    return {"p10_ms": round(q(0.1), 4), "p50_ms": round(q(0.5), 4), "p90_ms": round(q(0.9), 4)}


# host time per staged call (ms), generous: the wrappers allocate nothing but
# build a shape and query a workspace size per call
_STAGE_HOST_MS = {"route": 0.1, "permute": 0.1, "gate_up": 0.1, "down": 0.1, "combine": 0.1}
_SPIN_MS_PER_MCYCLE = []


def gpu_lead(ms):
    """Enqueue a spin kernel that keeps the GPU busy for about `ms` (at most 100)."""
    import torch
    if not _SPIN_MS_PER_MCYCLE:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        e1.synchronize()
        _SPIN_MS_PER_MCYCLE.append(max(e0.elapsed_time(e1), 1e-3))
    torch.cuda._sleep(int(min(ms, 100.0) / _SPIN_MS_PER_MCYCLE[0] * 1_000_000))


def time_stages(layer, x, path, steps, warmup, dense=False):
    """Average duration (us) of each kernel of the step, HIP events on the launch stream.

    A dense MLP layer has no routing: its row layout (every token once, weight
    1) is set up once, outside the timed stages, and only the FFN passes and
    the combine are timed."""
    import torch
    from int8_weight_moe_amd import moe_combine, moe_expert_down, moe_expert_gate_up, moe_permute, moe_route
    from int8_weight_moe_amd.ops import down_workspace_size, gate_up_workspace_size, make_shape
    ex, K = layer.experts, layer.K
    T = x.shape[0]
    names = ["gate_up", "down", "combine"] if dense else ["route", "permute", "gate_up", "down", "combine"]
    h = torch.empty((T * K, ex.f), dtype=torch.bfloat16, device=x.device)
    rows = torch.empty((T * K, ex.d), dtype=torch.float32, device=x.device)
    dshape = make_shape(T, ex.d, ex.f, ex.E, K, x.dtype, ex.scale_dtype, path, ex.fmt)
    dws = torch.empty(max(down_workspace_size(dshape), 256), dtype=torch.uint8, device=x.device)
    gws = torch.empty(max(gate_up_workspace_size(dshape), 256), dtype=torch.uint8, device=x.device)
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
        moe_expert_gate_up(x, off, ss, ex, K, path=path, h=h, workspace=gws)
        ev[i + 1].record()
        moe_expert_down(h, off, ex, T, K, act=x.dtype, path=path, y_rows=rows, workspace=dws)
        ev[i + 2].record()
        moe_combine(rows, s2r, gw, x.dtype)
        ev[i + 3].record()

    n_ev = len(names) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    prewarm(lambda: step([torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]))
    for _ in range(warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(n_ev)])
    torch.cuda.synchronize()
    # The staged calls cost more host time per step than a decode step takes on
    # the GPU, so the GPU would idle between them and the idle time would count
    # in the stage after it. A spin kernel ahead of the timed steps keeps the
    # GPU busy while the host enqueues them; they then run back to back.
    gpu_lead(1.5 * steps * sum(_STAGE_HOST_MS.get(n, 0.05) for n in names))
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
def cpu_baseline(w, x_host, layer, src, experts_sampled=(0, 15), rows_fit=(32, 160)):
    """The oracle (unchanged, fp64 NumPy) on the host cores, on a bounded sample of the step.

    Timed in full: the router + top-K gate over all T tokens. Timed on a
    sample: the SwiGLU expert FFN plus the combine of a few experts at two row
    counts each (the first rows of each sampled expert's segment). The oracle's
    cost of one expert over n rows is a + b*n (a: its per-call conversion of the
    expert's int8 weights to fp64; b: the three contractions per row, linear in
    n), all experts having the same shape; a and b come from a least-squares
    fit over the sampled calls, and the step estimate is
        route(T) + sum over touched experts e of (a + b * rows_e).
    BLAS threads are pinned to the cores this process may run on.
    """
    import numpy as np
    from oracle import moe as omoe
    from oracle import quant as oquant
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limiter = None
    try:
        x64 = x_host.double().numpy()
        wr64 = layer.router_w.double().cpu().numpy()
        b64 = None if layer.bias is None else layer.bias.double().cpu().numpy()
        t_route = []
        for _ in range(3):
            t0 = time.perf_counter()
            ids, gw, _ = omoe.route(x64, wr64, b64, w.K)
            t_route.append(time.perf_counter() - t0)
        tr = statistics.median(t_route)
        flat = ids.reshape(-1)
        counts = np.bincount(flat, minlength=w.E)
        sample = [e for e in experts_sampled if e < w.E and counts[e] > 0]
        pts = []   # (rows, seconds)
        for e in sample:
            W = {}
            for k in ("gate", "up", "down"):   # load-time quantization by the oracle: not timed
                q, sc = oquant.quantize_rows(src["w_" + k][e].double().cpu().numpy(), w.scale)
                W["q_" + k], W["s_" + k] = {e: q}, {e: sc}
            tt, kk = np.nonzero(ids == e)      # the expert's slots in sorted (slot) order
            for n in rows_fit:
                n = min(n, tt.size)
                sel = np.full_like(ids, -1)
                sel[tt[:n], kk[:n]] = e
                t0 = time.perf_counter()
                o = omoe.expert_outputs(x64, sel, W, experts=[e])
                m = sel >= 0
                omoe.combine(np.where(m[..., None], o, 0.0), np.where(m, gw, 0.0))
                pts.append((n, time.perf_counter() - t0))
            del W
        A = np.array([[1.0, n] for n, _ in pts])
        a_fit, b_fit = np.linalg.lstsq(A, np.array([t for _, t in pts]), rcond=None)[0]
        touched = counts[counts > 0]
        est = tr + len(touched) * a_fit + b_fit * float(touched.sum())
    finally:
        if limiter is not None:
            limiter.unregister()
    flops = 6.0 * w.T * w.K * w.d * w.f + 2.0 * w.T * w.d * w.E
    return {"value": round(w.T / est, 2), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "dtype": "f64",
            "sample": (f"router+gate over all {w.T} tokens timed in full (median of 3); SwiGLU expert FFN + combine "
                       f"of experts {sample} timed on the first {list(rows_fit)} rows of each segment; per-expert "
                       f"cost fit as a + b*rows (a = {a_fit * 1e3:.1f} ms, b = {b_fit * 1e3:.3f} ms/row) and summed "
                       f"over the {len(touched)} touched experts' {int(touched.sum())} rows"),
            "step_ms_estimate": round(est * 1e3, 1), "route_ms": round(tr * 1e3, 1),
            "gflops": round(flops / est / 1e9, 1)}


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


def measure(layer, wl, x, bias, steps, warmup, dense, path, wfmt="int8"):
    """Step time, spread, kernel split, layer rates and dominant-kernel roofline of one workload."""
    orig_bias = layer.bias
    layer.bias = bias
    try:
        counts = touched_rows(layer, x, path)
        alg = algorithmic(wl, counts, wfmt)
        ms, wall_ms, per_step = time_forward(layer, x, path, steps, warmup, dense)
        stages = time_stages(layer, x, path, max(3, steps // 2) if wl.T * wl.K > 64 * wl.E else steps,
                             max(1, warmup // 2), dense)
    finally:
        layer.bias = orig_bias
    used = ffn_path_used(wl, path)
    dom = max(("gate_up", "down"), key=lambda k: stages[k])
    s = ms * 1e-3
    out = {"workload": wl.name, "T": wl.T, "ffn_path": used, "steps": steps, "ms_per_step": round(ms, 4),
           "wall_ms_per_step": round(wall_ms, 4), **spread(per_step),
           "tokens_per_s": round(wl.T / s, 1),
           "layer": {"algorithmic_GB": round(alg["layer_bytes"] / 1e9, 4),
                     "hbm_GBps": round(alg["layer_bytes"] / s / 1e9, 1),
                     "hbm_frac": round(alg["layer_bytes"] / s / 1e9 / HBM_PEAK_GBPS, 4),
                     "tflops": round(alg["layer_flops"] / s / 1e12, 2),
                     "mfma_frac": round(alg["layer_flops"] / s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "touched_experts": alg["touched"]},
           "kernels_us": {k: round(v, 2) for k, v in stages.items()}}
    if wfmt == "int8":
        out["roofline"] = roofline(wl, alg, stages, dom, wl.name, used == "stream")
        if used == "stream" and wl.T * wl.K <= 256 and not dense:
            out["roofline"]["note"] = ("timed as the staged moe_expert_gate_up call, which reads the permutation; "
                                       "inside moe_forward the same pass derives it from the routing ids")
    log(f"{wl.name} ({wfmt} weights): {ms:.4f} ms/step (p10 {out['p10_ms']}, p90 {out['p90_ms']}); stages (us): "
        + ", ".join(f"{k}={v:.1f}" for k, v in stages.items()))
    return out


def workload_bias(wl, dev):
    import torch
    if not wl.has_bias:
        return None
    return torch.tensor([wl.hot_bias, wl.hot_bias] + [0.0] * (wl.E - 2), device=dev)


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
    bias = workload_bias(w, dev)

    head = measure(layer, w, x, bias, args.steps, args.warmup, dense, path)
    result = {
        "metric": "MLP-layer tokens/s" if dense else "MoE-layer tokens/s",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_ms": PREWARM_MS,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "f": w.f, "E": w.E, "K": w.K,
                   "weights": f"int8 per-output-channel, {w.scale} scales", "activations": w.act,
                   "router_bias": f"+{w.hot_bias} on experts 0 and 1" if w.has_bias else "none",
                   "ffn_path": head["ffn_path"], "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "spread": {k: head[k] for k in ("p10_ms", "p50_ms", "p90_ms")},
        "wall_ms_per_step": head["wall_ms_per_step"],
        "layer": head["layer"],
        "kernels_us": head["kernels_us"],
        "quantize_ms": round(qms, 2),
    }

    # the sibling workload on the same weights (decode next to prefill, or the reverse)
    sib_x, sib_bias, sib = None, None, SIBLING.get(w.name)
    if sib and not args.no_sibling:
        ws_ = workloads.ALL_WORKLOADS[sib]
        if (ws_.d, ws_.f, ws_.E) == (w.d, w.f, w.E):
            sib_x = workloads.draw_activations(ws_).to(dev)
            sib_bias = workload_bias(ws_, dev)
            key = "decode" if ws_.T * ws_.K <= 64 * ws_.E else "prefill"
            steps = args.sibling_steps if key == "decode" else max(5, args.sibling_steps // 5)
            result[key] = measure(layer, ws_, sib_x, sib_bias, steps, max(2, args.warmup), dense, MOE_PATH_AUTO)

    if not args.no_vendor:
        wp = w if w.T * w.K > 64 * w.E else (workloads.ALL_WORKLOADS[sib] if sib else None)
        if wp is not None and wp.T * wp.K > 64 * wp.E:
            result["vendor_bf16_gemm"] = {"workload": wp.name, **vendor_gemm_reference(wp, dev)}
            log(f"vendor bf16 GEMM reference (hipBLASLt, ungrouped): {result['vendor_bf16_gemm']}")

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
            entry = {"weights": "bf16 as stored, no scales" if name == "bf16" else
                     f"fp8 e4m3 per-output-channel, {w.scale} scales"}
            c = measure(clayer, w, x, bias, args.steps, args.warmup, dense, path, wfmt=name)
            entry[w.name] = {"ms_per_step": c["ms_per_step"], "int8_speedup": round(c["ms_per_step"] / head["ms_per_step"], 3),
                             "layer_GBps": c["layer"]["hbm_GBps"], "layer_tflops": c["layer"]["tflops"],
                             "kernels_us": c["kernels_us"]}
            if sib_x is not None and not args.no_sibling:
                ws_ = workloads.ALL_WORKLOADS[sib]
                key = "decode" if ws_.T * ws_.K <= 64 * ws_.E else "prefill"
                steps = args.sibling_steps if key == "decode" else max(5, args.sibling_steps // 5)
                c2 = measure(clayer, ws_, sib_x, sib_bias, steps, max(2, args.warmup), dense, MOE_PATH_AUTO, wfmt=name)
                entry[ws_.name] = {"ms_per_step": c2["ms_per_step"],
                                   "int8_speedup": round(c2["ms_per_step"] / result[key]["ms_per_step"], 3),
                                   "layer_GBps": c2["layer"]["hbm_GBps"], "layer_tflops": c2["layer"]["tflops"],
                                   "kernels_us": c2["kernels_us"]}
            comp[name + "_weights"] = entry
            del ex, clayer
            torch.cuda.empty_cache()
        result["comparators"] = comp
    del sib_x

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {args.copy_calibration_mib} MiB device copies")
        del a, b

    if not args.no_cpu_baseline and not dense:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w, x_host, layer, src)
        log(f"cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
