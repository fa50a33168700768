"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

Also run: one GPU's share of the Large layer under 8-way tensor parallelism
(f = 3072, workloads.SHARD_WORKLOADS).

Weights are drawn on the GPU by workloads.py and quantized by the library's
moe_quantize_rows; the layer runs through MoeLayer.forward (moe_forward, auto
schedule). What the oracle can afford at these sizes, and what is compared:
  * routing of every token (fp64 logits): ids bit-exact except near ties, gate
    weights within 1e-5;
  * the gate/up pass on EVERY routed row of EVERY expert, at a sample of each
    expert's hidden channels (the first and last channels, and one channel in
    each of many channel tiles spread over f): the oracle quantizes just those
    channels' weight rows (the quantizer works row by row) and computes
    h = silu(g) * u for them;
  * the whole expert output (y_rows, all d channels) of rows spread over the
    entire segment of each sampled expert: the first rows, one row in every
    128-row tile, the last rows (so the last partial tile), for experts chosen
    so that across the workloads every expert is compared, and at the skewed
    workload the two hot experts (every row-tile group of theirs) and experts
    late in index order; the oracle re-quantizes those experts in full, and
    their codes and scales must equal the library's bit for bit;
  * whole-token outputs y of tokens whose experts are all sampled, among them
    the highest token indices;
  * properties that hold at any size: two runs are bitwise identical, and the
    fused call equals the staged calls bitwise.
Near-tie tokens are excluded from the sampled output checks; their routing is
checked for validity.
"""
import gc
import os
import sys

import numpy as np
import pytest
import torch

import workloads
from int8_weight_moe_amd import (MoeLayer, moe_combine, moe_expert_ffn, moe_expert_gate_up, moe_permute, moe_route,
                                 quantize_experts)
from oracle import moe as omoe
from oracle import quant as oquant
from tests.helpers import assert_close_to_oracle, check_routing, np64, tiled_to_rowmajor

pytestmark = pytest.mark.gpu

# experts whose whole outputs are compared, per workload (every expert appears
# for each layer shape; the oracle re-quantizes each one in full)
FULL_EXPERTS = {
    "tiny": list(range(16)),
    "mini-decode": list(range(0, 8)), "mini-prefill": list(range(8, 16)),
    "large-decode": [2, 7, 12], "large-prefill-skewed": [0, 1, 9, 15],
    "large-decode-tp8": list(range(16)), "large-prefill-skewed-tp8": list(range(16)),
}
ROW_TILE = 128          # rows per tile of the prefill schedule
LAST_ROWS = 16          # trailing rows of each segment always compared
CHANNELS = 48           # hidden channels per expert in the gate/up check
WHOLE_TOKENS = 48       # tokens compared end to end (when that many are fully sampled)


def _say(msg):
    print(f"[workload-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", params=list(workloads.WORKLOADS) + list(workloads.SHARD_WORKLOADS))
def run(request):
    w = workloads.ALL_WORKLOADS[request.param]
    dev = torch.device("cuda:0")
    _say(f"{w.name}: drawing inputs T={w.T} d={w.d} f={w.f}")
    src = workloads.draw_expert_weights(w, dev)
    ex = quantize_experts(src["w_gate"], src["w_up"], src["w_down"], workloads.TORCH_DTYPE[w.scale])
    wr, bias = workloads.draw_router(w)
    x_host = workloads.draw_activations(w)
    layer = MoeLayer(wr.to(dev), None if bias is None else bias.to(dev), ex, w.K)
    x = x_host.to(dev)
    _say(f"{w.name}: forward")
    y, ids, gw = layer.forward(x)
    y2, ids2, gw2 = layer.forward(x)
    torch.cuda.synchronize()
    state = dict(w=w, src=src, ex=ex, wr=wr, bias=bias, x_host=x_host, x=x, layer=layer,
                 y=y, ids=ids, gw=gw, y2=y2, ids2=ids2, gw2=gw2)
    yield state
    state.clear()
    del src, ex, layer, x, y, y2
    gc.collect()
    torch.cuda.empty_cache()


def _oracle_routing(st):
    w = st["w"]
    x64 = np64(st["x_host"])
    wr64 = np64(st["wr"])
    b64 = None if st["bias"] is None else np64(st["bias"])
    logits = omoe.router_logits(x64, wr64, b64)
    return x64, wr64, b64, logits


def test_routing_all_tokens(run):
    st = run
    _, _, _, logits = _oracle_routing(st)
    flags = check_routing(st["ids"].cpu().numpy(), st["gw"].cpu().numpy(), logits, st["w"].K)
    _say(f"{st['w'].name}: routing ok, {int(flags.sum())} near-tie tokens")
    if st["w"].has_bias:
        ids = st["ids"].cpu().numpy()
        share = np.mean(np.isin(ids, [0, 1]))
        assert 0.3 < share < 0.5, share   # the skewed router sends ~40% of assignments to experts 0 and 1


def test_deterministic_and_staged_equals_fused(run):
    st = run
    assert torch.equal(st["ids"], st["ids2"]) and torch.equal(st["gw"], st["gw2"])
    assert torch.equal(st["y"].view(torch.int16), st["y2"].view(torch.int16)) if st["y"].dtype == torch.bfloat16 \
        else torch.equal(st["y"], st["y2"])
    layer, x, K = st["layer"], st["x"], st["w"].K
    ids, gw = moe_route(x, layer.router_w, layer.bias, K)
    off, ss, s2r = moe_permute(ids, layer.experts.E)
    rows = moe_expert_ffn(x, off, ss, layer.experts, K)
    y = moe_combine(rows, s2r, gw, x.dtype)
    torch.cuda.synchronize()
    assert torch.equal(ids, st["ids"]) and torch.equal(gw, st["gw"])
    if y.dtype == torch.bfloat16:
        assert torch.equal(y.view(torch.int16), st["y"].view(torch.int16))
    else:
        assert torch.equal(y, st["y"])


def _oracle_state(st):
    """Oracle routing of every token, computed once per workload."""
    if "oracle" not in st:
        w = st["w"]
        x64, wr64, b64, logits = _oracle_routing(st)
        ids_o, w_o = omoe.topk_gate(logits, w.K)
        flags = omoe.near_tie_flags(logits, w.K)
        ids_g = st["ids"].cpu().numpy()
        agree = (ids_o == ids_g) & (~flags)[:, None]      # slots compared
        st["oracle"] = dict(x64=x64, ids_o=ids_o, w_o=w_o, flags=flags, agree=agree)
    return st["oracle"]


def _staged_layout(st):
    if "layout" not in st:
        off, ss, s2r = moe_permute(st["ids"], st["layer"].experts.E)
        torch.cuda.synchronize()
        st["layout"] = (off, ss, s2r, off.cpu().numpy(), s2r.cpu().numpy())
    return st["layout"]


def _channel_sample(f: int, rng) -> np.ndarray:
    """First, last and tile-edge channels plus one random channel in each of many 128-channel tiles."""
    tiles = f // 128
    fixed = [0, 15, 16, min(127, f - 1), f - 16, f - 1]
    if tiles > 1:
        fixed += [128, f - 128]
    picks = rng.choice(tiles, size=min(tiles, CHANNELS - len(fixed)), replace=False) if tiles else []
    rand = [128 * t + int(rng.integers(0, min(128, f - 128 * t))) for t in picks]
    return np.unique(np.array(fixed + rand, dtype=np.int64).clip(0, f - 1))


def test_gate_up_every_row_sampled_channels(run):
    """h of every routed row of every expert at sampled channels, against the oracle."""
    st = run
    w, layer, x = st["w"], st["layer"], st["x"]
    o = _oracle_state(st)
    off_t, ss_t, _, off, s2r = _staged_layout(st)
    h = moe_expert_gate_up(x, off_t, ss_t, layer.experts, w.K)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1000 + len(w.name))
    flat_ids = o["ids_o"].reshape(-1)
    flat_ok = o["agree"].reshape(-1)
    worst, rows_total = 0.0, 0
    for e in range(w.E):
        slots = np.nonzero((flat_ids == e) & flat_ok)[0]
        if slots.size == 0:
            continue
        ch = _channel_sample(w.f, rng)
        q, sc = {}, {}
        for k in ("gate", "up"):
            src_rows = st["src"]["w_" + k][e][torch.from_numpy(ch).to(st["src"]["w_" + k].device)]
            q[k], sc[k] = oquant.quantize_rows(np64(src_rows), w.scale)   # row by row: exact for a subset
        ref = omoe.expert_hidden(o["x64"][slots // w.K], q["gate"], sc["gate"], q["up"], sc["up"])
        rows = torch.from_numpy(s2r[slots].astype(np.int64)).to(h.device)
        got = np64(h.index_select(0, rows)[:, torch.from_numpy(ch).to(h.device)])
        assert np.all((s2r[slots] >= off[e]) & (s2r[slots] < off[e + 1])), f"expert {e}: rows outside its segment"
        worst = max(worst, assert_close_to_oracle(got, ref, f"h (expert {e}, {slots.size} rows, {ch.size} channels)"))
        rows_total += slots.size
    del h
    _say(f"{w.name}: gate/up compared on {rows_total} rows x {CHANNELS} channels per expert (worst err/tol {worst:.3f})")
    assert rows_total == int(o["agree"].sum())


def _segment_positions(n: int, rng) -> np.ndarray:
    """Positions inside a segment of n rows: the first rows, one in every row tile, the last rows."""
    if n <= 2 * LAST_ROWS + 4:
        return np.arange(n)
    pos = [0, 1]
    for t in range((n + ROW_TILE - 1) // ROW_TILE):
        lo, hi = t * ROW_TILE, min(n, (t + 1) * ROW_TILE)
        pos.append(int(rng.integers(lo, hi)))
        pos.append(lo)                               # the first row of every tile
    pos += list(range(n - LAST_ROWS, n))
    return np.unique(np.array(pos))


def test_expert_rows_across_whole_segments(run):
    st = run
    w, layer, x = st["w"], st["layer"], st["x"]
    o = _oracle_state(st)
    ids_o, w_o, agree = o["ids_o"], o["w_o"], o["agree"]
    off_t, ss_t, _, off, s2r = _staged_layout(st)
    sample = [e for e in FULL_EXPERTS[w.name] if np.any(ids_o == e)]
    _say(f"{w.name}: oracle re-quantizes experts {sample}")
    W = {k: {} for k in ("q_gate", "s_gate", "q_up", "s_up", "q_down", "s_down")}
    for e in sample:
        for k in ("gate", "up", "down"):
            q, s = oquant.quantize_rows(np64(st["src"]["w_" + k][e]), w.scale)
            qg = tiled_to_rowmajor(getattr(st["ex"], "q_" + k)[e].cpu().numpy())
            sg = np64(getattr(st["ex"], "s_" + k)[e])
            assert np.array_equal(qg, q), f"quantized codes differ (expert {e}, {k})"
            assert np.array_equal(sg, s), f"scales differ (expert {e}, {k})"
            W["q_" + k][e], W["s_" + k][e] = q, s

    rows = moe_expert_ffn(x, off_t, ss_t, layer.experts, w.K)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2000 + len(w.name))
    T, K = w.T, w.K
    keep = np.zeros((T, K), dtype=bool)
    # rows spread over each sampled expert's whole segment (positions in the library's sorted order)
    ss = ss_t.cpu().numpy()
    for e in sample:
        seg = ss[off[e]:off[e + 1]]
        for p in _segment_positions(seg.size, rng):
            t, k = divmod(int(seg[p]), K)
            if agree[t, k]:
                keep[t, k] = True
    # whole tokens whose every expert is sampled: the highest indices, the lowest, and some in between
    full = np.nonzero(np.all(np.isin(ids_o, sample) & agree, axis=1))[0]
    if 0 < full.size <= 2 * WHOLE_TOKENS:
        tok = full
        keep[tok] = True
    elif full.size:
        third = WHOLE_TOKENS // 3
        mid = rng.choice(full, size=min(full.size, third), replace=False)
        tok = np.unique(np.concatenate([full[:third], full[-third:], mid]))
        keep[tok] = True
    else:
        tok = full
    oo = omoe.expert_outputs(o["x64"], np.where(keep, ids_o, -1), W, experts=sample)
    tt, kk = np.nonzero(keep)
    rows_g = rows.index_select(0, torch.from_numpy(s2r.reshape(T, K)[tt, kk].astype(np.int64)).to(rows.device))
    r = assert_close_to_oracle(np64(rows_g), oo[tt, kk], "y_rows (rows over whole segments)")
    top = int(s2r.reshape(T, K)[tt, kk].max())
    _say(f"{w.name}: compared {tt.size} expert rows of {len(sample)} experts (highest sorted row {top} of "
         f"{int(off[-1]) - 1}; err/tol {r:.3f})")
    for e in sample:   # every row tile of every sampled expert was reached
        seg_rows = s2r.reshape(T, K)[tt, kk]
        mine = seg_rows[(seg_rows >= off[e]) & (seg_rows < off[e + 1])] - off[e]
        n = int(off[e + 1] - off[e])
        tiles_hit = np.unique(mine // ROW_TILE)
        assert tiles_hit.size >= (n + ROW_TILE - 1) // ROW_TILE - 1, f"expert {e}: row tiles not covered"
    if tok.size:
        y_ref = omoe.combine(oo[tok], w_o[tok])
        assert_close_to_oracle(np64(st["y"][torch.from_numpy(tok).to(st["y"].device)]), y_ref, "y (sampled tokens)")
        _say(f"{w.name}: compared {tok.size} whole tokens (highest token {int(tok.max())} of {T - 1})")
    elif w.name == "tiny":
        raise AssertionError("tiny workload must compare every token")
