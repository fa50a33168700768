"""GPU parity at oracle-sized shapes: every C-ABI call against the oracle.

Shapes span several tiles of both expert-FFN schedules and have ragged tails
(token counts and per-expert row counts that are not tile multiples). Inputs
are drawn by workloads.py or numpy; expected values come from the oracle only.
"""
import numpy as np
import pytest
import torch

import workloads
from int8_weight_moe_amd import (MoeError, moe_combine, moe_expert_down, moe_expert_ffn, moe_expert_gate_up, moe_forward,
                                 moe_mlp_forward, moe_pack_rows, moe_permute, moe_quantize_pack_rows, moe_quantize_rows,
                                 moe_quantize_rows_fp8, moe_route)
from int8_weight_moe_amd._lib import MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED, MOE_W_FP8, MOE_W_INT8
from oracle import moe as omoe
from oracle import quant as oquant
from tests.helpers import (assert_close_to_oracle, check_routing, experts_to_device, np64,
                           quantize_experts_oracle, rowmajor_to_tiled, tiled_to_rowmajor)

pytestmark = pytest.mark.gpu

PATHS = [MOE_PATH_STREAM, MOE_PATH_TILED]
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _case(T, d, f, E, K, act="bf16", scale="bf16", bias=None, seed=0, wscale=0.02):
    w = workloads.Workload("case", T=T, d=d, f=f, E=E, K=K, act=act, scale=scale,
                           weight_src="f32" if act == "f32" else "bf16", seed=seed)
    x = workloads.draw_activations(w)
    wr, _ = workloads.draw_router(w)
    src = workloads.draw_expert_weights(w, "cpu")
    W = quantize_experts_oracle(src, scale)
    b = None if bias is None else torch.tensor(bias, dtype=torch.float32)
    return w, x, wr, b, W


# --------------------------------------------------------------------------- quantizer
@pytest.mark.parametrize("src,scale", [("f32", "f32"), ("f32", "bf16"), ("bf16", "bf16"), ("bf16", "f32")])
def test_quantize_rows_bit_exact(src, scale):
    rng = np.random.default_rng(0)
    w = rng.standard_normal((3, 37, 320)).astype(np.float32) * np.float32(0.02)
    w[0, 3] = 0.0                                   # zero row
    w[1, 5] = np.round(w[1, 5] * 2 ** 14) / 2 ** 14  # coarse grid -> ties
    w[2, 7, :] = np.arange(320) * 2.0 ** -7 - 1.0    # dyadic row, exact ties at scale 2^-7 multiples
    wt = torch.from_numpy(w).to(TDT[src])
    q, s = moe_quantize_rows(wt.cuda(), TDT[scale])
    torch.cuda.synchronize()
    qr, sr = oquant.quantize_rows(np64(wt), scale)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(np64(s), sr)


@pytest.mark.parametrize("fmt", [MOE_W_INT8, MOE_W_FP8])
@pytest.mark.parametrize("src,scale,rows,cols", [("bf16", "bf16", 48, 320), ("f32", "f32", 16, 64),
                                                 ("bf16", "bf16", 3 * 512, 4096), ("f32", "bf16", 64, 192)])
def test_quantize_pack_rows_equals_quantize_then_pack(fmt, src, scale, rows, cols):
    """The one-pass quantizer writes the codes of the row-major quantizer straight
    into the tiled layout: equal to quantize-then-pack bit for bit, same scales;
    the int8 codes, untiled, equal the oracle's."""
    rng = np.random.default_rng(rows + cols)
    w = rng.standard_normal((rows, cols)).astype(np.float32) * np.float32(0.02)
    w[5] = 0.0                                          # a zero row
    wt = torch.from_numpy(w).to(TDT[src]).cuda()
    qt, st = moe_quantize_pack_rows(wt, TDT[scale], fmt)
    if fmt == MOE_W_INT8:
        q, s = moe_quantize_rows(wt, TDT[scale])
    else:
        q, s = moe_quantize_rows_fp8(wt, TDT[scale])
    p = moe_pack_rows(q.view(torch.int8))
    torch.cuda.synchronize()
    assert torch.equal(qt.view(torch.int8), p) and torch.equal(st, s)
    if fmt == MOE_W_INT8:
        qr, sr = oquant.quantize_rows(np64(wt), scale)
        assert np.array_equal(tiled_to_rowmajor(qt.cpu().numpy()), qr)
        assert np.array_equal(np64(st), sr)


@pytest.mark.parametrize("rows,cols", [(16, 64), (48, 320), (3 * 512, 256), (16 * 64, 4096)])
def test_pack_rows_is_the_documented_permutation(rows, cols):
    rng = np.random.default_rng(rows + cols)
    q = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    p = moe_pack_rows(torch.from_numpy(q).cuda())
    torch.cuda.synchronize()
    got = p.cpu().numpy()
    assert np.array_equal(got, rowmajor_to_tiled(q))
    assert np.array_equal(tiled_to_rowmajor(got), q)
    # spot-check the byte formula of the header directly
    flat = got.reshape(-1)
    for r, c in ((0, 0), (rows - 1, cols - 1), (17 % rows, 63), (5, 16 % cols)):
        idx = ((r // 16) * (cols // 64) + c // 64) * 1024 + 256 * ((c % 64) // 16) + 16 * (r % 16) + c % 16
        assert flat[idx] == q[r, c]


# --------------------------------------------------------------------------- router
@pytest.mark.parametrize("T,d,E,K,act,bias", [
    (64, 256, 16, 2, "f32", None),          # tiny workload shape
    (1, 512, 16, 2, "bf16", None),
    (77, 1024, 16, 2, "bf16", "hot"),
    (300, 256, 4, 1, "bf16", None),
    (50, 192, 40, 3, "f32", "hot"),
    (33, 128, 64, 8, "bf16", None),
    (20, 64, 1, 1, "bf16", None),
])
def test_route_matches_oracle(T, d, E, K, act, bias):
    w = workloads.Workload("r", T=T, d=d, f=64, E=E, K=K, act=act, seed=3)
    x = workloads.draw_activations(w)
    wr, _ = workloads.draw_router(w)
    b = None
    if bias == "hot":
        b = torch.zeros(E, dtype=torch.float32)
        b[0] = 2.0
        if E > 1:
            b[1] = 2.0
    ids, gw = moe_route(x.cuda(), wr.cuda(), None if b is None else b.cuda(), K)
    torch.cuda.synchronize()
    logits = omoe.router_logits(np64(x), np64(wr), None if b is None else np64(b))
    check_routing(ids.cpu().numpy(), gw.cpu().numpy(), logits, K)


def test_route_does_not_depend_on_the_batch():
    """Small batches (<= 64 tokens) are scored one token per workgroup, larger ones
    sixteen per workgroup: a token's ids and weights must be the same bit for bit."""
    w = workloads.Workload("rb", T=100, d=1024, f=64, E=16, K=2, act="bf16", seed=9)
    x = workloads.draw_activations(w).cuda()
    wr = workloads.draw_router(w)[0].cuda()
    ids, gw = moe_route(x, wr, None, 2)
    ids_a, gw_a = moe_route(x[:64].contiguous(), wr, None, 2)
    ids_b, gw_b = moe_route(x[64:].contiguous(), wr, None, 2)
    torch.cuda.synchronize()
    assert torch.equal(ids, torch.cat([ids_a, ids_b])) and torch.equal(gw, torch.cat([gw_a, gw_b]))


def test_route_exact_ties_go_to_lower_index():
    T, d, E = 16, 128, 8
    x = torch.randn(T, d, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    wr = torch.randn(E, d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16) * 0.05
    wr[5] = wr[2]          # experts 2 and 5 have identical logits
    wr[6] = wr[2]
    b = torch.zeros(E)
    b[2] = b[5] = b[6] = 50.0   # ... and they are the top three
    ids, gw = moe_route(x.cuda(), wr.cuda(), b.cuda(), 2)
    torch.cuda.synchronize()
    assert ids.cpu().tolist() == [[2, 5]] * T
    assert torch.all(gw.cpu() == 0.5)


# --------------------------------------------------------------------------- permute
@pytest.mark.parametrize("T,K,E,kind", [
    (1, 2, 16, "rand"), (64, 2, 16, "rand"), (1000, 2, 16, "hot"), (4096, 2, 16, "one"),
    (333, 3, 5, "rand"), (16384, 2, 16, "hot"), (70, 1, 64, "rand"), (7, 8, 8, "perm"),
    (20001, 2, 16, "rand"),   # 40002 slots: several 8-chunk batches per wave and a ragged last one
])
def test_permute_bit_exact(T, K, E, kind):
    rng = np.random.default_rng(T + K + E)
    if kind == "rand":
        ids = rng.integers(0, E, size=(T, K))
    elif kind == "hot":
        ids = np.where(rng.random((T, K)) < 0.4, rng.integers(0, 2, size=(T, K)), rng.integers(0, E, size=(T, K)))
    elif kind == "one":
        ids = np.full((T, K), E - 1)
    else:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    ids = ids.astype(np.int32)
    off, ss, s2r = moe_permute(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    ro, rs, rr = omoe.permute(ids, E)
    assert np.array_equal(off.cpu().numpy(), ro)
    assert np.array_equal(ss.cpu().numpy(), rs)
    assert np.array_equal(s2r.cpu().numpy(), rr)


@pytest.mark.parametrize("T,K,E", [(6000, 2, 16), (9000, 3, 64)])
def test_permute_many_slots_out_of_range_ids_are_not_placed(T, K, E):
    """The multi-workgroup permutation (many slots) with ids outside [0, E): the
    valid slots keep the order of a stable sort, invalid ones map to -1, and the
    sorted rows past the valid ones hold -1."""
    rng = np.random.default_rng(T)
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    bad = rng.random((T, K)) < 0.01
    ids[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, E)
    off, ss, s2r = moe_permute(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    n = int(valid.sum())
    order = np.nonzero(valid)[0][np.argsort(flat[valid], kind="stable")]
    ro, rs, rr = omoe.permute(flat[valid].reshape(-1, 1), E)
    assert np.array_equal(off.cpu().numpy(), ro)
    ss_h, s2r_h = ss.cpu().numpy(), s2r.cpu().numpy()
    assert np.array_equal(ss_h[:n], order) and np.all(ss_h[n:] == -1)
    assert np.all(s2r_h[~valid] == -1)
    assert np.array_equal(s2r_h[order], np.arange(n))


def test_permute_out_of_range_ids_are_not_placed():
    ids = np.array([[0, 3], [16, 1], [2, -1]], dtype=np.int32)
    off, ss, s2r = moe_permute(torch.from_numpy(ids).cuda(), 16)
    torch.cuda.synchronize()
    s2r = s2r.cpu().numpy()
    assert off.cpu().numpy()[-1] == 4
    assert s2r[2] == -1 and s2r[5] == -1
    assert ss.cpu().numpy()[4:].tolist() == [-1, -1]
    valid = [0, 1, 3, 4]
    assert sorted(s2r[valid].tolist()) == [0, 1, 2, 3]


# --------------------------------------------------------------------------- expert FFN
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T,d,f,E,K,act,scale,routing", [
    (64, 256, 512, 16, 2, "f32", "f32", "router"),     # the tiny workload
    (200, 384, 640, 16, 2, "bf16", "bf16", "router"),  # ragged rows per expert
    (600, 256, 384, 4, 2, "bf16", "bf16", "skew"),     # several row tiles per expert, ragged tail
    (9, 128, 192, 16, 2, "bf16", "bf16", "router"),    # most experts empty
    (150, 192, 256, 8, 1, "bf16", "f32", "one"),        # every row on one expert
])
def test_expert_ffn_matches_oracle(path, T, d, f, E, K, act, scale, routing):
    w, x, wr, _, W = _case(T, d, f, E, K, act, scale, seed=7)
    rng = np.random.default_rng(11)
    if routing == "router":
        ids, _ = omoe.topk_gate(omoe.router_logits(np64(x), np64(wr)), K)
    elif routing == "skew":
        ids = np.stack([rng.choice(E, size=K, replace=False, p=[0.55, 0.25, 0.15, 0.05]) for _ in range(T)])
    else:
        ids = np.zeros((T, K), dtype=np.int32) + 3
    ids = ids.astype(np.int32)
    off, ss, s2r = omoe.permute(ids, E)
    ex = experts_to_device(W, TDT[scale])
    y_rows = moe_expert_ffn(x.cuda(), torch.from_numpy(off).cuda(), torch.from_numpy(ss).cuda(), ex, K, path=path)
    torch.cuda.synchronize()
    o = omoe.expert_outputs(np64(x), ids, W)               # [T, K, d] per slot
    ref_rows = o.reshape(T * K, -1)[ss]                    # sorted-row order
    assert_close_to_oracle(np64(y_rows), ref_rows, "y_rows")


@pytest.mark.parametrize("path", [MOE_PATH_AUTO, MOE_PATH_TILED])
def test_long_and_short_experts_in_one_launch(path):
    """One expert with more than 24 row tiles of 128 rows (its gate/up row tiles are
    visited in groups of up to 16) in the same launch as experts with fewer (groups
    of up to 8), every segment with a ragged last tile, and ragged channel tiles
    (f = 320: 2.5 gate/up channel tiles; d = 192: three quarters of a down tile).
    Every row of y_rows and every token of y against the oracle."""
    T, d, f, E, K = 4000, 192, 320, 4, 2
    w, x, wr, b, W = _case(T, d, f, E, K, "bf16", "bf16", bias=[8.0, 0.0, 0.0, 0.0], seed=21)
    ex = experts_to_device(W, torch.bfloat16)
    xg, wrg, bg = x.cuda(), wr.cuda(), b.cuda()
    y, ids, gw = moe_forward(xg, wrg, bg, ex, K, path=path)
    off, ss, s2r = moe_permute(ids, E)
    rows = moe_expert_ffn(xg, off, ss, ex, K, path=path)
    torch.cuda.synchronize()
    ids_g = ids.cpu().numpy()
    counts = np.bincount(ids_g.reshape(-1), minlength=E)
    assert counts[0] >= 24 * 128 and np.all(counts[1:] < 24 * 128) and np.all(counts[1:] >= 128), counts
    assert np.all(counts % 128 != 0), counts
    x64, wr64, b64 = np64(x), np64(wr), np64(b)
    check_routing(ids_g, gw.cpu().numpy(), omoe.router_logits(x64, wr64, b64), K)
    o = omoe.expert_outputs(x64, ids_g, W)
    assert_close_to_oracle(np64(rows), o.reshape(T * K, -1)[ss.cpu().numpy()], "y_rows (every row)")
    ref = omoe.moe_forward(x64, wr64, b64, W, K, ids=ids_g)["y"]
    assert_close_to_oracle(np64(y), ref, "y (every token)")


@pytest.mark.parametrize("T,d,f,E,K,bias", [
    (4000, 192, 320, 4, 2, [8.0, 0.0, 0.0, 0.0]),    # one long expert, short ones, ragged tiles
    (8000, 128, 1024, 8, 2, None),                   # more tiles than the GPU holds at once
    (600, 256, 384, 16, 2, None),
])
def test_tile_claims_equal_static_order_bitwise(T, d, f, E, K, bias):
    """The tiled passes with tile claim words (the tails of the XCD queues are
    claimed with atomics) and without (every tile fixed by the workgroup id)
    compute every tile the same way: h and y_rows are identical bit for bit,
    also twice in a row on the same claim words, and match the oracle. The
    second shape has more tiles than the GPU holds at once, so tails are
    claimed across XCDs."""
    w, x, wr, b, W = _case(T, d, f, E, K, "bf16", "bf16", bias=bias, seed=31)
    ex = experts_to_device(W, torch.bfloat16)
    xg = x.cuda()
    ids, _ = moe_route(xg, wr.cuda(), None if b is None else b.cuda(), K)
    off, ss, s2r = moe_permute(ids, E)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    h = moe_expert_gate_up(xg, off, ss, ex, K, path=MOE_PATH_TILED, workspace=ws)
    h_sta = moe_expert_gate_up(xg, off, ss, ex, K, path=MOE_PATH_TILED, use_workspace=False)
    h2 = moe_expert_gate_up(xg, off, ss, ex, K, path=MOE_PATH_TILED, workspace=ws)   # claim words reused: cleared by the pass
    r_dyn = moe_expert_down(h, off, ex, T, K, path=MOE_PATH_TILED, workspace=ws)
    r_sta = moe_expert_down(h, off, ex, T, K, path=MOE_PATH_TILED, split_workspace=False)
    r_dyn2 = moe_expert_down(h, off, ex, T, K, path=MOE_PATH_TILED, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h_sta.view(torch.int16)) and torch.equal(h.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(r_dyn, r_sta) and torch.equal(r_dyn, r_dyn2)
    ids_h = ids.cpu().numpy()
    o = omoe.expert_outputs(np64(x), ids_h, W)
    assert_close_to_oracle(np64(r_dyn), o.reshape(T * K, -1)[ss.cpu().numpy()], "y_rows with tile claims")
    del h


def test_tiled_register_staged_bf16_past_32bit_offsets():
    """bf16 activations whose h needs byte offsets of 2^32 and more run on the
    register-staged tiled kernel (the direct-to-LDS kernel addresses with 32-bit
    offsets): h = 16384 rows x 131072 channels x 2 bytes = 4 GiB exactly.
    Sampled rows spread over every expert's segment, among them the last rows of
    h, and sampled whole tokens, against the oracle."""
    T, d, f, E, K = 8192, 64, 131072, 16, 2
    w, x, wr, b, W = _case(T, d, f, E, K, "bf16", "bf16", seed=23)
    ex = experts_to_device(W, torch.bfloat16)
    xg, wrg = x.cuda(), wr.cuda()
    y, ids, gw = moe_forward(xg, wrg, None, ex, K)
    off, ss, s2r = moe_permute(ids, E)
    rows = moe_expert_ffn(xg, off, ss, ex, K)
    torch.cuda.synchronize()
    ids_g = ids.cpu().numpy()
    x64, wr64 = np64(x), np64(wr)
    logits = omoe.router_logits(x64, wr64)
    flags = check_routing(ids_g, gw.cpu().numpy(), logits, K)
    off_h, ss_h = off.cpu().numpy(), ss.cpu().numpy()
    assert int(off_h[-1]) * f * 2 >= 2 ** 32
    rng = np.random.default_rng(3)
    pick = []
    for e in range(E):
        n = off_h[e + 1] - off_h[e]
        if n:
            pick += [off_h[e], off_h[e + 1] - 1] + list(off_h[e] + rng.integers(0, n, size=6))
    pick += list(range(off_h[-1] - 8, off_h[-1]))           # the highest rows of h
    pick = np.unique(np.array(pick))
    slots = ss_h[pick]
    keep = np.zeros((T, K), dtype=bool)
    keep.reshape(-1)[slots] = True
    keep &= ~flags[:, None]
    tok = np.nonzero(~flags)[0][-16:]                        # the last tokens, whole
    keep[tok] = True
    o = omoe.expert_outputs(x64, np.where(keep, ids_g, -1), W, experts=range(E))
    tt, kk = np.nonzero(keep)
    r_idx = s2r.cpu().numpy().reshape(T, K)[tt, kk]
    assert_close_to_oracle(np64(rows[torch.from_numpy(r_idx.astype(np.int64)).cuda()]), o[tt, kk], "y_rows (sampled)")
    ref_y = omoe.combine(o[tok], omoe.topk_gate(logits, K)[1][tok])
    assert_close_to_oracle(np64(y[torch.from_numpy(tok).cuda()]), ref_y, "y (last tokens)")


# --------------------------------------------------------------------------- combine
@pytest.mark.parametrize("T,d,K,act", [(1, 64, 2, "bf16"), (129, 320, 2, "f32"), (40, 128, 5, "bf16")])
def test_combine_matches_oracle(T, d, K, act):
    rng = np.random.default_rng(5)
    E = 8
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    off, ss, s2r = omoe.permute(ids, E)
    rows = rng.standard_normal((T * K, d)).astype(np.float32)
    gw = rng.random((T, K)).astype(np.float32)
    gw /= gw.sum(axis=1, keepdims=True)
    y = moe_combine(torch.from_numpy(rows).cuda(), torch.from_numpy(s2r).cuda(), torch.from_numpy(gw).cuda(),
                    TDT[act])
    torch.cuda.synchronize()
    o = rows.astype(np.float64)[s2r].reshape(T, K, d)
    ref = omoe.combine(o, gw)
    got = np64(y)
    # fp32 accumulation of K terms, then the output rounding of the dtype
    rel = 2.0 ** -8 if act == "bf16" else 1e-6
    assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-6 * np.abs(ref).max())


# --------------------------------------------------------------------------- whole layer
@pytest.mark.parametrize("path", [MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED])
@pytest.mark.parametrize("T,d,f,E,K,act,scale,bias", [
    (64, 256, 512, 16, 2, "f32", "f32", None),       # tiny workload
    (1, 256, 512, 16, 2, "bf16", "bf16", None),      # a single token
    (257, 256, 320, 16, 2, "bf16", "bf16", [2.0, 2.0] + [0.0] * 14),  # skewed router, ragged
    (40, 128, 192, 8, 8, "bf16", "bf16", None),      # K = E: dense mixture
    (33, 192, 256, 1, 1, "bf16", "bf16", None),      # E = K = 1: dense int8 MLP
    (100, 128, 128, 16, 2, "bf16", "bf16", [0.0] * 5 + [100.0] + [0.0] * 10),  # hot expert 5 in every token
    (50, 128, 128, 64, 8, "bf16", "bf16", None),     # the largest E and K
    (300, 128, 2048, 16, 2, "bf16", "bf16", None),   # 37 rows per expert: shared-activation gate/up, 4 waves
    (300, 128, 1536, 16, 2, "bf16", "bf16", None),   # the same with 3 items per workgroup, reductions cut in two
    (600, 128, 1536, 16, 2, "bf16", "bf16", None),   # ... and more than 64 rows per expert: several passes
    (300, 192, 1536, 16, 2, "bf16", "bf16", None),   # 3 items per workgroup, no cut (an odd number of steps)
    (5, 65536, 64, 2, 1, "bf16", "bf16", None),      # the largest d
    (3, 64, 131072, 2, 2, "bf16", "f32", None),      # the largest f
])
def test_forward_matches_oracle(path, T, d, f, E, K, act, scale, bias):
    w, x, wr, b, W = _case(T, d, f, E, K, act, scale, bias=bias, seed=9)
    ex = experts_to_device(W, TDT[scale])
    y, ids, gw = moe_forward(x.cuda(), wr.cuda(), None if b is None else b.cuda(), ex, K, path=path)
    torch.cuda.synchronize()
    x64, wr64 = np64(x), np64(wr)
    b64 = None if b is None else np64(b)
    logits = omoe.router_logits(x64, wr64, b64)
    ids_g = ids.cpu().numpy()
    check_routing(ids_g, gw.cpu().numpy(), logits, K)
    ref = omoe.moe_forward(x64, wr64, b64, W, K, ids=ids_g)["y"]
    assert_close_to_oracle(np64(y), ref, "y")
    if K == E:
        assert_close_to_oracle(np64(y), omoe.dense_mixture(x64, wr64, b64, W), "y vs dense mixture")


@pytest.mark.parametrize("path", PATHS)
def test_forward_equals_staged_calls_bitwise(path):
    w, x, wr, b, W = _case(300, 256, 384, 16, 2, "bf16", "bf16", bias=[1.0] + [0.0] * 15, seed=4)
    ex = experts_to_device(W, torch.bfloat16)
    xg, wrg, bg = x.cuda(), wr.cuda(), b.cuda()
    y, ids, gw = moe_forward(xg, wrg, bg, ex, 2, path=path)
    ids2, gw2 = moe_route(xg, wrg, bg, 2)
    off, ss, s2r = moe_permute(ids2, 16)
    rows = moe_expert_ffn(xg, off, ss, ex, 2, path=path)
    y2 = moe_combine(rows, s2r, gw2, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(gw, gw2)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("T,d,f,E,K,act", [
    (1, 128, 192, 16, 2, "bf16"), (32, 256, 384, 16, 2, "bf16"), (64, 128, 128, 64, 1, "bf16"),
    (8, 128, 256, 8, 8, "bf16"), (20, 192, 256, 1, 1, "bf16"), (32, 256, 512, 16, 2, "f32"),
    (21, 128, 192, 5, 3, "bf16"), (64, 256, 384, 16, 2, "bf16"), (100, 128, 256, 16, 2, "bf16"),
    (256, 128, 192, 8, 1, "bf16"), (85, 128, 128, 64, 3, "bf16"),
])
def test_forward_small_batch_equals_staged(T, d, f, E, K, act):
    """At most 256 slots (and at most 32 per expert on average): moe_forward lets
    the gate/up pass derive the permutation from the expert ids (no permutation
    launch); it must equal the staged calls, which use moe_permute, bit for bit,
    and match the oracle. Shapes span one to four 64-slot chunks."""
    scale = act
    w, x, wr, b, W = _case(T, d, f, E, K, act, scale, bias=[1.5] + [0.0] * (E - 1) if E > 1 else None, seed=T + E)
    ex = experts_to_device(W, TDT[scale])
    xg, wrg = x.cuda(), wr.cuda()
    bg = None if b is None else b.cuda()
    y, ids, gw = moe_forward(xg, wrg, bg, ex, K, path=MOE_PATH_STREAM)
    y_auto, _, _ = moe_forward(xg, wrg, bg, ex, K)
    ids2, gw2 = moe_route(xg, wrg, bg, K)
    off, ss, s2r = moe_permute(ids2, E)
    rows = moe_expert_ffn(xg, off, ss, ex, K, path=MOE_PATH_STREAM)
    y2 = moe_combine(rows, s2r, gw2, TDT[act])
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(gw, gw2)
    assert torch.equal(y, y2) and torch.equal(y, y_auto)
    logits = omoe.router_logits(np64(x), np64(wr), None if b is None else np64(b))
    check_routing(ids.cpu().numpy(), gw.cpu().numpy(), logits, K)
    ref = omoe.moe_forward(np64(x), np64(wr), None if b is None else np64(b), W, K, ids=ids.cpu().numpy())
    assert_close_to_oracle(np64(y), ref["y"], f"small batch T={T} E={E} K={K} {act}")


@pytest.mark.parametrize("path", PATHS)
def test_forward_degenerate_inputs(path):
    """Degenerate cases of the method: an expert whose weights are all zero (scale 0,
    codes 0), a down matrix row that is zero, a token that is all zeros (its router
    logits are the bias: ties go to the lowest indices), and a token scaled by 100."""
    T, d, f, E, K = 150, 256, 384, 8, 2
    w = workloads.Workload("degen", T=T, d=d, f=f, E=E, K=K, act="bf16", scale="bf16", weight_src="bf16", seed=17)
    x = workloads.draw_activations(w)
    wr, _ = workloads.draw_router(w)
    src = workloads.draw_expert_weights(w, "cpu")
    for k in ("w_gate", "w_up", "w_down"):
        src[k][3] = 0.0                 # expert 3: all zero
    src["w_down"][5, 7] = 0.0           # one output channel of expert 5: zero row
    x[4] = 0.0
    x[9] = (x[9].float() * 100.0).to(torch.bfloat16)
    b = torch.zeros(E)
    b[3] = 3.0                          # route plenty of tokens to the zero expert
    W = quantize_experts_oracle(src, "bf16")
    assert np.all(W["s_gate"][3] == 0) and np.all(W["q_gate"][3] == 0)
    ex = experts_to_device(W, torch.bfloat16)
    y, ids, gw = moe_forward(x.cuda(), wr.cuda(), b.cuda(), ex, K, path=path)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    assert ids_h[4].tolist() == [3, 0]   # zero token: logits = bias, expert 3 first, then the lowest index
    logits = omoe.router_logits(np64(x), np64(wr), np64(b))
    check_routing(ids_h, gw.cpu().numpy(), logits, K)
    ref = omoe.moe_forward(np64(x), np64(wr), np64(b), W, K, ids=ids_h)
    assert_close_to_oracle(np64(y), ref["y"], f"degenerate inputs path={path}")
    assert torch.all(y[4] == 0)          # the zero token's output is exactly zero


@pytest.mark.parametrize("path", PATHS)
def test_forward_deterministic_and_token_permutation_equivariant(path):
    w, x, wr, b, W = _case(192, 256, 256, 16, 2, "bf16", "bf16", seed=6)
    ex = experts_to_device(W, torch.bfloat16)
    xg, wrg = x.cuda(), wr.cuda()
    y1, i1, g1 = moe_forward(xg, wrg, None, ex, 2, path=path)
    y2, i2, g2 = moe_forward(xg, wrg, None, ex, 2, path=path)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(192)).cuda()
    y3, i3, g3 = moe_forward(xg[perm].contiguous(), wrg, None, ex, 2, path=path)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(i3, i1[perm]) and torch.equal(g3, g1[perm])
    assert torch.equal(y3.view(torch.int16), y1[perm].view(torch.int16))


def test_library_errors_raise():
    x = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda")   # d not a multiple of 64
    wr = torch.zeros((16, 100), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MoeError):
        moe_route(x, wr, None, 2)


@pytest.mark.parametrize("path", [MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED])
def test_empty_batch(path):
    """T = 0 through every call: empty outputs, nothing launched, no error."""
    w, x, wr, _, W = _case(4, 128, 192, 8, 2, seed=2)
    ex = experts_to_device(W, TDT["bf16"])
    x0 = x[:0].cuda()
    y, ids, gw = moe_forward(x0, wr.cuda(), None, ex, 2, path=path)
    assert y.shape == (0, 128) and ids.shape == (0, 2) and gw.shape == (0, 2)
    ids, gw = moe_route(x0, wr.cuda(), None, 2)
    off, ss, s2r = moe_permute(ids, 8)
    rows = moe_expert_ffn(x0, off, ss, ex, 2, path=path)
    y2 = moe_combine(rows, s2r, gw, torch.bfloat16)
    torch.cuda.synchronize()
    assert rows.shape == (0, 128) and y2.shape == (0, 128)
    _, _, _, _, W1 = _case(4, 128, 192, 1, 1, seed=2)
    y3 = moe_mlp_forward(x0, experts_to_device(W1, TDT["bf16"]), path=path)
    torch.cuda.synchronize()
    assert y3.shape == (0, 128)
