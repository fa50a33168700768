"""MOE_DEBUG: the C ABI's host-side permutation checks, through the library
(and MOE_LOG, the line per FFN pass naming the schedule taken).

With MOE_DEBUG set, the calls that take a permutation from the caller check it
before anything is launched, and the calls that produce one check it after it
is computed (the check logic itself is pinned on the CPU in
test_debug_checks_host.py). Every broken input below would stay inside its
buffers even if a kernel did read it (the buffers have a spare row and the
spare entries hold valid values), and each test checks that nothing was
written.
"""
import numpy as np
import pytest
import torch

import workloads
from int8_weight_moe_amd import (MoeError, moe_combine, moe_expert_down, moe_expert_ffn, moe_expert_gate_up,
                                 moe_forward, moe_forward_noalloc, moe_mlp_forward, moe_permute)
from int8_weight_moe_amd._lib import MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED
from oracle import moe as omoe
from tests.helpers import experts_to_device, quantize_experts_oracle

pytestmark = pytest.mark.gpu

MOE_ERR_CHECK = 8


def _layer(T, d, f, E, K, seed=3):
    w = workloads.Workload("dbg", T=T, d=d, f=f, E=E, K=K, seed=seed)
    x = workloads.draw_activations(w)
    wr, _ = workloads.draw_router(w)
    W = quantize_experts_oracle(workloads.draw_expert_weights(w, "cpu"), "bf16")
    return x, wr, experts_to_device(W, torch.bfloat16)


def _expect_check(fn, text):
    with pytest.raises(MoeError) as ei:
        fn()
    assert ei.value.status == MOE_ERR_CHECK, str(ei.value)
    assert text in str(ei.value), str(ei.value)


@pytest.mark.parametrize("T,path", [(8, MOE_PATH_AUTO), (200, MOE_PATH_STREAM), (600, MOE_PATH_TILED),
                                    (5000, MOE_PATH_TILED)])
def test_checks_pass_and_change_nothing(monkeypatch, T, path):
    """Valid permutations pass every check, and the results are bitwise those of
    a run without the checks: the fused layer (the gate/up pass that derives the
    permutation from the ids for T=8, the permutation kernels otherwise, with
    the multi-workgroup ones for T=5000) and the staged calls."""
    d, f, E, K = 256, 512, 16, 2
    x, wr, ex = _layer(T, d, f, E, K)
    xg, wrg = x.cuda(), wr.cuda()
    monkeypatch.delenv("MOE_DEBUG", raising=False)
    y0, ids0, w0 = moe_forward(xg, wrg, None, ex, K, path=path)
    torch.cuda.synchronize()
    monkeypatch.setenv("MOE_DEBUG", "1")
    y1, ids1, w1 = moe_forward(xg, wrg, None, ex, K, path=path)
    off, ss, s2r = moe_permute(ids1, E)
    h = moe_expert_gate_up(xg, off, ss, ex, K, path=path)
    rows = moe_expert_down(h, off, ex, T, K, path=path)
    rows2 = moe_expert_ffn(xg, off, ss, ex, K, path=path)
    y2 = moe_combine(rows, s2r, w1, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(ids0, ids1) and torch.equal(w0, w1)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(rows, rows2)
    ref_off, ref_ss, ref_s2r = omoe.permute(ids1.cpu().numpy(), E)
    assert np.array_equal(off.cpu().numpy(), ref_off) and np.array_equal(ss.cpu().numpy(), ref_ss)
    assert np.array_equal(s2r.cpu().numpy(), ref_s2r)
    monkeypatch.setenv("MOE_DEBUG", "0")           # "0" turns the checks off
    moe_permute(ids1, E)
    torch.cuda.synchronize()


@pytest.mark.parametrize("T", [32, 5000])
def test_permute_reports_ids_outside_range(monkeypatch, T):
    """Ids outside [0, E) are left unplaced by the permutation (documented); with
    MOE_DEBUG the call reports them."""
    E, K = 16, 2
    rng = np.random.default_rng(5)
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    ids[1, 1] = E
    ids[5, 0] = -1
    idg = torch.from_numpy(ids).cuda()
    monkeypatch.delenv("MOE_DEBUG", raising=False)
    off, _, _ = moe_permute(idg, E)
    torch.cuda.synchronize()
    assert int(off[E]) == T * K - 2
    monkeypatch.setenv("MOE_DEBUG", "1")
    _expect_check(lambda: moe_permute(idg, E), "2 slots have an expert id outside [0, 16) (first: slot 3, id 16)")


def test_bad_caller_permutations_are_rejected_before_launch(monkeypatch):
    """Broken offsets, sorted slots and slot_to_row handed to the FFN and combine
    calls: MOE_ERR_CHECK, and the outputs are left as they were."""
    T, d, f, E, K = 64, 128, 256, 4, 2
    S = T * K
    x, _, ex = _layer(T, d, f, E, K, seed=9)
    rng = np.random.default_rng(2)
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    off, ss, s2r = omoe.permute(ids, E)
    x_big = torch.cat([x, x[:1]]).cuda()            # a spare token row
    xg = x_big[:T]
    monkeypatch.setenv("MOE_DEBUG", "1")

    def dev(a, spare=0):
        big = np.concatenate([a, np.full(spare, 0, dtype=np.int32)]) if spare else a
        return torch.from_numpy(np.ascontiguousarray(big, dtype=np.int32)).cuda()

    h_big = torch.full((S + 1, f), 7.0, dtype=torch.bfloat16, device="cuda")
    y_big = torch.full((S + 1, d), 7.0, dtype=torch.float32, device="cuda")
    h_ref, y_ref = h_big.clone(), y_big.clone()

    def gate_up(o, s):
        return lambda: moe_expert_gate_up(xg, o, s, ex, K, h=h_big[:S])

    def unchanged():
        torch.cuda.synchronize()
        assert torch.equal(h_big, h_ref) and torch.equal(y_big, y_ref)

    bad = off.copy(); bad[0] = 1
    _expect_check(gate_up(dev(bad), dev(ss, 1)), "expert_offsets[0] = 1")
    bad = off.copy(); bad[2] = bad[1] - 1
    _expect_check(gate_up(dev(bad), dev(ss, 1)), "expert_offsets decrease at expert 1")
    bad = off.copy(); bad[E] = S + 1
    _expect_check(gate_up(dev(bad), dev(ss, 1)), f"expert_offsets[E] = {S + 1} exceeds the {S} slots")
    s = ss.copy(); s[5] = S                          # its token row T is the spare row of x_big
    _expect_check(gate_up(dev(off), dev(s, 1)), f"sorted_slots[5] = {S} is outside [0, {S})")
    s = ss.copy(); s[7] = s[6]
    _expect_check(gate_up(dev(off), dev(s, 1)), f"slot {ss[6]} is held by two sorted rows (the second: 7)")
    unchanged()

    s = ss.copy(); s[0] = -1
    _expect_check(lambda: moe_expert_ffn(xg, dev(off), dev(s, 1), ex, K), "sorted_slots[0] = -1")
    bad = off.copy(); bad[E] = S + 1
    _expect_check(lambda: moe_expert_down(h_big[:S], dev(bad), ex, T, K, y_rows=y_big[:S]),
                  f"expert_offsets[E] = {S + 1} exceeds")
    unchanged()

    r = s2r.copy(); r[3] = S                         # row S is the spare row of y_big
    w = torch.full((T, K), 0.5, dtype=torch.float32, device="cuda")
    _expect_check(lambda: moe_combine(y_big[:S], dev(r), w, torch.bfloat16), f"slot_to_row[3] = {S} is outside")
    unchanged()
    # the valid arrays pass
    moe_expert_gate_up(xg, dev(off), dev(ss), ex, K, h=h_big[:S])
    torch.cuda.synchronize()
    assert not torch.equal(h_big[:S], h_ref[:S]) and torch.equal(h_big[S:], h_ref[S:])


def test_moe_log_names_the_schedule(monkeypatch, capfd):
    """With MOE_LOG set, one stderr line per FFN pass names the schedule: the
    stream passes of a decode batch (segments from the ids), of a larger batch
    (segments from the permutation), the tiled passes with claimed tails, and a
    dense layer whose down reduction is split with the combine folded in.
    Unset, the library writes nothing."""
    d, f, E, K = 256, 512, 16, 2
    monkeypatch.delenv("MOE_LOG", raising=False)
    x, wr, ex = _layer(600, d, f, E, K)
    xg, wrg = x.cuda(), wr.cuda()
    moe_forward(xg[:8], wrg, None, ex, K)
    torch.cuda.synchronize()
    assert "[moe]" not in capfd.readouterr().err
    monkeypatch.setenv("MOE_LOG", "1")
    moe_forward(xg[:8], wrg, None, ex, K)
    moe_forward_noalloc(xg[:200], wrg, None, ex, K, path=MOE_PATH_STREAM)
    moe_forward(xg, wrg, None, ex, K, path=MOE_PATH_TILED)
    dx, _, dex = _layer(64, d, 1024, 1, 1, seed=4)
    moe_mlp_forward(dx.cuda(), dex)
    torch.cuda.synchronize()
    lines = [l for l in capfd.readouterr().err.splitlines() if l.startswith("[moe]")]
    assert len(lines) == 8, lines
    assert lines[0].startswith("[moe] moe_forward gate/up: T=8 d=256 f=512 E=16 K=2 act=bf16 scale=bf16 weights=int8;")
    assert "stream schedule, 32-row passes, expert segments derived from the expert ids" in lines[0]
    assert "moe_forward down:" in lines[1] and "reduction inside the workgroup" in lines[1]
    assert lines[2].startswith("[moe] moe_forward_noalloc gate/up: T=200")
    assert "expert segments read from the permutation" in lines[2]
    assert "tiled schedule, the last tiles of each XCD queue claimed" in lines[4]
    assert "tiled schedule" in lines[5]
    assert lines[6].startswith("[moe] moe_mlp_forward gate/up: T=64 d=256 f=1024 E=1 K=1")
    assert "64-row passes" in lines[6]
    assert "reduction split over workgroups in 8 slices, their sum written to y" in lines[7]
