"""Host-side checks of bench.py (no GPU): the algorithmic byte and flop
counts the roofline divides by, the roofline record, the counter lookup and
the one-GPU guard.
"""
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_counts_mini_decode():
    w = workloads.MINI_DECODE
    counts = [4] * 16                               # every expert touched, 64 rows in all
    a = bench.algorithmic(w, counts)
    d, f, S = 4096, 14336, 64
    # int8 weights of 16 experts plus bf16 scales, x read once, h written
    assert a["gate_up_bytes"] == 16 * (2 * d * f + 2 * f * 2) + 32 * d * 2 + S * f * 2
    assert a["down_bytes"] == 16 * (d * f + d * 2) + S * f * 2 + S * d * 4
    assert a["gate_up_flops"] == 4.0 * S * d * f
    assert a["layer_flops"] == 6.0 * S * d * f
    assert a["touched"] == 16


def test_algorithmic_counts_weight_encodings():
    w = workloads.LARGE_DECODE
    counts = [0] * 14 + [64, 64]                    # two touched experts
    i8 = bench.algorithmic(w, counts, "int8")
    f8 = bench.algorithmic(w, counts, "fp8")
    b16 = bench.algorithmic(w, counts, "bf16")
    assert i8 == f8                                 # same bytes: one byte per weight plus scales
    d, f = 8192, 24576
    assert b16["gate_up_bytes"] - i8["gate_up_bytes"] == 2 * (2 * d * f) - 2 * (2 * f * 2)
    assert i8["touched"] == 2


def test_roofline_records():
    w = workloads.MINI_DECODE
    a = bench.algorithmic(w, [4] * 16)
    r = bench.roofline(w, a, {"gate_up": 300.0, "down": 150.0}, "gate_up", "no-such-workload", True)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(a["gate_up_bytes"] / 300e-6 / 1e9, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, rel=1e-3)
    assert r["traffic"] is None                     # no counter file for this name
    p = bench.roofline(w, a, {"gate_up": 3000.0, "down": 1500.0}, "gate_up", "no-such-workload", False)
    assert p["bound"] == "mfma" and p["unit"] == "TFLOP/s" and p["peak"] == 2500.0
    assert p["achieved"] == pytest.approx(a["gate_up_flops"] / 3000e-6 / 1e12, abs=0.05)   # rounded to 0.1


def test_counter_lookup_follows_the_kernel_code(tmp_path, monkeypatch):
    h = bench.kernel_hash()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_gate_up_wl.txt").write_text(f"# note\nhbm_bytes_per_launch=123\nkernel_source_hash={h}\n")
    (prof / "traffic_gate_up_old.txt").write_text("hbm_bytes_per_launch=123\nkernel_source_hash=0000\n")
    csrc = tmp_path / "int8_weight_moe_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("ffn_stream.hip", "ffn_tiled.hip", "device_common.h"):
        (csrc / f).write_text(open(os.path.join(ROOT, "int8_weight_moe_amd", "csrc", f)).read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("wl", "gate_up") == 123.0
    assert bench.measured_traffic("old", "gate_up") is None          # stale counters are not reported
    assert bench.measured_traffic("missing", "gate_up") is None
    # a comment edit keeps the key, a code edit changes it
    with open(csrc / "ffn_tiled.hip", "a") as fh:
        fh.write("\n// a new comment\n")
    assert bench.kernel_hash() == h
    with open(csrc / "ffn_tiled.hip", "a") as fh:
        fh.write("\nint extra_symbol;\n")
    assert bench.kernel_hash() != h
    code = "int a; // note\n/* block\n comment */ int  b;"
    assert bench._code_only(code) == bench._code_only("int a;\nint b;")
    assert bench._code_only(code) != bench._code_only("int a; int c;")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_spread_quantiles():
    s = bench.spread([float(i) for i in range(1, 12)])     # 1..11
    assert s["p50_ms"] == 6.0 and s["p10_ms"] == 2.0 and s["p90_ms"] == 10.0


def test_default_workload_is_the_largest_single_gpu_config(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.workload == "large-prefill-skewed" and a.gpus == 1
    assert bench.SIBLING["large-prefill-skewed"] == "large-decode"
    assert bench.SIBLING["large-decode"] == "large-prefill-skewed"


def test_cpu_baseline_fit_on_a_small_workload():
    """The oracle baseline runs on the host: every field present, cores from the affinity mask."""
    import types
    w = workloads.TINY.with_(T=96)
    x = workloads.draw_activations(w)
    wr, bias = workloads.draw_router(w)
    src = workloads.draw_expert_weights(w, "cpu")
    layer = types.SimpleNamespace(router_w=wr, bias=bias)
    r = bench.cpu_baseline(w, x, layer, src, experts_sampled=(0, 3), rows_fit=(2, 8))
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["dtype"] == "f64"
    assert r["cores"] == len(os.sched_getaffinity(0))
    assert r["value"] > 0 and r["step_ms_estimate"] > 0 and r["gflops"] > 0
    assert "a + b*rows" in r["sample"]
