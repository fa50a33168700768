"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of an oracle function (on the CPU,
through monkeypatch) and checks that at least one pin test then fails. A pin
suite that passed with a dropped term, a wrong sign or a wrong rounding would
not be pinning anything.
"""
import numpy as np
import pytest

from oracle import fp8, moe, quant
import tests.test_oracle_fp8 as pf
import tests.test_oracle_moe as pm
import tests.test_oracle_quant as pq


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def _swiglu_no_up_scale(xrows, q_gate, s_gate, q_up, s_up, q_down, s_down):
    x = np.asarray(xrows, dtype=np.float64)
    g = (x @ q_gate.T.astype(np.float64)) * s_gate[None, :]
    u = x @ q_up.T.astype(np.float64)
    return ((moe.silu(g) * u) @ q_down.T.astype(np.float64)) * s_down[None, :]


def _swiglu_swapped(xrows, q_gate, s_gate, q_up, s_up, q_down, s_down):
    x = np.asarray(xrows, dtype=np.float64)
    g = (x @ q_gate.T.astype(np.float64)) * s_gate[None, :]
    u = (x @ q_up.T.astype(np.float64)) * s_up[None, :]
    return ((g * moe.silu(u)) @ q_down.T.astype(np.float64)) * s_down[None, :]


def _hidden_up_scale_from_gate(xrows, q_gate, s_gate, q_up, s_up):
    x = np.asarray(xrows, dtype=np.float64)
    g = (x @ q_gate.T.astype(np.float64)) * s_gate[None, :]
    u = (x @ q_up.T.astype(np.float64)) * s_gate[None, :]
    return moe.silu(g) * u


def _silu_wrong_sign(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(z))


def _gate_no_renorm(logits, K):
    l = np.asarray(logits, dtype=np.float64)
    ids = np.argsort(-l, axis=1, kind="stable")[:, :K].astype(np.int32)
    return ids, np.take_along_axis(moe.softmax(l), ids.astype(np.int64), 1)


def _gate_ties_high(logits, K):
    l = np.asarray(logits, dtype=np.float64)
    E = l.shape[1]
    order = (E - 1 - np.argsort(-l[:, ::-1], axis=1, kind="stable"))
    ids = order[:, :K].astype(np.int32)
    pk = np.take_along_axis(moe.softmax(l), ids.astype(np.int64), 1)
    return ids, pk / pk.sum(1, keepdims=True)


def _quant_scale_128(w, scale_dtype):
    w = np.asarray(w, dtype=np.float64)
    s = quant.round_to(np.max(np.abs(w), axis=-1) / 128.0, scale_dtype)
    safe = np.where(s > 0, s, 1.0)
    q = np.clip(np.rint(w / safe[..., None]), -127, 127).astype(np.int8)
    return q, s


def _quant_floor(w, scale_dtype):
    w = np.asarray(w, dtype=np.float64)
    s = quant.round_to(np.max(np.abs(w), axis=-1) / 127.0, scale_dtype)
    safe = np.where(s > 0, s, 1.0)
    q = np.clip(np.trunc(w / safe[..., None]), -127, 127).astype(np.int8)
    return q, s


def _quant_half_away(w, scale_dtype):
    w = np.asarray(w, dtype=np.float64)
    s = quant.round_to(np.max(np.abs(w), axis=-1) / 127.0, scale_dtype)
    safe = np.where(s > 0, s, 1.0)
    r = w / safe[..., None]
    q = np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -127, 127).astype(np.int8)
    return q, s


def _bf16_seven_bits(v):
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(m * 128.0), e - 7)


def _bf16_truncate(v):
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.trunc(m * 256.0), e - 8)


def _combine_swapped(o, w):
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)[:, ::-1]
    return sum(w[:, k, None] * o[:, k] for k in range(o.shape[1]))


def _permute_unstable(ids, E):
    off, ss, s2r = moe.__dict__["_orig_permute"](ids, E)
    ss = ss.copy()
    for e in range(E):
        ss[off[e]:off[e + 1]] = ss[off[e]:off[e + 1]][::-1]
    s2r = np.empty_like(ss)
    s2r[ss] = np.arange(ss.size)
    return off, ss, s2r


def _e4m3_truncate(v):
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    step = np.maximum(e - 4, -9)
    return np.clip(np.ldexp(np.trunc(np.ldexp(v, -step)), step), -448.0, 448.0)


def _e4m3_no_saturation(v):
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    step = np.maximum(e - 4, -9)
    return np.ldexp(np.rint(np.ldexp(v, -step)), step)


def _e4m3_fnuz_range(v):
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    step = np.maximum(e - 4, -10)
    return np.clip(np.ldexp(np.rint(np.ldexp(v, -step)), step), -240.0, 240.0)


def _e4m3_decode_bias8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef, mf = (c >> 3) & 0xF, c & 0x7
    val = sign * np.where(ef == 0, np.ldexp(mf.astype(np.float64), -10), np.ldexp(1.0 + mf / 8.0, ef - 8))
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def _fp8_scale_240(w, scale_dtype):
    w = np.asarray(w, dtype=np.float64)
    s = quant.round_to(np.max(np.abs(w), axis=-1) / 240.0, scale_dtype)
    safe = np.where(s > 0, s, 1.0)
    q = fp8.round_to_e4m3(w / safe[..., None])
    return fp8.e4m3_encode(np.where((s > 0)[..., None], q, 0.0)), s


MUTATIONS = [
    ("moe", "expert_swiglu", _swiglu_no_up_scale, [pm.test_single_expert_is_textbook_swiglu_mlp]),
    ("moe", "expert_swiglu", _swiglu_swapped, [pm.test_single_expert_is_textbook_swiglu_mlp]),
    ("moe", "silu", _silu_wrong_sign, [pm.test_single_expert_is_textbook_swiglu_mlp]),
    ("moe", "expert_hidden", _hidden_up_scale_from_gate,
     [pm.test_expert_hidden_is_textbook_gated_activation_on_any_channel_subset]),
    ("moe", "topk_gate", _gate_no_renorm, [pm.test_top2_weights_are_logistic_of_gap]),
    ("moe", "topk_gate", _gate_ties_high, [pm.test_exact_ties_go_to_lower_index]),
    ("moe", "combine", _combine_swapped, [pm.test_vectorised_layer_matches_scalar_loop]),
    ("moe", "permute", _permute_unstable, [pm.test_permute_matches_counting_sort]),
    ("quant", "quantize_rows", _quant_scale_128, [pq.test_quantize_round_trip_bound_and_range]),
    ("quant", "quantize_rows", _quant_floor, [pq.test_quantize_round_trip_bound_and_range]),
    ("quant", "quantize_rows", _quant_half_away, [pq.test_quantize_ties_go_to_even]),
    ("quant", "round_to_bf16", _bf16_seven_bits, [pq.test_round_to_bf16_matches_torch_conversion]),
    ("quant", "round_to_bf16", _bf16_truncate, [pq.test_round_to_bf16_matches_torch_conversion]),
    ("fp8", "round_to_e4m3", _e4m3_truncate, [pf.test_round_matches_torch_conversion]),
    ("fp8", "round_to_e4m3", _e4m3_no_saturation, [pf.test_round_saturates_and_ties_to_even]),
    ("fp8", "round_to_e4m3", _e4m3_fnuz_range, [pf.test_round_matches_brute_force_nearest]),
    ("fp8", "e4m3_decode", _e4m3_decode_bias8, [pf.test_decode_matches_torch_for_every_code]),
    ("fp8", "quantize_rows_fp8", _fp8_scale_240, [pf.test_quantize_fp8_absmax_lands_on_448_and_round_trip_bound]),
]


@pytest.mark.parametrize("mod,name,bad,pins", MUTATIONS, ids=[f"{m[1]}:{m[2].__name__}" for m in MUTATIONS])
def test_pins_catch_planted_mistake(monkeypatch, mod, name, bad, pins):
    target = {"moe": moe, "quant": quant, "fp8": fp8}[mod]
    monkeypatch.setitem(moe.__dict__, "_orig_permute", moe.permute)
    monkeypatch.setattr(target, name, bad)
    if mod == "quant" and name == "round_to_bf16":
        # quantize_rows reaches bf16 rounding through round_to
        monkeypatch.setattr(quant, "round_to", lambda v, dt: bad(v) if dt == "bf16" else quant.round_to_f32(v))
    assert any(_fails(p) for p in pins), f"no pin failed with {bad.__name__} planted in {mod}.{name}"
