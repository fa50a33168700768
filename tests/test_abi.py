"""Host-side checks of the C ABI (no GPU needed: nothing here launches a kernel).

  * libmoe_int8.so loads and exports every function include/moe_int8.h declares;
  * the header's enums agree with the binding's constants;
  * argument validation returns the documented status before any launch
    (null and misaligned pointers, bad shapes and dtypes, small workspace);
  * workspace sizes follow the documented layout;
  * T = 0 is accepted and enqueues nothing.
"""
import ctypes
import os
import re

import pytest

from int8_weight_moe_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_int8.h")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name, val in (("MOE_OK", 0), ("MOE_ERR_NULL", 1), ("MOE_ERR_SHAPE", 2), ("MOE_ERR_DTYPE", 3),
                      ("MOE_ERR_ALIGN", 4), ("MOE_ERR_WORKSPACE", 5), ("MOE_ERR_UNSUPPORTED", 6),
                      ("MOE_ERR_HIP", 7), ("MOE_F32", 0), ("MOE_BF16", 1), ("MOE_PATH_AUTO", 0),
                      ("MOE_PATH_STREAM", 1), ("MOE_PATH_TILED", 2), ("MOE_W_INT8", 0), ("MOE_W_BF16", 1),
                      ("MOE_W_FP8", 2)):
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name
    assert ctypes.sizeof(_lib.MoeShape) == 36
    assert re.search(r"#define MOE_ABI_VERSION\s+%d\b" % _lib.ABI_VERSION, text)


def test_status_strings(lib):
    for st in range(8):
        assert lib.moe_status_str(st)
    assert lib.moe_abi_version() == _lib.ABI_VERSION


def _shape(**kw):
    base = dict(T=32, d=256, f=512, E=16, K=2, act_dtype=1, scale_dtype=1, ffn_path=0)
    base.update(kw)
    return _lib.MoeShape(**base)


# fake but 256-aligned "device" addresses: validation never dereferences them
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), 2), (dict(d=100), 2), (dict(d=0), 2), (dict(f=96), 2), (dict(E=0), 2), (dict(E=65), 2),
    (dict(K=0), 2), (dict(K=17), 2), (dict(E=4, K=5), 2), (dict(K=9, E=16), 2), (dict(act_dtype=5), 3),
    (dict(scale_dtype=-1), 3), (dict(ffn_path=3), 2), (dict(weight_fmt=3), 3), (dict(weight_fmt=-1), 3),
])
def test_shape_validation(lib, kw, status):
    n = ctypes.c_size_t(0)
    s = _shape(**kw)
    assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == status
    assert lib.moe_last_error()
    assert lib.moe_route(ctypes.byref(s), A, A, None, A, A, None) == status


def test_null_and_alignment(lib):
    s = _shape()
    assert lib.moe_route(None, A, A, None, A, A, None) == 1
    assert lib.moe_route(ctypes.byref(s), None, A, None, A, A, None) == 1
    assert b"x is NULL" in lib.moe_last_error()
    assert lib.moe_route(ctypes.byref(s), MIS, A, None, A, A, None) == 4
    assert lib.moe_route(ctypes.byref(s), A, A, MIS, A, A, None) == 4
    assert lib.moe_permute(ctypes.byref(s), A, None, A, A, None) == 1
    assert lib.moe_combine(ctypes.byref(s), A, A, A, MIS, None) == 4
    args = [A] * 10
    assert lib.moe_expert_ffn(ctypes.byref(s), *args, None, ctypes.c_size_t(1 << 30), None) == 1
    assert lib.moe_forward(ctypes.byref(s), A, A, None, A, A, A, A, A, MIS, A, None, None, A,
                           ctypes.c_size_t(1 << 30), None) == 4


def test_workspace_checks(lib):
    s = _shape(T=64)
    need = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(need)) == 0
    S = 64 * 2
    r = lambda v: (v + 255) // 256 * 256
    assert need.value == 4 * r(S * 4) + r(17 * 4) + r(S * 512 * 2) + r(S * 256 * 4)
    ffn = ctypes.c_size_t(0)
    assert lib.moe_ffn_workspace_size(ctypes.byref(s), ctypes.byref(ffn)) == 0
    assert ffn.value == r(S * 512 * 2)
    st = lib.moe_forward(ctypes.byref(s), A, A, None, A, A, A, A, A, A, A, None, None, A,
                         ctypes.c_size_t(need.value - 1), None)
    assert st == 5
    st = lib.moe_expert_ffn(ctypes.byref(s), A, A, A, A, A, A, A, A, A, A, A, ctypes.c_size_t(ffn.value - 1), None)
    assert st == 5


def test_workspace_holds_split_down_planes(lib):
    """A stream down pass whose reduction splits 8 ways over workgroups gets 8
    fp32 partial-sum planes [8, S, d] after y_rows; other shapes get none."""
    r = lambda v: (v + 255) // 256 * 256

    def sizes(T, d, f, E, K, path):
        s = _shape(T=T, d=d, f=f, E=E, K=K, ffn_path=path)
        n = ctypes.c_size_t(0)
        assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0
        S = T * K
        base = 4 * r(S * 4) + r((E + 1) * 4) + r(S * f * 2) + r(S * d * 4)
        return n.value, base, S

    # dense MLP at decode (64 rows on one expert, 256 items of 32 channels: 8-way split)
    n, base, S = sizes(64, 8192, 24576, 1, 1, 0)
    assert n == base + r(8 * S * 8192 * 4)
    m = ctypes.c_size_t(0)
    s = _shape(T=64, d=8192, f=24576, E=1, K=1)
    assert lib.moe_mlp_workspace_size(ctypes.byref(s), ctypes.byref(m)) == 0 and m.value == n
    # 37 rows per expert on the stream schedule, 8 reduction steps: split
    n, base, S = sizes(300, 256, 512, 16, 2, 1)
    assert n == base + r(8 * S * 256 * 4)
    # the down pass alone: the planes, or an error for a short or misaligned workspace
    s = _shape(T=300, d=256, f=512, E=16, K=2, ffn_path=1)
    dn = ctypes.c_size_t(0)
    assert lib.moe_down_workspace_size(ctypes.byref(s), ctypes.byref(dn)) == 0 and dn.value == 8 * S * 256 * 4
    assert lib.moe_expert_down(ctypes.byref(s), A, A, A, A, A, A, ctypes.c_size_t(dn.value - 1), None) == 5
    assert lib.moe_expert_down(ctypes.byref(s), A, A, A, A, A, MIS, ctypes.c_size_t(dn.value), None) == 4
    f = ctypes.c_size_t(0)
    assert lib.moe_ffn_workspace_size(ctypes.byref(s), ctypes.byref(f)) == 0
    assert f.value == r(S * 512 * 2) + r(dn.value)
    # the same with 6 reduction steps (fewer than the split): none
    n, base, _ = sizes(300, 256, 384, 16, 2, 1)
    assert n == base
    # at most 32 rows per expert (the 32-row variant): none
    n, base, _ = sizes(256, 256, 512, 16, 2, 1)
    assert n == base
    n, base, _ = sizes(300, 256, 512, 16, 2, 2)
    assert n == base + 2 * 256          # the tiled schedule: tile claim words of both passes


def test_empty_input_enqueues_nothing(lib):
    s = _shape(T=0)
    need = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(need)) == 0
    assert lib.moe_route(ctypes.byref(s), A, A, None, A, A, None) == 0
    assert lib.moe_permute(ctypes.byref(s), A, A, A, A, None) == 0
    assert lib.moe_combine(ctypes.byref(s), A, A, A, A, None) == 0
    assert lib.moe_forward(ctypes.byref(s), A, A, None, A, A, A, A, A, A, A, None, None, A,
                           ctypes.c_size_t(need.value), None) == 0
    # empty tensors may be NULL: nothing is read or written
    assert lib.moe_route(ctypes.byref(s), None, None, None, None, None, None) == 0
    assert lib.moe_forward(ctypes.byref(s), *([None] * 13), ctypes.c_size_t(0), None) == 0
    # an invalid shape is still reported
    bad = _shape(T=0, d=100)
    assert lib.moe_forward(ctypes.byref(bad), *([None] * 13), ctypes.c_size_t(0), None) == 2


def test_mlp_validation(lib):
    s = _shape(E=2, K=1)
    n = ctypes.c_size_t(0)
    assert lib.moe_mlp_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 2
    assert lib.moe_mlp_forward(ctypes.byref(s), A, A, A, A, A, A, A, A, A, ctypes.c_size_t(1 << 30), None) == 2
    s = _shape(E=1, K=1)
    assert lib.moe_mlp_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0
    assert lib.moe_mlp_forward(ctypes.byref(s), A, A, A, A, A, A, None, A, A, ctypes.c_size_t(1 << 30), None) == 1
    assert lib.moe_mlp_forward(ctypes.byref(s), A, A, A, A, A, A, A, A, A, ctypes.c_size_t(n.value - 1), None) == 5


def test_pack_validation(lib):
    assert lib.moe_pack_rows(8, 64, A, B, None) == 2        # rows % 16
    assert lib.moe_pack_rows(16, 96, A, B, None) == 2       # cols % 64
    assert lib.moe_pack_rows(16, 64, None, B, None) == 1
    assert lib.moe_pack_rows(16, 64, A, MIS, None) == 4
    assert lib.moe_pack_rows(16, 64, A, A, None) == 6       # not in place
    assert lib.moe_pack_rows(0, 64, A, B, None) == 0


def test_quantize_validation(lib):
    assert lib.moe_quantize_rows(4, 100, 1, A, 1, A, A, None) == 2      # cols % 16
    assert lib.moe_quantize_rows(-1, 64, 1, A, 1, A, A, None) == 2
    assert lib.moe_quantize_rows(4, 64, 7, A, 1, A, A, None) == 3
    assert lib.moe_quantize_rows(4, 64, 1, A, 1, None, A, None) == 1
    assert lib.moe_quantize_rows(4, 64, 1, MIS, 1, A, A, None) == 4
    assert lib.moe_quantize_rows(0, 64, 1, A, 1, A, A, None) == 0


def test_tiled_passes_take_tile_claim_words(lib):
    """On the tiled schedule each FFN pass can take 256 bytes of tile claim words:
    moe_forward's and moe_expert_ffn's workspaces hold both, the staged passes
    take them in their optional workspace (short or misaligned: an error)."""
    r = lambda v: (v + 255) // 256 * 256
    T, d, f, E, K = 512, 256, 512, 4, 2
    S = T * K
    s = _shape(T=T, d=d, f=f, E=E, K=K, ffn_path=2)
    n, g, dn, ff = (ctypes.c_size_t(0) for _ in range(4))
    assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0
    assert n.value == 4 * r(S * 4) + r((E + 1) * 4) + r(S * f * 2) + r(S * d * 4) + 2 * 256
    assert lib.moe_gate_up_workspace_size(ctypes.byref(s), ctypes.byref(g)) == 0 and g.value == 256
    assert lib.moe_down_workspace_size(ctypes.byref(s), ctypes.byref(dn)) == 0 and dn.value == 256
    assert lib.moe_ffn_workspace_size(ctypes.byref(s), ctypes.byref(ff)) == 0
    assert ff.value == r(S * f * 2) + 256 + 256
    assert lib.moe_expert_gate_up(ctypes.byref(s), A, A, A, A, A, A, A, A, A, ctypes.c_size_t(255), None) == 5
    assert lib.moe_expert_gate_up(ctypes.byref(s), A, A, A, A, A, A, A, A, MIS, ctypes.c_size_t(256), None) == 4
    assert lib.moe_expert_down(ctypes.byref(s), A, A, A, A, A, A, ctypes.c_size_t(255), None) == 5
    assert lib.moe_expert_down(ctypes.byref(s), A, A, A, A, A, MIS, ctypes.c_size_t(256), None) == 4
    # the stream schedule's gate/up pass takes none
    s = _shape(T=8, ffn_path=1)
    assert lib.moe_gate_up_workspace_size(ctypes.byref(s), ctypes.byref(g)) == 0 and g.value == 0


def test_weight_format_rules(lib):
    # bf16 weights carry no scales: NULL scale pointers pass validation
    s = _shape(T=0, weight_fmt=1)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0
    assert lib.moe_forward(ctypes.byref(s), A, A, None, A, A, A, None, None, None, A, None, None, A,
                           ctypes.c_size_t(n.value), None) == 0
    # int8 and fp8 weights need their scales
    for fmt in (0, 2):
        s = _shape(T=8, weight_fmt=fmt)
        assert lib.moe_forward(ctypes.byref(s), A, A, None, A, A, A, None, A, A, A, None, None, A,
                               ctypes.c_size_t(1 << 30), None) == 1
    # the comparator encodings run with bf16 activations only
    for fmt in (1, 2):
        s = _shape(T=8, act_dtype=0, weight_fmt=fmt)
        assert lib.moe_forward(ctypes.byref(s), A, A, None, A, A, A, A, A, A, A, None, None, A,
                               ctypes.c_size_t(1 << 30), None) == 6
        assert b"bf16 activations" in lib.moe_last_error()
        assert lib.moe_expert_down(ctypes.byref(s), A, A, A, A, A, None, 0, None) == 6


def test_noalloc_forward_rejects_shapes_beyond_its_scratch(lib):
    """moe_forward_noalloc checks its fixed 32 MiB scratch before anything else is
    touched: an oversized shape is MOE_ERR_WORKSPACE with no pointer read and no
    HIP call; T = 0 is accepted."""
    big = _shape(T=40000, d=128, f=192, E=4, K=2)          # y_rows alone: 80000 x 128 x 4 bytes > 32 MiB
    st = lib.moe_forward_noalloc(ctypes.byref(big), None, None, None, None, None, None, None, None, None,
                                 None, None, None, None)
    assert st == 5 and b"scratch" in lib.moe_last_error()
    empty = _shape(T=0)
    assert lib.moe_forward_noalloc(ctypes.byref(empty), None, None, None, None, None, None, None, None, None,
                                   None, None, None, None) == 0
