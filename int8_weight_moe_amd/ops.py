"""Python binding of libmoe_int8: argument marshalling only.

Each function takes torch tensors that already live on the current HIP device,
allocates the outputs (torch is the memory and stream provider), and calls the
C entry point of the same name on torch's current stream. Every step of the
layer runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import (MOE_BF16, MOE_F32, MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_TILED, MOE_W_BF16,  # noqa: F401
                   MOE_W_FP8, MOE_W_INT8, MoeError, MoeShape)

_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}


@dataclasses.dataclass
class Int8Experts:
    """Expert weights of one MoE layer as the FFN kernels read them.

    fmt MOE_W_INT8 (ExpertsInt8, the default): q_gate, q_up [E, f, d] int8 and
    q_down [E, d, f] int8 codes plus per-output-channel scales s_gate, s_up
    [E, f], s_down [E, d] (all fp32 or all bf16). fmt MOE_W_FP8: the same with
    OCP e4m3 codes (uint8 tensors). fmt MOE_W_BF16 (comparator): q_* are the
    bf16 weights themselves and s_* are None. Every q_* holds its bytes in the
    tiled layout of moe_pack_rows; the tensor shape is kept for the sizes.
    """
    q_gate: torch.Tensor
    q_up: torch.Tensor
    q_down: torch.Tensor
    s_gate: Optional[torch.Tensor]
    s_up: Optional[torch.Tensor]
    s_down: Optional[torch.Tensor]
    fmt: int = MOE_W_INT8

    @property
    def E(self) -> int:
        return self.q_gate.shape[0]

    @property
    def f(self) -> int:
        return self.q_gate.shape[1]

    @property
    def d(self) -> int:
        return self.q_gate.shape[2]

    @property
    def scale_dtype(self) -> torch.dtype:
        return self.s_gate.dtype if self.s_gate is not None else torch.bfloat16


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe_int8 must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    return _DT[dt]


def make_shape(T: int, d: int, f: int, E: int, K: int, act: torch.dtype, scale: torch.dtype,
               path: int = MOE_PATH_AUTO, fmt: int = MOE_W_INT8) -> MoeShape:
    return MoeShape(T, d, f, E, K, _dtype_code(act), _dtype_code(scale), path, fmt)


def _lib_handle():
    return _lib.load()


def workspace_size(shape: MoeShape) -> int:
    lib = _lib_handle()
    n = ctypes.c_size_t(0)
    _lib.check(lib.moe_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def ffn_workspace_size(shape: MoeShape) -> int:
    lib = _lib_handle()
    n = ctypes.c_size_t(0)
    _lib.check(lib.moe_ffn_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def moe_route(x: torch.Tensor, router_w: torch.Tensor, bias: Optional[torch.Tensor], K: int):
    """Router + top-K gate. Returns (topk_ids int32 [T,K], topk_w fp32 [T,K])."""
    lib = _lib_handle()
    T, d = x.shape
    E = router_w.shape[0]
    shape = make_shape(T, d, 64, E, K, x.dtype, torch.float32)
    ids = torch.empty((T, K), dtype=torch.int32, device=x.device)
    w = torch.empty((T, K), dtype=torch.float32, device=x.device)
    _lib.check(lib.moe_route(ctypes.byref(shape), _ptr(x), _ptr(router_w), _ptr(bias), _ptr(ids), _ptr(w),
                             _stream()))
    return ids, w


def moe_permute(topk_ids: torch.Tensor, E: int):
    """Returns (expert_offsets [E+1], sorted_slots [T*K], slot_to_row [T*K]), all int32."""
    lib = _lib_handle()
    T, K = topk_ids.shape
    shape = MoeShape(T, 64, 64, E, K, MOE_BF16, MOE_BF16, MOE_PATH_AUTO)
    dev = topk_ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_slots = torch.empty(T * K, dtype=torch.int32, device=dev)
    slot_to_row = torch.empty(T * K, dtype=torch.int32, device=dev)
    _lib.check(lib.moe_permute(ctypes.byref(shape), _ptr(topk_ids), _ptr(offsets), _ptr(sorted_slots),
                               _ptr(slot_to_row), _stream()))
    return offsets, sorted_slots, slot_to_row


def moe_expert_ffn(x: torch.Tensor, expert_offsets: torch.Tensor, sorted_slots: torch.Tensor,
                   experts: Int8Experts, K: int, path: int = MOE_PATH_AUTO,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Expert SwiGLU FFNs on the permuted rows. Returns y_rows fp32 [T*K, d] (sorted-row order)."""
    lib = _lib_handle()
    T, d = x.shape
    shape = make_shape(T, d, experts.f, experts.E, K, x.dtype, experts.scale_dtype, path, experts.fmt)
    y_rows = torch.empty((T * K, d), dtype=torch.float32, device=x.device)
    need = ffn_workspace_size(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _lib.check(lib.moe_expert_ffn(
        ctypes.byref(shape), _ptr(x), _ptr(expert_offsets), _ptr(sorted_slots), _ptr(experts.q_gate),
        _ptr(experts.q_up), _ptr(experts.q_down), _ptr(experts.s_gate), _ptr(experts.s_up),
        _ptr(experts.s_down), _ptr(y_rows), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream()))
    return y_rows


def gate_up_workspace_size(shape: MoeShape) -> int:
    lib = _lib_handle()
    n = ctypes.c_size_t(0)
    _lib.check(lib.moe_gate_up_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def moe_expert_gate_up(x: torch.Tensor, expert_offsets: torch.Tensor, sorted_slots: torch.Tensor,
                       experts: Int8Experts, K: int, path: int = MOE_PATH_AUTO,
                       h: Optional[torch.Tensor] = None, use_workspace: bool = True,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gate/up pass: h [T*K, f] bf16 (sorted-row order). With use_workspace the call
    gets the workspace it can use (`workspace` if given, else a new one: the tiled
    schedule's tile claim words); without it every tile follows the static order
    (same result, bit for bit)."""
    lib = _lib_handle()
    T, d = x.shape
    shape = make_shape(T, d, experts.f, experts.E, K, x.dtype, experts.scale_dtype, path, experts.fmt)
    if h is None:
        h = torch.empty((T * K, experts.f), dtype=torch.bfloat16, device=x.device)
    ws = None
    need = gate_up_workspace_size(shape) if use_workspace else 0
    if need:
        ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=x.device)
    _lib.check(lib.moe_expert_gate_up(
        ctypes.byref(shape), _ptr(x), _ptr(expert_offsets), _ptr(sorted_slots), _ptr(experts.q_gate),
        _ptr(experts.q_up), _ptr(experts.s_gate), _ptr(experts.s_up), _ptr(h), _ptr(ws),
        ctypes.c_size_t(ws.numel() if ws is not None else 0), _stream()))
    return h


def down_workspace_size(shape: MoeShape) -> int:
    lib = _lib_handle()
    n = ctypes.c_size_t(0)
    _lib.check(lib.moe_down_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def moe_expert_down(h: torch.Tensor, expert_offsets: torch.Tensor, experts: Int8Experts, T: int, K: int,
                    act: torch.dtype = torch.bfloat16, path: int = MOE_PATH_AUTO,
                    y_rows: Optional[torch.Tensor] = None, split_workspace: bool = True,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Down pass: y_rows [T*K, d] fp32 from h [T*K, f] bf16. With split_workspace the
    call gets the workspace it can use (`workspace` if given, else a new one: the
    stream schedule's partial sums of a split reduction, none for most stream
    shapes, or the tiled schedule's tile claim words); without it a split
    reduction stays inside one workgroup and tiles follow the static order (same
    result, bit for bit)."""
    lib = _lib_handle()
    shape = make_shape(T, experts.d, experts.f, experts.E, K, act, experts.scale_dtype, path, experts.fmt)
    if y_rows is None:
        y_rows = torch.empty((T * K, experts.d), dtype=torch.float32, device=h.device)
    ws = None
    need = down_workspace_size(shape) if split_workspace else 0
    if need:
        ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=h.device)
    _lib.check(lib.moe_expert_down(ctypes.byref(shape), _ptr(h), _ptr(expert_offsets), _ptr(experts.q_down),
                                   _ptr(experts.s_down), _ptr(y_rows), _ptr(ws),
                                   ctypes.c_size_t(ws.numel() if ws is not None else 0), _stream()))
    return y_rows


def moe_combine(y_rows: torch.Tensor, slot_to_row: torch.Tensor, topk_w: torch.Tensor,
                out_dtype: torch.dtype) -> torch.Tensor:
    """y[t] = sum_k topk_w[t,k] * y_rows[slot_to_row[t*K+k]]. Returns y [T, d] in out_dtype."""
    lib = _lib_handle()
    T, K = topk_w.shape
    d = y_rows.shape[1]
    shape = make_shape(T, d, 64, max(K, 1), K, out_dtype, torch.float32)
    y = torch.empty((T, d), dtype=out_dtype, device=y_rows.device)
    _lib.check(lib.moe_combine(ctypes.byref(shape), _ptr(y_rows), _ptr(slot_to_row), _ptr(topk_w), _ptr(y),
                               _stream()))
    return y


class MoeLayer:
    """A resident MoE layer: router weights, int8 experts and a reusable workspace."""

    def __init__(self, router_w: torch.Tensor, bias: Optional[torch.Tensor], experts: Int8Experts, K: int):
        self.router_w = router_w
        self.bias = bias
        self.experts = experts
        self.K = K
        self._ws = None

    def workspace(self, shape: MoeShape) -> torch.Tensor:
        need = max(workspace_size(shape), 256)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.router_w.device)
        return self._ws

    def forward(self, x: torch.Tensor, path: int = MOE_PATH_AUTO, y: Optional[torch.Tensor] = None,
                ids: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None):
        return moe_forward(x, self.router_w, self.bias, self.experts, self.K, path=path, y=y, ids=ids, w=w,
                           workspace=self.workspace(self.shape(x, path)))

    def shape(self, x: torch.Tensor, path: int = MOE_PATH_AUTO) -> MoeShape:
        e = self.experts
        return make_shape(x.shape[0], x.shape[1], e.f, e.E, self.K, x.dtype, e.scale_dtype, path, e.fmt)


def moe_forward(x: torch.Tensor, router_w: torch.Tensor, bias: Optional[torch.Tensor], experts: Int8Experts,
                K: int, path: int = MOE_PATH_AUTO, y: Optional[torch.Tensor] = None,
                ids: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None):
    """The whole layer. Returns (y [T, d] in x.dtype, topk_ids [T, K], topk_w [T, K])."""
    lib = _lib_handle()
    T, d = x.shape
    shape = make_shape(T, d, experts.f, experts.E, K, x.dtype, experts.scale_dtype, path, experts.fmt)
    dev = x.device
    if y is None:
        y = torch.empty((T, d), dtype=x.dtype, device=dev)
    if ids is None:
        ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, K), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(workspace_size(shape), 256), dtype=torch.uint8, device=dev)
    _lib.check(lib.moe_forward(
        ctypes.byref(shape), _ptr(x), _ptr(router_w), _ptr(bias), _ptr(experts.q_gate), _ptr(experts.q_up),
        _ptr(experts.q_down), _ptr(experts.s_gate), _ptr(experts.s_up), _ptr(experts.s_down), _ptr(y), _ptr(ids),
        _ptr(w), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream()))
    return y, ids, w


def moe_forward_noalloc(x: torch.Tensor, router_w: torch.Tensor, bias: Optional[torch.Tensor],
                        experts: Int8Experts, K: int, path: int = MOE_PATH_AUTO, y: torch.Tensor = None,
                        ids: torch.Tensor = None, w: torch.Tensor = None):
    """The whole layer on the library's fixed per-GPU scratch (no workspace argument;
    the C call allocates nothing). Outputs y, ids and w must be given by the caller
    that cannot allocate; they are allocated here only when omitted."""
    lib = _lib_handle()
    T, d = x.shape
    shape = make_shape(T, d, experts.f, experts.E, K, x.dtype, experts.scale_dtype, path, experts.fmt)
    dev = x.device
    if y is None:
        y = torch.empty((T, d), dtype=x.dtype, device=dev)
    if ids is None:
        ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, K), dtype=torch.float32, device=dev)
    _lib.check(lib.moe_forward_noalloc(
        ctypes.byref(shape), _ptr(x), _ptr(router_w), _ptr(bias), _ptr(experts.q_gate), _ptr(experts.q_up),
        _ptr(experts.q_down), _ptr(experts.s_gate), _ptr(experts.s_up), _ptr(experts.s_down), _ptr(y), _ptr(ids),
        _ptr(w), _stream()))
    return y, ids, w


def moe_mlp_forward(x: torch.Tensor, experts: Int8Experts, path: int = MOE_PATH_AUTO,
                    y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense int8-weight SwiGLU MLP (one expert, E = K = 1). Returns y [T, d] in x.dtype."""
    lib = _lib_handle()
    T, d = x.shape
    if experts.E != 1:
        raise ValueError("the dense MLP takes one expert (E = 1)")
    shape = make_shape(T, d, experts.f, 1, 1, x.dtype, experts.scale_dtype, path, experts.fmt)
    if y is None:
        y = torch.empty((T, d), dtype=x.dtype, device=x.device)
    if workspace is None:
        n = ctypes.c_size_t(0)
        _lib.check(lib.moe_mlp_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
        workspace = torch.empty(max(n.value, 256), dtype=torch.uint8, device=x.device)
    _lib.check(lib.moe_mlp_forward(
        ctypes.byref(shape), _ptr(x), _ptr(experts.q_gate), _ptr(experts.q_up), _ptr(experts.q_down),
        _ptr(experts.s_gate), _ptr(experts.s_up), _ptr(experts.s_down), _ptr(y), _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), _stream()))
    return y


def moe_quantize_rows(w: torch.Tensor, scale_dtype: torch.dtype):
    """ExpertsInt8 quantizer on the GPU: w [..., cols] (fp32/bf16) -> (q int8 [..., cols], s [...])."""
    lib = _lib_handle()
    cols = w.shape[-1]
    rows = w.numel() // cols
    q = torch.empty(w.shape, dtype=torch.int8, device=w.device)
    s = torch.empty(w.shape[:-1], dtype=scale_dtype, device=w.device)
    _lib.check(lib.moe_quantize_rows(ctypes.c_int64(rows), ctypes.c_int32(cols), _dtype_code(w.dtype), _ptr(w),
                                     _dtype_code(scale_dtype), _ptr(q), _ptr(s), _stream()))
    return q, s


def moe_quantize_rows_fp8(w: torch.Tensor, scale_dtype: torch.dtype):
    """FP8 comparator quantizer on the GPU: w [..., cols] -> (e4m3 code bytes uint8 [..., cols], s [...])."""
    lib = _lib_handle()
    cols = w.shape[-1]
    rows = w.numel() // cols
    q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    s = torch.empty(w.shape[:-1], dtype=scale_dtype, device=w.device)
    _lib.check(lib.moe_quantize_rows_fp8(ctypes.c_int64(rows), ctypes.c_int32(cols), _dtype_code(w.dtype), _ptr(w),
                                         _dtype_code(scale_dtype), _ptr(q), _ptr(s), _stream()))
    return q, s


def moe_quantize_pack_rows(w: torch.Tensor, scale_dtype: torch.dtype, fmt: int = MOE_W_INT8):
    """Quantize w [..., rows, cols] (int8 or fp8 e4m3 codes) straight into the tiled layout:
    (codes [..., rows, cols] in the tiled byte order, scales [..., rows]), one pass."""
    lib = _lib_handle()
    cols = w.shape[-1]
    rows = w.numel() // cols
    q = torch.empty(w.shape, dtype=torch.int8 if fmt == MOE_W_INT8 else torch.uint8, device=w.device)
    s = torch.empty(w.shape[:-1], dtype=scale_dtype, device=w.device)
    _lib.check(lib.moe_quantize_pack_rows(ctypes.c_int64(rows), ctypes.c_int32(cols), _dtype_code(w.dtype), _ptr(w),
                                          _dtype_code(scale_dtype), ctypes.c_int32(fmt), _ptr(q), _ptr(s), _stream()))
    return q, s


def moe_pack_rows(q: torch.Tensor) -> torch.Tensor:
    """Row-major int8 codes [..., rows, cols] -> the tiled layout (same shape, permuted bytes)."""
    lib = _lib_handle()
    cols = q.shape[-1]
    rows = q.numel() // cols
    out = torch.empty_like(q)
    _lib.check(lib.moe_pack_rows(ctypes.c_int64(rows), ctypes.c_int32(cols), _ptr(q), _ptr(out), _stream()))
    return out


def pack_bf16_experts(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor) -> Int8Experts:
    """bf16 expert weights (the unquantized comparator) -> the tiled layout of their bytes."""
    out = []
    for w in (w_gate, w_up, w_down):
        if w.dtype != torch.bfloat16:
            raise TypeError("pack_bf16_experts takes bf16 weights")
        b = w.contiguous().view(torch.int8)           # [..., rows, 2*cols] bytes
        out.append(moe_pack_rows(b).view(torch.bfloat16))
    return Int8Experts(out[0], out[1], out[2], None, None, None, fmt=MOE_W_BF16)


def pack_experts(q_gate: torch.Tensor, q_up: torch.Tensor, q_down: torch.Tensor, s_gate: torch.Tensor,
                 s_up: torch.Tensor, s_down: torch.Tensor) -> Int8Experts:
    """Row-major int8 codes + scales -> Int8Experts in the kernels' tiled layout."""
    return Int8Experts(moe_pack_rows(q_gate), moe_pack_rows(q_up), moe_pack_rows(q_down), s_gate, s_up, s_down)


def quantize_experts_fp8(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                         scale_dtype: torch.dtype) -> Int8Experts:
    """FP8 comparator: quantize the (out, in) expert weights to e4m3 codes in the tiled layout (one pass)."""
    out, scales = [], []
    for w in (w_gate, w_up, w_down):
        q, s = moe_quantize_pack_rows(w, scale_dtype, MOE_W_FP8)
        out.append(q)
        scales.append(s)
    return Int8Experts(out[0], out[1], out[2], scales[0], scales[1], scales[2], fmt=MOE_W_FP8)


def quantize_experts(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                     scale_dtype: torch.dtype) -> Int8Experts:
    """Load-time ExpertsInt8: quantize the (out, in) expert weights straight into the tiled layout (one pass)."""
    out = []
    scales = []
    for w in (w_gate, w_up, w_down):
        q, s = moe_quantize_pack_rows(w, scale_dtype, MOE_W_INT8)
        out.append(q)
        scales.append(s)
    return Int8Experts(out[0], out[1], out[2], scales[0], scales[1], scales[2])
