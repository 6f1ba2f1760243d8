"""Thin Python binding of libmoe_int4.so (the C ABI in include/moe_int4.h).

Functions carry the C names and take torch tensors on the GPU; the binding
only checks dtypes/shapes, marshals device pointers and the current HIP
stream, and raises on a non-OK status.  Every step runs in the library's HIP
kernels; there is no fallback.  Importing this module loads the library and
raises when it has not been built (python -m int4_routed_expert_moe_amd.build).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_int4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                      "(python -m int4_routed_expert_moe_amd.build)")

_lib = ctypes.CDLL(LIB_PATH)

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_LAUNCH = -4
MOE_MODE_BF16 = 0
MOE_MODE_EXACT_I8 = 1
MOE_MODE_BF16_F16P = 2
MOE_MODE_EXACT_I16 = 3

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

EXPORTS = {
    "moe_abi_version": ([], _I),
    "moe_status_string": ([_I], ctypes.c_char_p),
    "moe_last_error_detail": ([], ctypes.c_char_p),
    "moe_route_workspace_bytes": ([_I, _I, _I], _SZ),
    "moe_route": ([_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P], _I),
    "moe_route_grouped": ([_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P, _P, _P, _SZ, _P], _I),
    "moe_permute_workspace_bytes": ([_I, _I, _I], _SZ),
    "moe_permute": ([_P, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "moe_permute_noalloc": ([_P, _I, _I, _I, _P, _P, _P, _P, _P], _I),
    "moe_quant_act_int8": ([_P, _I, _I, _P, _P, _P], _I),
    "moe_int4_prepack": ([_P, _P, _I, _I, _I, _P, _P, _P], _I),
    "moe_int4_check_scales": ([_P, _SZ, _P, _P], _I),
    "moe_act_f16p": ([_P, _I, _I, _P, _P], _I),
    "moe_quant_act_int16": ([_P, _I, _I, _P, _P, _P], _I),
    "moe_exact_linear_i8w": ([_P, _P, _P, _P, _I, _I, _I, _P, _P], _I),
    "moe_int4_grouped_swiglu": ([_I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "moe_int4_grouped_down": ([_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P], _I),
    "moe_combine": ([_I, _P, _P, _P, _P, _I, _I, _I, _P, _P], _I),
    "moe_dense_workspace_bytes": ([_I, _I, _I], _SZ),
    "moe_linear_bf16": ([_P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P], _I),
    "moe_dense_swiglu_bf16": ([_P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P], _I),
    "moe_silu_mul_bf16": ([_P, _P, _P, ctypes.c_int64, _P], _I),
    "moe_rmsnorm_bf16": ([_P, _P, ctypes.c_float, _P, _I, _I, _P], _I),
    "moe_int4_group_sums_i32": ([_P, _P, _I, _I, _I, _P, _P], _I),
}
for _name, (_args, _res) in EXPORTS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class MoEError(RuntimeError):
    def __init__(self, fn, status):
        detail = _lib.moe_last_error_detail().decode()
        text = _lib.moe_status_string(status).decode()
        super().__init__(f"{fn}: {text} ({status}): {detail}")
        self.status = status


def _check(fn, status):
    if status != MOE_OK:
        raise MoEError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, shape=None, name="tensor"):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def moe_abi_version() -> int:
    return _lib.moe_abi_version()


def moe_route_workspace_bytes(T, H, E) -> int:
    return _lib.moe_route_workspace_bytes(T, H, E)


def moe_route(x, w_router, bias, k, renormalize, topk_idx, topk_w, ws):
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, torch.bfloat16, (T, H), "x")
    _need(w_router, torch.bfloat16, (E, H), "w_router")
    _need(bias, torch.float32, (E,), "bias")
    _need(topk_idx, torch.int32, (T, k), "topk_idx")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _check("moe_route", _lib.moe_route(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, int(bool(renormalize)),
                                       _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream()))


def moe_route_grouped(x, w_router, bias, k, renormalize, n_group, topk_group, routed_scale, topk_idx, topk_w, ws):
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, torch.bfloat16, (T, H), "x")
    _need(w_router, torch.bfloat16, (E, H), "w_router")
    _need(bias, torch.float32, (E,), "bias")
    _need(topk_idx, torch.int32, (T, k), "topk_idx")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _check("moe_route_grouped", _lib.moe_route_grouped(
        _ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, int(bool(renormalize)), n_group, topk_group,
        float(routed_scale), _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws.numel() * ws.element_size(), _stream()))


def moe_permute_workspace_bytes(T, k, E) -> int:
    return _lib.moe_permute_workspace_bytes(T, k, E)


def moe_permute(topk_idx, E, counts, offsets, sorted_slot, slot_pos, ws=None):
    T, k = topk_idx.shape
    _need(topk_idx, torch.int32, (T, k), "topk_idx")
    _need(counts, torch.int32, (E,), "counts")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    _need(sorted_slot, torch.int32, (T * k,), "sorted_slot")
    _need(slot_pos, torch.int32, (T * k,), "slot_pos")
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("moe_permute", _lib.moe_permute(_ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets),
                                           _ptr(sorted_slot), _ptr(slot_pos), _ptr(ws), nbytes, _stream()))


def moe_permute_noalloc(topk_idx, E, counts, offsets, sorted_slot, slot_pos):
    """moe_permute without a workspace (the library's fixed device buffer holds the block counts)."""
    T, k = topk_idx.shape
    _need(topk_idx, torch.int32, (T, k), "topk_idx")
    _need(counts, torch.int32, (E,), "counts")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    _need(sorted_slot, torch.int32, (T * k,), "sorted_slot")
    _need(slot_pos, torch.int32, (T * k,), "slot_pos")
    _check("moe_permute_noalloc", _lib.moe_permute_noalloc(_ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets),
                                                           _ptr(sorted_slot), _ptr(slot_pos), _stream()))


def moe_quant_act_int8(x, q, s):
    M, K = x.shape
    _need(x, torch.bfloat16, (M, K), "x")
    _need(q, torch.int8, (M, K), "q")
    _need(s, torch.float32, (M, K // 32), "s")
    _check("moe_quant_act_int8", _lib.moe_quant_act_int8(_ptr(x), M, K, _ptr(q), _ptr(s), _stream()))


def moe_quant_act_int16(x, q, s):
    M, K = x.shape
    _need(x, torch.bfloat16, (M, K), "x")
    _need(q, torch.int16, (M, K), "q")
    _need(s, torch.float32, (M, K // 32), "s")
    _check("moe_quant_act_int16", _lib.moe_quant_act_int16(_ptr(x), M, K, _ptr(q), _ptr(s), _stream()))


def moe_exact_linear_i8w(qx, sx, qw, sw, y):
    """ExactLinear with 8-bit weights: y [M,N] fp32 from int8 codes and fp32 group scales."""
    M, K = qx.shape
    N = qw.shape[0]
    _need(qx, torch.int8, (M, K), "qx")
    _need(sx, torch.float32, (M, K // 32), "sx")
    _need(qw, torch.int8, (N, K), "qw")
    _need(sw, torch.float32, (N, K // 32), "sw")
    _need(y, torch.float32, (M, N), "y")
    _check("moe_exact_linear_i8w", _lib.moe_exact_linear_i8w(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), M, N, K,
                                                             _ptr(y), _stream()))


def moe_int4_prepack(packed, scale, packed_out, scale_out):
    """Checkpoint-layout expert matrices [E, N, K/2] uint8 + [E, N, K/32] bf16 -> the
    fragment layout the grouped GEMMs read (same shapes, out of place; the scales
    come out as fp16)."""
    if packed.dim() != 3:
        raise ValueError("packed must be [E, N, K/2]")
    E, N, K2 = packed.shape
    K = 2 * K2
    _need(packed, torch.uint8, (E, N, K // 2), "packed")
    _need(scale, torch.bfloat16, (E, N, K // 32), "scale")
    _need(packed_out, torch.uint8, (E, N, K // 2), "packed_out")
    _need(scale_out, torch.float16, (E, N, K // 32), "scale_out")
    _check("moe_int4_prepack", _lib.moe_int4_prepack(_ptr(packed), _ptr(scale), E, N, K, _ptr(packed_out),
                                                     _ptr(scale_out), _stream()))


def moe_int4_check_scales(scale, count=None):
    """Raise MoEError (MOE_ERR_UNSUPPORTED) when a bf16 scale tensor holds values that
    are neither 0 nor of magnitude in [2^-14, 2^9]; synchronises the current stream."""
    _need(scale, torch.bfloat16, None, "scale")
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=scale.device)
    _need(count, torch.int32, (1,), "count")
    _check("moe_int4_check_scales", _lib.moe_int4_check_scales(_ptr(scale), scale.numel(), _ptr(count), _stream()))


_ACT_DTYPE = {MOE_MODE_BF16: torch.bfloat16, MOE_MODE_EXACT_I8: torch.int8, MOE_MODE_BF16_F16P: torch.float16,
              MOE_MODE_EXACT_I16: torch.int16}
_EXACT_MODES = (MOE_MODE_EXACT_I8, MOE_MODE_EXACT_I16)


def moe_act_f16p(x, out):
    """x [rows, K] bf16 -> out [rows, K] fp16 in the staging format of the routed GEMMs
    (8-element blocks stored as e0,e4,e1,e5,e2,e6,e3,e7)."""
    if x.dim() != 2:
        raise ValueError("x: expected a 2-D tensor")
    rows, K = x.shape
    _need(x, torch.bfloat16, (rows, K), "x")
    _need(out, torch.float16, (rows, K), "out")
    _check("moe_act_f16p", _lib.moe_act_f16p(_ptr(x), rows, K, _ptr(out), _stream()))


def moe_int4_grouped_swiglu(mode, act, act_scale, gate_packed, gate_scale, up_packed, up_scale, offsets,
                            sorted_slot, T, k, E, H, I, h, h_scale):
    _need(act, _ACT_DTYPE.get(mode, torch.bfloat16), (T, H), "act")
    for t, dt, shp, nm in ((gate_packed, torch.uint8, (E, I, H // 2), "gate_packed"),
                           (gate_scale, torch.float16, (E, I, H // 32), "gate_scale"),
                           (up_packed, torch.uint8, (E, I, H // 2), "up_packed"),
                           (up_scale, torch.float16, (E, I, H // 32), "up_scale"),
                           (offsets, torch.int32, (E + 1,), "offsets"),
                           (sorted_slot, torch.int32, (T * k,), "sorted_slot")):
        _need(t, dt, shp, nm)
    if mode not in _EXACT_MODES:
        _need(h, _ACT_DTYPE.get(mode, torch.bfloat16), (T * k, I), "h")
    else:
        _need(act_scale, torch.float32, (T, H // 32), "act_scale")
        _need(h, _ACT_DTYPE[mode], (T * k, I), "h")
        _need(h_scale, torch.float32, (T * k, I // 32), "h_scale")
    _check("moe_int4_grouped_swiglu", _lib.moe_int4_grouped_swiglu(
        mode, _ptr(act), _ptr(act_scale), _ptr(gate_packed), _ptr(gate_scale), _ptr(up_packed), _ptr(up_scale),
        _ptr(offsets), _ptr(sorted_slot), T, k, E, H, I, _ptr(h), _ptr(h_scale), _stream()))


def moe_int4_grouped_down(mode, h, h_scale, down_packed, down_scale, offsets, T, k, E, I, H, y):
    _need(h, _ACT_DTYPE.get(mode, torch.bfloat16), (T * k, I), "h")
    _need(down_packed, torch.uint8, (E, H, I // 2), "down_packed")
    _need(down_scale, torch.float16, (E, H, I // 32), "down_scale")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    if mode not in _EXACT_MODES:
        _need(y, torch.bfloat16, (T * k, H), "y")
    else:
        _need(h_scale, torch.float32, (T * k, I // 32), "h_scale")
        _need(y, torch.float32, (T * k, H), "y")
    _check("moe_int4_grouped_down", _lib.moe_int4_grouped_down(
        mode, _ptr(h), _ptr(h_scale), _ptr(down_packed), _ptr(down_scale), _ptr(offsets), T, k, E, I, H, _ptr(y),
        _stream()))


def moe_combine(mode, y, slot_pos, topk_w, shared, T, k, H, out):
    ydt = torch.bfloat16 if mode == MOE_MODE_BF16 else torch.float32
    _need(y, ydt, (T * k, H), "y")
    _need(slot_pos, torch.int32, (T * k,), "slot_pos")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(shared, torch.bfloat16, (T, H), "shared")
    _need(out, ydt, (T, H), "out")
    _check("moe_combine", _lib.moe_combine(mode, _ptr(y), _ptr(slot_pos), _ptr(topk_w), _ptr(shared), T, k, H,
                                           _ptr(out), _stream()))


def moe_dense_workspace_bytes(M, N_total, K) -> int:
    return _lib.moe_dense_workspace_bytes(M, N_total, K)


def moe_linear_bf16(x, w, add, y, ws=None):
    M, K = x.shape
    N = w.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(w, torch.bfloat16, (N, K), "w")
    _need(add, torch.bfloat16, (M, N), "add")
    _need(y, torch.bfloat16, (M, N), "y")
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("moe_linear_bf16", _lib.moe_linear_bf16(_ptr(x), _ptr(w), _ptr(add), _ptr(y), M, N, K, _ptr(ws), nbytes,
                                                   _stream()))


def moe_dense_swiglu_bf16(x, w_gate, w_up, h, ws=None):
    M, H = x.shape
    I = w_gate.shape[0]
    _need(x, torch.bfloat16, (M, H), "x")
    _need(w_gate, torch.bfloat16, (I, H), "w_gate")
    _need(w_up, torch.bfloat16, (I, H), "w_up")
    _need(h, torch.bfloat16, (M, I), "h")
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("moe_dense_swiglu_bf16", _lib.moe_dense_swiglu_bf16(_ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(h), M, H, I,
                                                               _ptr(ws), nbytes, _stream()))


def moe_silu_mul_bf16(g, u, h):
    _need(g, torch.bfloat16, None, "g")
    _need(u, torch.bfloat16, tuple(g.shape), "u")
    _need(h, torch.bfloat16, tuple(g.shape), "h")
    _check("moe_silu_mul_bf16", _lib.moe_silu_mul_bf16(_ptr(g), _ptr(u), _ptr(h), g.numel(), _stream()))


def moe_rmsnorm_bf16(x, gain, eps, y):
    M, N = x.shape
    _need(x, torch.bfloat16, (M, N), "x")
    _need(gain, torch.bfloat16, (N,), "gain")
    _need(y, torch.bfloat16, (M, N), "y")
    _check("moe_rmsnorm_bf16", _lib.moe_rmsnorm_bf16(_ptr(x), _ptr(gain), float(eps), _ptr(y), M, N, _stream()))


def moe_int4_group_sums_i32(q_x, packed, G):
    M, K = q_x.shape
    N = packed.shape[0]
    _need(q_x, torch.int8, (M, K), "q_x")
    _need(packed, torch.uint8, (N, K // 2), "packed")
    _need(G, torch.int32, (M, N, K // 32), "G")
    _check("moe_int4_group_sums_i32", _lib.moe_int4_group_sums_i32(_ptr(q_x), _ptr(packed), M, N, K, _ptr(G),
                                                                   _stream()))
