"""Thin Python binding of libmoe.so (argument marshalling only).

Every function has the name of the C entry point it calls and the same argument
order; torch tensors stand in for device pointers (None for NULL) and the
current torch stream is passed unless `stream` is given. All computation runs in
the HIP kernels of the library; importing this module fails if the library is
missing.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError("libmoe.so is not built (python -m quantized_moe_expert_fp32_amd.build)")
_lib = ctypes.CDLL(_LIB_PATH)

ROUTER_F32 = 0
ROUTER_AFFINE8 = 1

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_TIMEOUT = 0, -1, -2, -3, -4, -5


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.moe_last_error().decode()
        super().__init__("%s: %s (%s)" % (where, _lib.moe_status_str(status).decode(), msg))


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("hidden", "inter", "n_experts", "top_k", "has_shared", "group", "bits", "router_fmt")]

    @classmethod
    def make(cls, hidden, inter, n_experts, top_k, has_shared=1, router_fmt=ROUTER_AFFINE8, group=64, bits=4):
        return cls(hidden, inter, n_experts, top_k, has_shared, group, bits, router_fmt)

    @property
    def slots(self):
        return self.top_k + self.has_shared

    @property
    def n_mats(self):
        return self.n_experts + self.has_shared


class PrefillDispatchView(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_size_t), ("offsets", ctypes.c_size_t), ("ntiles", ctypes.c_size_t),
                ("tiles", ctypes.c_size_t), ("order", ctypes.c_size_t), ("max_tiles", ctypes.c_int32),
                ("tile_rows", ctypes.c_int32)]


class ExpertCanon(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q_gate", "s_gate", "b_gate", "q_up", "s_up", "b_up", "q_down", "s_down", "b_down")]


_P = ctypes.c_void_p
_S = ctypes.POINTER(Shape)
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

_lib.moe_abi_version.restype = _I32
_lib.moe_status_str.restype = ctypes.c_char_p
_lib.moe_status_str.argtypes = [_I32]
_lib.moe_last_error.restype = ctypes.c_char_p
_lib.moe_shape_check.restype = _I32
_lib.moe_shape_check.argtypes = [_S]
_lib.moe_experts_packed_bytes.restype = _SZ
_lib.moe_experts_packed_bytes.argtypes = [_S]
_lib.moe_pack_experts.restype = _I32
_lib.moe_pack_experts.argtypes = [_S, ctypes.POINTER(ExpertCanon), _P, _SZ, _P]
_lib.moe_router_packed_bytes.restype = _SZ
_lib.moe_router_packed_bytes.argtypes = [_S]
_lib.moe_pack_router.restype = _I32
_lib.moe_pack_router.argtypes = [_S, _P, _P, _P, _P, _SZ, _P]
_lib.moe_route.restype = _I32
_lib.moe_route.argtypes = [_S, _P, _P, _P, _I32, _P, _P, _P, _P, _P]
_lib.moe_route_from_logits.restype = _I32
_lib.moe_route_from_logits.argtypes = [_S, _P, _I32, _P, _P, _P, _P]
_lib.moe_decode_workspace_bytes.restype = _SZ
_lib.moe_decode_workspace_bytes.argtypes = [_S, _I32]
_lib.moe_experts_decode.restype = _I32
_lib.moe_experts_decode.argtypes = [_S, _P, _P, _I32, _P, _P, _SZ, _P, _P]
_lib.moe_experts_decode_noalloc.restype = _I32
_lib.moe_experts_decode_noalloc.argtypes = [_S, _P, _P, _I32, _P, _P, _P]
_lib.moe_decode_layer.restype = _I32
_lib.moe_decode_layer.argtypes = [_S, _P, _P, _P, _P, _I32, _P, _SZ, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.moe_decode_block.restype = _I32
_lib.moe_decode_block.argtypes = [_S, _P, _P, _P, _P, _I32, ctypes.c_float, _P, _SZ, _P, _P, _P, _P, _P, _P, _P]
_lib.moe_decode_layer_check.restype = _I32
_lib.moe_decode_layer_check.argtypes = [_S, _I32, _P, _SZ, _P]
_lib.moe_dispatch.restype = _I32
_lib.moe_dispatch.argtypes = [_S, _P, _I32, _P, _P, _P, _P]
_lib.moe_prefill_workspace_bytes.restype = _SZ
_lib.moe_prefill_workspace_bytes.argtypes = [_S, _I32]
_lib.moe_prefill_dispatch_layout.restype = _I32
_lib.moe_prefill_dispatch_layout.argtypes = [_S, _I32, ctypes.POINTER(PrefillDispatchView)]
_lib.moe_pack_experts_prefill.restype = _I32
_lib.moe_pack_experts_prefill.argtypes = [_S, _P, _P, _SZ, _P]
_lib.moe_experts_prefill.restype = _I32
_lib.moe_experts_prefill.argtypes = [_S, _P, _P, _I32, _P, _P, _SZ, _P, _P]
_lib.moe_experts_fp8_bytes.restype = _SZ
_lib.moe_experts_fp8_bytes.argtypes = [_S]
_lib.moe_pack_experts_fp8.restype = _I32
_lib.moe_pack_experts_fp8.argtypes = [_S, ctypes.POINTER(ExpertCanon), _P, _SZ, _P]
_lib.moe_prefill_fp8_workspace_bytes.restype = _SZ
_lib.moe_prefill_fp8_workspace_bytes.argtypes = [_S, _I32]
_lib.moe_experts_prefill_fp8.restype = _I32
_lib.moe_experts_prefill_fp8.argtypes = [_S, _P, _P, _I32, _P, _P, _SZ, _P, _P]
_lib.moe_combine.restype = _I32
_lib.moe_combine.argtypes = [_S, _P, _P, _P, _I32, _P, _P, _P]
_lib.moe_rmsnorm.restype = _I32
_lib.moe_rmsnorm.argtypes = [_I32, _P, _I32, ctypes.c_float, _P, _P]

EXPORTS = ("moe_abi_version", "moe_status_str", "moe_last_error", "moe_shape_check",
           "moe_experts_packed_bytes", "moe_pack_experts", "moe_router_packed_bytes", "moe_pack_router",
           "moe_route", "moe_route_from_logits", "moe_decode_workspace_bytes", "moe_experts_decode",
           "moe_experts_decode_noalloc", "moe_decode_layer", "moe_decode_block",
           "moe_decode_layer_check", "moe_dispatch", "moe_prefill_workspace_bytes", "moe_prefill_dispatch_layout",
           "moe_pack_experts_prefill", "moe_experts_prefill", "moe_experts_fp8_bytes", "moe_pack_experts_fp8",
           "moe_prefill_fp8_workspace_bytes", "moe_experts_prefill_fp8", "moe_combine", "moe_rmsnorm")


def library_path() -> str:
    return _LIB_PATH


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(st, where):
    if st != OK:
        raise MoeError(st, where)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def moe_abi_version() -> int:
    return _lib.moe_abi_version()


def moe_shape_check(shape: Shape) -> int:
    return _lib.moe_shape_check(ctypes.byref(shape))


def moe_experts_packed_bytes(shape: Shape) -> int:
    return _lib.moe_experts_packed_bytes(ctypes.byref(shape))


def moe_router_packed_bytes(shape: Shape) -> int:
    return _lib.moe_router_packed_bytes(ctypes.byref(shape))


def moe_decode_workspace_bytes(shape: Shape, T: int) -> int:
    return _lib.moe_decode_workspace_bytes(ctypes.byref(shape), T)


def moe_prefill_workspace_bytes(shape: Shape, T: int) -> int:
    return _lib.moe_prefill_workspace_bytes(ctypes.byref(shape), T)


def moe_pack_experts(shape, src: dict, packed, stream=None):
    canon = ExpertCanon(*[_ptr(src[f[0]]) for f in ExpertCanon._fields_])
    _check(_lib.moe_pack_experts(ctypes.byref(shape), ctypes.byref(canon), _ptr(packed), _nbytes(packed),
                                 _stream(stream)), "moe_pack_experts")


def moe_pack_router(shape, w, s, b, packed, stream=None):
    _check(_lib.moe_pack_router(ctypes.byref(shape), _ptr(w), _ptr(s), _ptr(b), _ptr(packed), _nbytes(packed),
                                _stream(stream)), "moe_pack_router")


def moe_route(shape, router_packed, logit_bias, x, T, logits, ids, w, w_shared, stream=None):
    _check(_lib.moe_route(ctypes.byref(shape), _ptr(router_packed), _ptr(logit_bias), _ptr(x), T, _ptr(logits),
                          _ptr(ids), _ptr(w), _ptr(w_shared), _stream(stream)), "moe_route")


def moe_route_from_logits(shape, logits, T, ids, w, w_shared, stream=None):
    _check(_lib.moe_route_from_logits(ctypes.byref(shape), _ptr(logits), T, _ptr(ids), _ptr(w), _ptr(w_shared),
                                      _stream(stream)), "moe_route_from_logits")


def moe_experts_decode(shape, experts_packed, x, T, ids, ws, y, stream=None):
    _check(_lib.moe_experts_decode(ctypes.byref(shape), _ptr(experts_packed), _ptr(x), T, _ptr(ids), _ptr(ws),
                                   _nbytes(ws), _ptr(y), _stream(stream)), "moe_experts_decode")


def moe_experts_decode_noalloc(shape, experts_packed, x, T, ids, y, stream=None):
    _check(_lib.moe_experts_decode_noalloc(ctypes.byref(shape), _ptr(experts_packed), _ptr(x), T, _ptr(ids),
                                           _ptr(y), _stream(stream)), "moe_experts_decode_noalloc")


def moe_decode_layer(shape, router_packed, logit_bias, experts_packed, x, T, ws, logits, ids, w, w_shared, y,
                     residual, out, stream=None):
    _check(_lib.moe_decode_layer(ctypes.byref(shape), _ptr(router_packed), _ptr(logit_bias), _ptr(experts_packed),
                                 _ptr(x), T, _ptr(ws), _nbytes(ws), _ptr(logits), _ptr(ids), _ptr(w),
                                 _ptr(w_shared), _ptr(y), _ptr(residual), _ptr(out), _stream(stream)),
           "moe_decode_layer")


def moe_decode_block(shape, router_packed, logit_bias, experts_packed, x, T, eps, ws, logits, ids, w, w_shared, y,
                     x_out, stream=None):
    _check(_lib.moe_decode_block(ctypes.byref(shape), _ptr(router_packed), _ptr(logit_bias), _ptr(experts_packed),
                                 _ptr(x), T, ctypes.c_float(eps), _ptr(ws), _nbytes(ws), _ptr(logits), _ptr(ids),
                                 _ptr(w), _ptr(w_shared), _ptr(y), _ptr(x_out), _stream(stream)), "moe_decode_block")


def moe_decode_layer_check(shape, T, ws, stream=None):
    """True if no moe_decode_layer call on ws since the last check timed out in a
    bounded wait; False if one did (the word is cleared). Raises on bad arguments."""
    st = _lib.moe_decode_layer_check(ctypes.byref(shape), T, _ptr(ws), _nbytes(ws), _stream(stream))
    if st == ERR_TIMEOUT:
        return False
    _check(st, "moe_decode_layer_check")
    return True


def moe_dispatch(shape, ids, T, counts, offsets, order, stream=None):
    _check(_lib.moe_dispatch(ctypes.byref(shape), _ptr(ids), T, _ptr(counts), _ptr(offsets), _ptr(order),
                             _stream(stream)), "moe_dispatch")


def moe_prefill_dispatch_layout(shape, T) -> PrefillDispatchView:
    v = PrefillDispatchView()
    _check(_lib.moe_prefill_dispatch_layout(ctypes.byref(shape), T, ctypes.byref(v)), "moe_prefill_dispatch_layout")
    return v


def moe_pack_experts_prefill(shape, experts_packed, experts_prefill, stream=None):
    _check(_lib.moe_pack_experts_prefill(ctypes.byref(shape), _ptr(experts_packed), _ptr(experts_prefill),
                                         _nbytes(experts_prefill), _stream(stream)), "moe_pack_experts_prefill")


def moe_experts_prefill(shape, experts_prefill, x, T, ids, ws, y, stream=None):
    _check(_lib.moe_experts_prefill(ctypes.byref(shape), _ptr(experts_prefill), _ptr(x), T, _ptr(ids), _ptr(ws),
                                    _nbytes(ws), _ptr(y), _stream(stream)), "moe_experts_prefill")


def moe_experts_fp8_bytes(shape: Shape) -> int:
    return _lib.moe_experts_fp8_bytes(ctypes.byref(shape))


def moe_pack_experts_fp8(shape, src: dict, fp8, stream=None):
    canon = ExpertCanon(*[_ptr(src[f[0]]) for f in ExpertCanon._fields_])
    _check(_lib.moe_pack_experts_fp8(ctypes.byref(shape), ctypes.byref(canon), _ptr(fp8), _nbytes(fp8),
                                     _stream(stream)), "moe_pack_experts_fp8")


def moe_prefill_fp8_workspace_bytes(shape: Shape, T: int) -> int:
    return _lib.moe_prefill_fp8_workspace_bytes(ctypes.byref(shape), T)


def moe_experts_prefill_fp8(shape, experts_fp8, x, T, ids, ws, y, stream=None):
    _check(_lib.moe_experts_prefill_fp8(ctypes.byref(shape), _ptr(experts_fp8), _ptr(x), T, _ptr(ids), _ptr(ws),
                                        _nbytes(ws), _ptr(y), _stream(stream)), "moe_experts_prefill_fp8")


def fp8_expert_regions(shape: Shape):
    """Byte regions of one expert in the FP8 buffer (the layout moe.h documents):
    dict of (offset, rows, row bytes) for gate, up, down codes and (offset, count)
    for the float row scales, plus the per-expert stride."""
    Hp = -(-shape.hidden // 128) * 128
    Ip = -(-shape.inter // 128) * 128
    I, H = shape.inter, shape.hidden
    up = I * Hp
    down = 2 * up
    scales = down + H * Ip
    return {"gate": (0, I, Hp), "up": (up, I, Hp), "down": (down, H, Ip), "scales": (scales, 2 * I + H),
            "stride": -(-(scales + 4 * (2 * I + H)) // 256) * 256}


def moe_combine(shape, y, w, w_shared, T, residual, out, stream=None):
    _check(_lib.moe_combine(ctypes.byref(shape), _ptr(y), _ptr(w), _ptr(w_shared), T, _ptr(residual), _ptr(out),
                            _stream(stream)), "moe_combine")


def moe_rmsnorm(hidden, x, T, eps, out, stream=None):
    _check(_lib.moe_rmsnorm(hidden, _ptr(x), T, ctypes.c_float(eps), _ptr(out), _stream(stream)), "moe_rmsnorm")


def raw_call(name: str, *args):
    """Calls an entry point with raw ctypes arguments and returns its status (for argument-check tests)."""
    return getattr(_lib, name)(*args)
