"""ctypes binding of the C ABI in include/moe.h (argument marshalling only).

Every function here has the name of the C entry point it calls and forwards plain
device pointers and sizes; all work runs in the HIP kernels of libmoe.so. Arguments
may be torch tensors (their data_ptr() is passed) or integers (raw device pointers).
A missing library raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_SCRATCH_LIMIT = range(6)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_CALL_ROUTE, MOE_CALL_DISPATCH, MOE_CALL_GROUPED_FFN, MOE_CALL_COMBINE, MOE_CALL_BIAS_UPDATE = range(5)
MOE_CALL_GROUPED_FFN_BACKWARD, MOE_CALL_ROUTE_BACKWARD = 5, 6
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILED = 0, 1
MOE_W1, MOE_W3, MOE_W2 = 0, 1, 2
MOE_SCORE_SIGMOID, MOE_SCORE_SOFTMAX = 0, 1
ABI_VERSION = 5
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}
SCORES = {"sigmoid": MOE_SCORE_SIGMOID, "softmax": MOE_SCORE_SOFTMAX}


class MoeError(RuntimeError):
    def __init__(self, call: str, status: int, text: str):
        super().__init__(f"{call}: status {status} ({text})")
        self.status = status


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("n_routed", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("act", ctypes.c_int32), ("ffn", ctypes.c_int32), ("score", ctypes.c_int32)]


class moe_expert_set(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("s1", ctypes.c_void_p), ("s3", ctypes.c_void_p), ("s2", ctypes.c_void_p),
                ("layout", ctypes.c_int32)]


class moe_expert_grads(ctypes.Structure):
    _fields_ = [("dw1", ctypes.c_void_p), ("dw3", ctypes.c_void_p), ("dw2", ctypes.c_void_p)]


_lib = None


def load():
    """Load libmoe.so (build it first if it is absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sp = ctypes.POINTER(moe_shape)
    ep = ctypes.POINTER(moe_expert_set)
    gp = ctypes.POINTER(moe_expert_grads)
    sig = {
        "moe_route": [sp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_dispatch": [sp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_grouped_ffn": [sp, vp, vp, vp, ep, ep, vp, vp, vp, sz, vp],
        "moe_grouped_ffn_noalloc": [sp, vp, vp, vp, ep, ep, vp, vp, vp],
        "moe_combine": [sp, vp, vp, vp, vp, vp, vp, vp],
        "moe_bias_update": [sp, vp, f32, vp, vp],
        "moe_quantize_fp8": [vp, i32, i64, i64, i32, i32, vp, vp, vp],
        "moe_pack_weights": [sp, i32, i64, vp, vp, vp],
        "moe_combine_backward": [sp, vp, vp, vp, vp, vp, vp, vp],
        "moe_grouped_ffn_backward": [sp, vp, vp, vp, vp, ep, ep, vp, vp, vp, gp, gp, vp, sz, vp],
        "moe_route_backward": [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.moe_workspace_bytes.argtypes = [sp, i32]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_abi_version.argtypes = []
    lib.moe_abi_version.restype = i32
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(call: str, st: int):
    if st != MOE_OK:
        raise MoeError(call, st, load().moe_status_string(st).decode())


def make_shape(T, d, n_routed, top_k, n_shared, d_ff, act="bf16", ffn="bf16", score="sigmoid") -> moe_shape:
    return moe_shape(T, d, n_routed, top_k, n_shared, d_ff, DTYPES[act], DTYPES[ffn], SCORES[score])


def make_expert_set(w1, w3, w2, s1=None, s3=None, s2=None, layout: int = MOE_LAYOUT_ROWS) -> moe_expert_set:
    return moe_expert_set(_ptr(w1), _ptr(w3), _ptr(w2), _ptr(s1), _ptr(s3), _ptr(s2), layout)


def moe_workspace_bytes(shape: moe_shape, call: int) -> int:
    return load().moe_workspace_bytes(ctypes.byref(shape), call)


def moe_route(shape, u, centroids, bias, topk_idx, topk_gate, ws, ws_bytes: int, stream=None):
    _check("moe_route", load().moe_route(ctypes.byref(shape), _ptr(u), _ptr(centroids), _ptr(bias),
                                         _ptr(topk_idx), _ptr(topk_gate), _ptr(ws), ws_bytes, _stream(stream)))


def moe_dispatch(shape, topk_idx, expert_count, expert_offset, sorted_token, pair_row, ws, ws_bytes,
                 stream=None):
    _check("moe_dispatch", load().moe_dispatch(ctypes.byref(shape), _ptr(topk_idx), _ptr(expert_count),
                                               _ptr(expert_offset), _ptr(sorted_token), _ptr(pair_row),
                                               _ptr(ws), ws_bytes, _stream(stream)))


def moe_grouped_ffn(shape, u, expert_offset, sorted_token, routed: moe_expert_set, shared, y_routed,
                    y_shared, ws, ws_bytes, stream=None):
    sh = ctypes.byref(shared) if shared is not None else None
    _check("moe_grouped_ffn", load().moe_grouped_ffn(ctypes.byref(shape), _ptr(u), _ptr(expert_offset),
                                                     _ptr(sorted_token), ctypes.byref(routed), sh,
                                                     _ptr(y_routed), _ptr(y_shared), _ptr(ws), ws_bytes,
                                                     _stream(stream)))


def moe_grouped_ffn_noalloc(shape, u, expert_offset, sorted_token, routed: moe_expert_set, shared, y_routed,
                            y_shared, stream=None):
    sh = ctypes.byref(shared) if shared is not None else None
    _check("moe_grouped_ffn_noalloc", load().moe_grouped_ffn_noalloc(
        ctypes.byref(shape), _ptr(u), _ptr(expert_offset), _ptr(sorted_token), ctypes.byref(routed), sh,
        _ptr(y_routed), _ptr(y_shared), _stream(stream)))


def moe_combine(shape, u, y_routed, y_shared, pair_row, topk_gate, out, stream=None):
    _check("moe_combine", load().moe_combine(ctypes.byref(shape), _ptr(u), _ptr(y_routed), _ptr(y_shared),
                                             _ptr(pair_row), _ptr(topk_gate), _ptr(out), _stream(stream)))


def moe_bias_update(shape, expert_count, gamma, bias, stream=None):
    _check("moe_bias_update", load().moe_bias_update(ctypes.byref(shape), _ptr(expert_count), gamma,
                                                     _ptr(bias), _stream(stream)))


def make_expert_grads(dw1, dw3, dw2) -> moe_expert_grads:
    return moe_expert_grads(_ptr(dw1), _ptr(dw3), _ptr(dw2))


def moe_combine_backward(shape, dout, y_routed, pair_row, topk_gate, dy_routed, dgate, stream=None):
    _check("moe_combine_backward", load().moe_combine_backward(
        ctypes.byref(shape), _ptr(dout), _ptr(y_routed), _ptr(pair_row), _ptr(topk_gate), _ptr(dy_routed),
        _ptr(dgate), _stream(stream)))


def moe_grouped_ffn_backward(shape, u, dout, expert_offset, sorted_token, routed, shared, dy_routed, dx_routed,
                             dx_shared, d_routed, d_shared, ws, ws_bytes: int, stream=None):
    _check("moe_grouped_ffn_backward", load().moe_grouped_ffn_backward(
        ctypes.byref(shape), _ptr(u), _ptr(dout), _ptr(expert_offset), _ptr(sorted_token), ctypes.byref(routed),
        ctypes.byref(shared) if shared is not None else None, _ptr(dy_routed), _ptr(dx_routed), _ptr(dx_shared),
        ctypes.byref(d_routed), ctypes.byref(d_shared) if d_shared is not None else None, _ptr(ws), ws_bytes,
        _stream(stream)))


def moe_route_backward(shape, u, centroids, topk_idx, topk_gate, dgate, expert_offset, sorted_token, pair_row,
                       dout, dx_routed, dx_shared, du, dcentroids, dz, ws, ws_bytes: int, stream=None):
    _check("moe_route_backward", load().moe_route_backward(
        ctypes.byref(shape), _ptr(u), _ptr(centroids), _ptr(topk_idx), _ptr(topk_gate), _ptr(dgate),
        _ptr(expert_offset), _ptr(sorted_token), _ptr(pair_row), _ptr(dout), _ptr(dx_routed), _ptr(dx_shared),
        _ptr(du), _ptr(dcentroids), _ptr(dz), _ptr(ws), ws_bytes, _stream(stream)))


def moe_pack_weights(shape, matrix: int, n_experts: int, src, dst, stream=None):
    _check("moe_pack_weights", load().moe_pack_weights(ctypes.byref(shape), matrix, n_experts, _ptr(src), _ptr(dst),
                                                       _stream(stream)))


def moe_quantize_fp8(x, xt: int, rows: int, cols: int, tile_r: int, tile_c: int, q, scale, stream=None):
    _check("moe_quantize_fp8", load().moe_quantize_fp8(_ptr(x), xt, rows, cols, tile_r, tile_c, _ptr(q),
                                                       _ptr(scale), _stream(stream)))
