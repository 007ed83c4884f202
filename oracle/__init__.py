"""CPU oracle for the DeepSeekMoE layer forward pass (ctypes wrapper).

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code with
the HIP path and never imports it. The arithmetic lives in ``moe_oracle.c``; the
passages each function follows are cited there and in ``moe_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

ORC_F32, ORC_BF16, ORC_FP8 = 0, 1, 2
_DT = {"f32": ORC_F32, "bf16": ORC_BF16, "fp8": ORC_FP8}
ORC_SIGMOID, ORC_SOFTMAX = 0, 1
_SCORE = {"sigmoid": ORC_SIGMOID, "softmax": ORC_SOFTMAX}

_lib = None


def build():
    """Compile the oracle with the host C compiler (always recompiles)."""
    global _lib
    _lib = None
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _load()


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, dbl, flt = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                              ctypes.c_float)
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = dbl
    lib.orc_bf16_from_double.argtypes = [dbl]
    lib.orc_bf16_from_double.restype = ctypes.c_uint16
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_value.restype = dbl
    lib.orc_e4m3_from_float.argtypes = [flt]
    lib.orc_e4m3_from_float.restype = ctypes.c_uint8
    lib.orc_bf16_from_double_array.argtypes = [vp, i64, vp]
    lib.orc_e4m3_from_float_array.argtypes = [vp, i64, vp]
    lib.orc_quantize_tiles.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp]
    lib.orc_route.argtypes = [i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_dispatch.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp]
    lib.orc_bias_update.argtypes = [i64, i32, i32, vp, flt, vp]
    lib.orc_expert_rows.argtypes = [i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_layer.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp] + [vp] * 12 + \
        [vp] * 6
    lib.orc_layer.restype = i32
    lib.orc_combine.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.orc_combine.restype = None
    lib.orc_layer_backward.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp] + \
        [vp] * 6 + [vp] * 3 + [vp] * 6 + [vp] * 4
    lib.orc_layer_backward.restype = i32
    for f in (lib.orc_bf16_from_double_array, lib.orc_e4m3_from_float_array,
              lib.orc_quantize_tiles, lib.orc_route, lib.orc_dispatch, lib.orc_bias_update,
              lib.orc_expert_rows):
        f.restype = None
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _act_arr(a, dt):
    return _c(a, np.float32 if dt == ORC_F32 else np.uint16)


# ---------------------------------------------------------------- scalars

def bf16_value(bits: int) -> float:
    return _load().orc_bf16_value(bits)


def bf16_from_double(x) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().orc_bf16_from_double_array(_p(x), x.size, _p(out))
    return out


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(code)


def e4m3_table() -> np.ndarray:
    return np.array([e4m3_value(i) for i in range(256)], np.float64)


def e4m3_from_float(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().orc_e4m3_from_float_array(_p(x), x.size, _p(out))
    return out


# ---------------------------------------------------------------- the layer

def quantize(x, dtype: str, tr: int, tc: int):
    """Tile quantisation: returns (codes uint8 [rows, cols], scales fp32 [rows/tr, cols/tc])."""
    dt = _DT[dtype]
    x = _act_arr(x, dt)
    rows, cols = x.shape
    assert rows % tr == 0 and cols % tc == 0
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows // tr, cols // tc), np.float32)
    _load().orc_quantize_tiles(_p(x), dt, rows, cols, tr, tc, _p(q), _p(s))
    return q, s


def route(u, e, b, top_k: int, act: str, want_v: bool = False, score: str = "sigmoid"):
    """Routing of the rows of u: (idx [n,K] ascending, gate [n,K] double, gap [n], v or None).
    score "sigmoid": biased top-K of Sigmoid(z); "softmax": top-K of z, b unused (may be None)."""
    dt = _DT[act]
    u = _act_arr(u, dt)
    e = _act_arr(e, dt)
    n, d = u.shape
    n_r = e.shape[0]
    b = _c(np.zeros(n_r, np.float32) if b is None else b, np.float32)
    idx = np.empty((n, top_k), np.int32)
    gate = np.empty((n, top_k), np.float64)
    gap = np.empty(n, np.float64)
    v = np.empty((n, n_r), np.float64) if want_v else None
    _load().orc_route(n, d, n_r, top_k, dt, _SCORE[score], _p(u), _p(e), _p(b), _p(idx), _p(gate), _p(gap),
                      _p(v))
    return idx, gate, gap, v


def dispatch(idx, n_r: int):
    idx = _c(idx, np.int32)
    T, K = idx.shape
    count = np.empty(n_r, np.int32)
    offset = np.empty(n_r + 1, np.int32)
    sorted_token = np.empty(T * K, np.int32)
    pair_row = np.empty((T, K), np.int32)
    _load().orc_dispatch(T, n_r, K, _p(idx), _p(count), _p(offset), _p(sorted_token), _p(pair_row))
    return count, offset, sorted_token, pair_row


def bias_update(count, T: int, top_k: int, gamma: float, b):
    count = _c(count, np.int32)
    b = _c(b, np.float32).copy()
    _load().orc_bias_update(T, count.size, top_k, _p(count), gamma, _p(b))
    return b


def expert_rows(x, w1, w3, w2, ffn: str, s1=None, s3=None, s2=None):
    """One expert's SwiGLU FFN on the rows of x: (h at its rounding point, y) in double."""
    dt = _DT[ffn]
    x = _act_arr(x, ORC_F32 if dt == ORC_F32 else ORC_BF16)
    n, d = x.shape
    d_ff = w1.shape[0]
    wdt = np.uint8 if dt == ORC_FP8 else (np.float32 if dt == ORC_F32 else np.uint16)
    w1, w3, w2 = _c(w1, wdt), _c(w3, wdt), _c(w2, wdt)
    if dt == ORC_FP8:
        s1, s3, s2 = _c(s1, np.float32), _c(s3, np.float32), _c(s2, np.float32)
    h = np.empty((n, d_ff), np.float64)
    y = np.empty((n, d), np.float64)
    _load().orc_expert_rows(d, d_ff, dt, _p(x), n, _p(w1), _p(w3), _p(w2), _p(s1), _p(s3), _p(s2),
                            _p(h), _p(y))
    return h, y


def _ptr_array(items):
    arr = (ctypes.c_void_p * max(1, len(items)))()
    for i, a in enumerate(items):
        arr[i] = None if a is None else a.ctypes.data
    return arr


def layer(u, e, b, routed: dict, shared: list, *, top_k: int, d_ff: int, act: str, ffn: str,
          want_components: bool = False, score: str = "sigmoid"):
    """The layer output for the tokens whose rows are u, in double.

    routed: {expert id: (w1, w3, w2) or (w1, w3, w2, s1, s3, s2)} for at least every
    expert those tokens select; shared: list of the same tuples for the N_s shared experts.
    Routing as in route() with the given score. Returns a dict with out, idx, gate, gap
    (and shared_sum, routed_sum)."""
    adt, fdt = _DT[act], _DT[ffn]
    u = _act_arr(u, adt)
    e = _act_arr(e, adt)
    n, d = u.shape
    n_r = e.shape[0]
    b = _c(np.zeros(n_r, np.float32) if b is None else b, np.float32)
    wdt = np.uint8 if fdt == ORC_FP8 else (np.float32 if fdt == ORC_F32 else np.uint16)
    keep = []

    def prep(tup):
        ws = [_c(a, wdt) for a in tup[:3]]
        ss = [_c(a, np.float32) for a in tup[3:6]] if fdt == ORC_FP8 else [None, None, None]
        keep.extend(ws + ss)
        return ws, ss

    r = [prep(routed[i]) if i in routed else ([None] * 3, [None] * 3) for i in range(n_r)]
    s = [prep(t) for t in shared]
    arrs = [_ptr_array([x[0][j] for x in r]) for j in range(3)] + \
           [_ptr_array([x[1][j] for x in r]) for j in range(3)] + \
           [_ptr_array([x[0][j] for x in s]) for j in range(3)] + \
           [_ptr_array([x[1][j] for x in s]) for j in range(3)]
    out = np.empty((n, d), np.float64)
    idx = np.empty((n, top_k), np.int32)
    gate = np.empty((n, top_k), np.float64)
    gap = np.empty(n, np.float64)
    ssum = np.empty((n, d), np.float64) if want_components else None
    rsum = np.empty((n, d), np.float64) if want_components else None
    st = _load().orc_layer(n, d, n_r, top_k, len(shared), d_ff, adt, fdt, _SCORE[score], _p(u), _p(e), _p(b),
                           *[ctypes.cast(a, ctypes.c_void_p) for a in arrs],
                           _p(out), _p(idx), _p(gate), _p(gap), _p(ssum), _p(rsum))
    if st != 0:
        raise ValueError("oracle layer: a selected routed expert has no weights")
    res = {"out": out, "idx": idx, "gate": gate, "gap": gap}
    if want_components:
        res["shared_sum"] = ssum
        res["routed_sum"] = rsum
    return res


def combine(u, y_shared, y_routed, pair_row, gate, act: str):
    """out = u + y_shared + sum_k gate * y_routed[pair_row], in double."""
    dt = _DT[act]
    u = _act_arr(u, dt)
    y = _act_arr(y_routed, dt)
    ysh = None if y_shared is None else _c(y_shared, np.float32)
    pr = _c(pair_row, np.int32)
    g = _c(gate, np.float32)
    n, d = u.shape
    K = pr.shape[1]
    out = np.empty((n, d), np.float64)
    _load().orc_combine(n, d, K, dt, _p(u), _p(ysh), _p(y), _p(pr), _p(g), _p(out))
    return out


def layer_backward(u, e, b, routed: dict, shared: list, dout, *, top_k: int, d_ff: int, act: str,
                   ffn: str, score: str = "sigmoid", want_du: bool = True, want_de: bool = True,
                   grad_routed=(), grad_shared: bool = False):
    """Gradients of sum(dout * out) for the tokens whose rows are u, in double.

    routed: {expert id: (w1, w3, w2)} for at least every expert whose rows are needed
    (all selected experts when du or de is wanted, else those in grad_routed); shared: the
    N_s shared experts' tuples. grad_routed: routed ids whose dW1, dW3, dW2 are formed;
    grad_shared: form the shared experts' too. Returns a dict with du, de (or None),
    dw_routed {i: (dw1, dw3, dw2)}, dw_shared [(dw1, dw3, dw2)], idx, gate, dgate, dz."""
    adt, fdt = _DT[act], _DT[ffn]
    u = _act_arr(u, adt)
    e = _act_arr(e, adt)
    dout = _act_arr(dout, adt)
    n, d = u.shape
    n_r = e.shape[0]
    n_s = len(shared)
    b = _c(np.zeros(n_r, np.float32) if b is None else b, np.float32)
    wdt = np.float32 if fdt == ORC_F32 else np.uint16
    keep = []

    def prep(tup):
        ws = [_c(a, wdt) for a in tup[:3]]
        keep.extend(ws)
        return ws

    r = [prep(routed[i]) if i in routed else [None] * 3 for i in range(n_r)]
    s = [prep(t) for t in shared]
    warrs = [_ptr_array([x[j] for x in r]) for j in range(3)] + [_ptr_array([x[j] for x in s]) for j in range(3)]
    dwr = {int(i): (np.empty((d_ff, d)), np.empty((d_ff, d)), np.empty((d, d_ff))) for i in grad_routed}
    dws = [(np.empty((d_ff, d)), np.empty((d_ff, d)), np.empty((d, d_ff))) for _ in range(n_s)] \
        if grad_shared else []
    garrs = [_ptr_array([dwr[i][j] if i in dwr else None for i in range(n_r)]) for j in range(3)] + \
            [_ptr_array([x[j] for x in dws]) if dws else None for j in range(3)]
    du = np.empty((n, d)) if want_du else None
    de = np.empty((n_r, d)) if want_de else None
    idx = np.empty((n, top_k), np.int32)
    gate = np.empty((n, top_k))
    dgate = np.empty((n, top_k))
    dz = np.empty((n, top_k))
    full = want_du or want_de
    st = _load().orc_layer_backward(
        n, d, n_r, top_k, n_s, d_ff, adt, fdt, _SCORE[score], _p(u), _p(e), _p(b),
        *[ctypes.cast(a, ctypes.c_void_p) for a in warrs], _p(dout), _p(du), _p(de),
        *[None if a is None else ctypes.cast(a, ctypes.c_void_p) for a in garrs],
        _p(idx), _p(gate), _p(dgate) if full else None, _p(dz) if full else None)
    if st != 0:
        raise ValueError(f"oracle layer_backward: status {st}")
    return {"du": du, "de": de, "dw_routed": dwr, "dw_shared": dws, "idx": idx, "gate": gate,
            "dgate": dgate if full else None, "dz": dz if full else None}
