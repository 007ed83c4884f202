"""Seeded synthetic inputs for the DeepSeekMoE layer.

This module draws numbers and nothing else: it holds none of the layer's
arithmetic, and it is the only code that the HIP path's tests and the CPU
oracle's tests have in common.  Values come from ``gen.c`` (Philox4x32-10 bits,
Box-Muller normals), so element ``i`` of a tensor depends only on
``(seed, tensor id, i)`` and any slice can be regenerated alone.

The workloads follow the layer shapes of the DeepSeek-V3 explainer
("DeepSeek-V3 テクニカルレポート 論文解説", key ideas: 1 shared + 256 routed
experts with 8 active; method section 2 for the layer), one GPU's share of that
layer under 8-way expert parallelism, and two smaller shapes.  Shapes, distributions and seeds are fixed here; the design doc lists
the recipe.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_inputs.so")

# tensor ids: the third Philox counter word
TID_U, TID_E, TID_B, TID_W1, TID_W3, TID_W2, TID_SW1, TID_SW3, TID_SW2 = range(1, 10)
TID_U_BATCH = 0x100  # u of a later token batch: TID_U_BATCH + batch (batch >= 1)

F32, BF16, FP8 = "f32", "bf16", "fp8"


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    n_routed: int
    top_k: int
    n_shared: int
    d_ff: int
    act: str            # dtype of u, e and the layer output: "f32" or "bf16"
    ffn: str            # dtype of the expert GEMM operands: "f32", "bf16" or "fp8"
    seed: int
    bias_range: float   # b ~ U(-r, r); 0 means b = 0
    hot_experts: tuple = field(default=())   # expert ids whose centroid norm is scaled
    hot_scale: float = 1.0
    gamma: float = 0.001

    def with_tokens(self, T: int) -> "Workload":
        d = dict(self.__dict__)
        d["T"] = T
        return Workload(**d)

    @property
    def pairs(self) -> int:
        return self.T * self.top_k

    def flops(self) -> float:
        """Algorithmic FLOPs of one layer forward: router GEMM plus the SwiGLU FFN
        of every routed and shared row (3 GEMMs of d x d_ff each)."""
        router = 2.0 * self.T * self.d * self.n_routed
        rows = self.T * self.top_k + self.n_shared * self.T
        return router + 6.0 * self.d * self.d_ff * rows

    def ffn_flops(self) -> float:
        rows = self.T * self.top_k + self.n_shared * self.T
        return 6.0 * self.d * self.d_ff * rows


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", T=64, d=256, n_routed=16, top_k=2, n_shared=1, d_ff=128,
                         act=F32, ffn=F32, seed=2601, bias_range=0.0),
    "mid_bf16": Workload("mid_bf16", T=4096, d=2048, n_routed=64, top_k=6, n_shared=2, d_ff=1408,
                         act=BF16, ffn=BF16, seed=2602, bias_range=0.01),
    "v3_prefill_bf16": Workload("v3_prefill_bf16", T=8192, d=7168, n_routed=256, top_k=8, n_shared=1,
                                d_ff=2048, act=BF16, ffn=BF16, seed=2603, bias_range=0.01),
    # identical tensors to the bf16 prefill workload; the expert GEMMs run in FP8
    "v3_prefill_fp8": Workload("v3_prefill_fp8", T=8192, d=7168, n_routed=256, top_k=8, n_shared=1,
                               d_ff=2048, act=BF16, ffn=FP8, seed=2603, bias_range=0.01),
    "v3_decode_skewed": Workload("v3_decode_skewed", T=128, d=7168, n_routed=256, top_k=8, n_shared=1,
                                 d_ff=2048, act=BF16, ffn=BF16, seed=2605, bias_range=0.01,
                                 hot_experts=tuple(range(0, 256, 32)), hot_scale=3.0),
    # One GPU's share of the V3 layer under expert parallelism over 8 GPUs: 32 local routed
    # experts receiving about 2048 rows each (T*K/N_r of the 8 GPUs' tokens) and the local
    # shared expert over this GPU's 8192 tokens, drawn as a layer of 32 routed experts with
    # top-8 over 8192 tokens, which gives the grouped FFN that shape.
    "v3_ep8_share_bf16": Workload("v3_ep8_share_bf16", T=8192, d=7168, n_routed=32, top_k=8, n_shared=1,
                                  d_ff=2048, act=BF16, ffn=BF16, seed=2607, bias_range=0.01),
    "v3_ep8_share_fp8": Workload("v3_ep8_share_fp8", T=8192, d=7168, n_routed=32, top_k=8, n_shared=1,
                                 d_ff=2048, act=BF16, ffn=FP8, seed=2607, bias_range=0.01),
}

_lib = None


def _build():
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)


def build():
    """Compile the generator library (always recompiles)."""
    global _lib
    _lib = None
    _build()
    return _load()


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        _build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, u32, dbl = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double
    vp = ctypes.c_void_p
    lib.gen_philox4x32_10.argtypes = [vp, vp, vp]
    lib.gen_normal_f32.argtypes = [u64, u32, u64, u64, dbl, vp]
    lib.gen_normal_bf16.argtypes = [u64, u32, u64, u64, dbl, vp]
    lib.gen_uniform_f32.argtypes = [u64, u32, u64, u64, dbl, dbl, vp]
    for f in (lib.gen_philox4x32_10, lib.gen_normal_f32, lib.gen_normal_bf16, lib.gen_uniform_f32):
        f.restype = None
    _lib = lib
    return lib


def philox4x32_10(ctr, key):
    lib = _load()
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.gen_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def normal(seed: int, tid: int, start: int, n: int, std: float, dtype: str, out=None) -> np.ndarray:
    """n normal variates N(0, std^2): float32 array, or uint16 bf16 bit patterns."""
    lib = _load()
    if dtype == F32:
        out = np.empty(n, np.float32) if out is None else out
        lib.gen_normal_f32(seed, tid, start, n, std, out.ctypes.data)
    elif dtype == BF16:
        out = np.empty(n, np.uint16) if out is None else out
        lib.gen_normal_bf16(seed, tid, start, n, std, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out


def uniform(seed: int, tid: int, start: int, n: int, lo: float, hi: float) -> np.ndarray:
    lib = _load()
    out = np.empty(n, np.float32)
    lib.gen_uniform_f32(seed, tid, start, n, lo, hi, out.ctypes.data)
    return out


def weight_dtype(w: Workload) -> str:
    """Storage dtype of the generated expert weights (FP8 codes are made from the
    bf16 weights by block quantisation, not drawn)."""
    return F32 if w.ffn == F32 else BF16


def _tid_u(batch: int) -> int:
    return TID_U if batch == 0 else TID_U_BATCH + batch


def make_u(w: Workload, rows: slice = None, batch: int = 0) -> np.ndarray:
    """u ~ N(0,1), [T, d] (act dtype); `rows` selects a token range; `batch` > 0 draws
    the tokens of a later batch (an independent stream of the same distribution)."""
    r0, r1 = (0, w.T) if rows is None else (rows.start, rows.stop)
    a = normal(w.seed, _tid_u(batch), r0 * w.d, (r1 - r0) * w.d, 1.0, w.act)
    return a.reshape(r1 - r0, w.d)


def make_u_tokens(w: Workload, tokens) -> np.ndarray:
    """u rows of the listed tokens only."""
    dt = np.float32 if w.act == F32 else np.uint16
    out = np.empty((len(tokens), w.d), dt)
    for j, t in enumerate(tokens):
        normal(w.seed, TID_U, int(t) * w.d, w.d, 1.0, w.act, out=out[j])
    return out


def make_e(w: Workload) -> np.ndarray:
    """centroids e_i ~ N(0, 1/d), [N_r, d] (act dtype); hot experts scaled."""
    dt = np.float32 if w.act == F32 else np.uint16
    out = np.empty((w.n_routed, w.d), dt)
    base = 1.0 / np.sqrt(w.d)
    for i in range(w.n_routed):
        s = base * (w.hot_scale if i in w.hot_experts else 1.0)
        normal(w.seed, TID_E, i * w.d, w.d, s, w.act, out=out[i])
    return out


def make_b(w: Workload) -> np.ndarray:
    if w.bias_range == 0.0:
        return np.zeros(w.n_routed, np.float32)
    return uniform(w.seed, TID_B, 0, w.n_routed, -w.bias_range, w.bias_range)


def make_expert(w: Workload, shared: bool, idx: int):
    """(W1, W3, W2) of one expert: W1, W3 [d_ff, d] ~ N(0, 1/d); W2 [d, d_ff] ~ N(0, 1/d_ff)."""
    dt = weight_dtype(w)
    n = w.d_ff * w.d
    t1, t3, t2 = (TID_SW1, TID_SW3, TID_SW2) if shared else (TID_W1, TID_W3, TID_W2)
    w1 = normal(w.seed, t1, idx * n, n, 1.0 / np.sqrt(w.d), dt).reshape(w.d_ff, w.d)
    w3 = normal(w.seed, t3, idx * n, n, 1.0 / np.sqrt(w.d), dt).reshape(w.d_ff, w.d)
    w2 = normal(w.seed, t2, idx * n, n, 1.0 / np.sqrt(w.d_ff), dt).reshape(w.d, w.d_ff)
    return w1, w3, w2


def make_expert_stack(w: Workload, shared: bool, out1=None, out3=None, out2=None):
    """All experts of one kind stacked: W1, W3 [E, d_ff, d]; W2 [E, d, d_ff]."""
    E = w.n_shared if shared else w.n_routed
    dt = np.float32 if weight_dtype(w) == F32 else np.uint16
    n = w.d_ff * w.d
    t1, t3, t2 = (TID_SW1, TID_SW3, TID_SW2) if shared else (TID_W1, TID_W3, TID_W2)
    w1 = np.empty((E, w.d_ff, w.d), dt) if out1 is None else out1
    w3 = np.empty((E, w.d_ff, w.d), dt) if out3 is None else out3
    w2 = np.empty((E, w.d, w.d_ff), dt) if out2 is None else out2
    wd = weight_dtype(w)
    normal(w.seed, t1, 0, E * n, 1.0 / np.sqrt(w.d), wd, out=w1.reshape(-1))
    normal(w.seed, t3, 0, E * n, 1.0 / np.sqrt(w.d), wd, out=w3.reshape(-1))
    normal(w.seed, t2, 0, E * n, 1.0 / np.sqrt(w.d_ff), wd, out=w2.reshape(-1))
    return w1, w3, w2


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 (exact)."""
    return (a.astype(np.uint32) << 16).view(np.float32)
