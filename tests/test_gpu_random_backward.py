"""Seeded random shapes for the layer backward on the GPU against the oracle (needs an
MI355X).

Six bf16 shapes drawn once from a fixed seed within what the backward accepts (d % 256 == 0,
d_ff % 128 == 0, so both the 256- and the 128-column dh tiles occur): token counts 1..400,
2..64 routed experts, K up to min(N_r, 8), 0..2 shared experts, sigmoid or softmax scoring.
du, dz, dgate and the centroid gradient are checked in full, with the weight gradients of
the most-loaded expert and of every shared expert, within the output tolerances.
"""
import numpy as np
import pytest

import oracle
from mixture_experts_layer_26_amd import inputs as I
from mixture_experts_layer_26_amd.inputs import device as D
from tests.test_gpu_backward import _close, _edge_workload, _f, _run
from tests.gpu_util import log, to_np

pytestmark = pytest.mark.gpu


def _shapes(n=6, seed=20261204):
    rng = np.random.default_rng(seed)
    out = {}
    for i in range(n):
        n_r = int(rng.integers(2, 65))
        k = int(rng.integers(1, min(n_r, 8) + 1))
        kw = dict(T=int(rng.integers(1, 401)), d=int(rng.choice([256, 512, 768])), n_routed=n_r, top_k=k,
                  n_shared=int(rng.integers(0, 3)), d_ff=int(rng.choice([128, 256, 384, 640])), seed=4000 + i)
        score = "softmax" if i % 2 else "sigmoid"
        name = f"b{i}_{score}_T{kw['T']}_d{kw['d']}_nr{n_r}_k{k}_ns{kw['n_shared']}_ff{kw['d_ff']}"
        out[name] = (_edge_workload(name, **kw), score)
    return out


SHAPES = _shapes()


def _check(name, got, ref):
    """Within the output tolerances; a reference that is exactly zero (K = 1: the gate is 1
    whatever the logits, so dz and the centroid gradient vanish) must be matched exactly."""
    if not np.any(ref):
        log(f"[bwd] {name}: reference exactly zero")
        assert not np.any(got), name
    else:
        _close(name, got, ref)


@pytest.mark.parametrize("name", list(SHAPES))
def test_random_backward(name):
    w, score = SHAPES[name]
    log(f"[bwd random] {name}")
    dev = D.upload(w, "cuda")
    L, dout, _ = _run(w, dev, score)
    u, e, b = I.make_u(w), I.make_e(w), I.make_b(w)
    idx_g = to_np(L.topk_idx)
    count = np.bincount(idx_g.ravel(), minlength=w.n_routed)
    hot = int(np.argmax(count))
    routed = {int(i): I.make_expert(w, False, int(i)) for i in np.unique(idx_g)}
    shared = [I.make_expert(w, True, j) for j in range(w.n_shared)]
    g = oracle.layer_backward(u, e, b, routed, shared, dout, top_k=w.top_k, d_ff=w.d_ff, act=w.act, ffn=w.ffn,
                              score=score, grad_routed=[hot], grad_shared=w.n_shared > 0)
    assert np.array_equal(idx_g, g["idx"])
    _check("du", _f(L.du), g["du"])
    _check("dcentroids", _f(L.dcentroids), g["de"])
    _check("dgate", _f(L.dgate), g["dgate"])
    _check("dz", _f(L.dz), g["dz"])
    for m, mname in enumerate(("dW1", "dW3", "dW2")):
        _check(f"{mname}[{hot}] ({count[hot]} rows)", _f(L.dw_routed[m][hot]), g["dw_routed"][hot][m])
    for j in range(w.n_shared):
        for m, mname in enumerate(("dW1", "dW3", "dW2")):
            _check(f"shared {mname}[{j}]", _f(L.dw_shared[m][j]), g["dw_shared"][j][m])
