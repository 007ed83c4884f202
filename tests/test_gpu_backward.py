"""GPU parity of the layer backward (needs an MI355X).

The forward step runs through the C ABI, then moe_combine_backward,
moe_grouped_ffn_backward and moe_route_backward with an output gradient dout ~ N(0, 1)
(bf16, the generator's stream of a later batch), and the gradients are compared with the
oracle's layer_backward on the same inputs: gradients of sum(dout * h') with the routing
held fixed, h' the layer of the DeepSeek-V3 explainer's method section 2, bf16 operands
with h, da, dv and the routed rows' dy rounded to bf16 ("gradients in BF16").

Tolerances are those of the forward outputs (relative Frobenius 5e-3, max-abs 2e-2 of the
largest reference magnitude) for every gradient tensor; the routing must match the
oracle's on every token (no token of these inputs falls in the tie band). The mid shape
is checked in full (du, dz, dgate, the centroid gradient, the shared experts' and six
routed experts' weight gradients); the V3 shapes on sampled tokens and experts, with the
oracle evaluating only the rows those need; experts no token chose must get zero weight
gradients. Edge cases: one token, a ragged token count and no shared experts.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_26_amd import inputs as I
from mixture_experts_layer_26_amd.layer import MoeLayer
from tests.gpu_util import FROB_TOL, MAXABS_TOL, log, rel_errors, sample_tokens, to_dev, to_np, workload_on_device

pytestmark = pytest.mark.gpu


def _f(x):
    """device tensor -> float64 numpy (bf16 widened exactly)"""
    a = to_np(x)
    return I.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _close(name, got, ref):
    frob, mx = rel_errors(got, ref)
    log(f"[bwd] {name}: frob {frob:.2e} maxabs {mx:.2e}")
    assert frob <= FROB_TOL and mx <= MAXABS_TOL, name


def _run(w, dev, score="sigmoid"):
    L = MoeLayer(w.T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, w.ffn, score=score)
    L.set_experts(dev["routed"], dev["shared"])
    L.route(dev["u"], dev["e"], dev["b"])
    L.dispatch()
    L.grouped_ffn(dev["u"])
    L.combine(dev["u"])
    dout = I.make_u(w, batch=99)
    dout_dev = to_dev(dout, bf16=True)
    L.backward(dev["u"], dev["e"], dout_dev)
    torch.cuda.synchronize()
    return L, dout, dout_dev


@pytest.mark.parametrize("score", ["sigmoid", "softmax"])
def test_backward_mid_full(score):
    w, dev = workload_on_device("mid_bf16", 256)
    L, dout, _ = _run(w, dev, score)
    u, e, b = I.make_u(w), I.make_e(w), I.make_b(w)
    idx_g = to_np(L.topk_idx)
    count = np.bincount(idx_g.ravel(), minlength=w.n_routed)
    order = np.argsort(count, kind="stable")
    pick = sorted({int(order[0]), int(order[1]), int(order[w.n_routed // 2]), int(order[-2]), int(order[-1]),
                   int(idx_g[0, 0])})
    routed = {i: I.make_expert(w, False, i) for i in range(w.n_routed)}
    shared = [I.make_expert(w, True, j) for j in range(w.n_shared)]
    g = oracle.layer_backward(u, e, b, routed, shared, dout, top_k=w.top_k, d_ff=w.d_ff, act=w.act, ffn=w.ffn,
                              score=score, grad_routed=pick, grad_shared=True)
    assert np.array_equal(idx_g, g["idx"]), "routing differs from the oracle"
    _close("du", _f(L.du), g["du"])
    _close("dcentroids", _f(L.dcentroids), g["de"])
    _close("dgate", _f(L.dgate), g["dgate"])
    _close("dz", _f(L.dz), g["dz"])
    for i in pick:
        for m, name in enumerate(("dW1", "dW3", "dW2")):
            _close(f"{name}[{i}] ({count[i]} rows)", _f(L.dw_routed[m][i]), g["dw_routed"][i][m])
    for j in range(w.n_shared):
        for m, name in enumerate(("dW1", "dW3", "dW2")):
            _close(f"shared {name}[{j}]", _f(L.dw_shared[m][j]), g["dw_shared"][j][m])


def test_backward_v3_prefill_sampled():
    w, dev = workload_on_device("v3_prefill_bf16")
    L, dout, _ = _run(w, dev)
    u, e, b = I.make_u(w), I.make_e(w), I.make_b(w)
    idx_g = to_np(L.topk_idx)
    shared = [I.make_expert(w, True, j) for j in range(w.n_shared)]
    # sampled tokens: du, dgate and dz are token-local
    tok = sample_tokens(w.T, 16)
    need = sorted(set(idx_g[tok].ravel().tolist()))
    routed = {i: I.make_expert(w, False, i) for i in need}
    g = oracle.layer_backward(u[tok], e, b, routed, shared, dout[tok], top_k=w.top_k, d_ff=w.d_ff, act=w.act,
                              ffn=w.ffn, want_de=False)
    assert np.array_equal(idx_g[tok], g["idx"])
    _close("du (sampled tokens)", _f(L.du)[tok], g["du"])
    _close("dgate (sampled tokens)", _f(L.dgate)[tok], g["dgate"])
    _close("dz (sampled tokens)", _f(L.dz)[tok], g["dz"])
    # two experts' weight gradients: all their rows (every token is routed by the oracle)
    count = np.bincount(idx_g.ravel(), minlength=w.n_routed)
    pick = [int(np.argmax(count)), int(np.argmin(count))]
    g2 = oracle.layer_backward(u, e, b, {i: I.make_expert(w, False, i) for i in pick}, shared, dout,
                               top_k=w.top_k, d_ff=w.d_ff, act=w.act, ffn=w.ffn, want_du=False, want_de=False,
                               grad_routed=pick)
    assert np.array_equal(idx_g, g2["idx"])
    for i in pick:
        for m, name in enumerate(("dW1", "dW3", "dW2")):
            _close(f"{name}[{i}] ({count[i]} rows)", _f(L.dw_routed[m][i]), g2["dw_routed"][i][m])


def test_backward_v3_decode_skewed():
    """Skewed decode batch: du, dz, dgate and the centroid gradient in full; the hottest
    expert's weight gradients; zero weight gradients for an expert with no rows."""
    w, dev = workload_on_device("v3_decode_skewed")
    L, dout, _ = _run(w, dev)
    u, e, b = I.make_u(w), I.make_e(w), I.make_b(w)
    idx_g = to_np(L.topk_idx)
    count = np.bincount(idx_g.ravel(), minlength=w.n_routed)
    hot = int(np.argmax(count))
    unused = np.nonzero(count == 0)[0]
    need = sorted(set(idx_g.ravel().tolist()))
    routed = {i: I.make_expert(w, False, i) for i in need}
    shared = [I.make_expert(w, True, j) for j in range(w.n_shared)]
    g = oracle.layer_backward(u, e, b, routed, shared, dout, top_k=w.top_k, d_ff=w.d_ff, act=w.act, ffn=w.ffn,
                              grad_routed=[hot])
    assert np.array_equal(idx_g, g["idx"])
    _close("du", _f(L.du), g["du"])
    _close("dcentroids", _f(L.dcentroids), g["de"])
    _close("dgate", _f(L.dgate), g["dgate"])
    _close("dz", _f(L.dz), g["dz"])
    for m, name in enumerate(("dW1", "dW3", "dW2")):
        _close(f"{name}[{hot}] ({count[hot]} rows)", _f(L.dw_routed[m][hot]), g["dw_routed"][hot][m])
    assert unused.size > 0
    for m in range(3):
        assert not torch.any(L.dw_routed[m][int(unused[0])].float() != 0)
    assert not torch.any(L.dcentroids[int(unused[0])].float() != 0)


def test_backward_deterministic():
    w, dev = workload_on_device("mid_bf16", 256)
    L, _, dout_dev = _run(w, dev)
    first = [t.clone() for t in (L.du, L.dcentroids, L.dz, *L.dw_routed, *L.dw_shared)]
    L.backward(dev["u"], dev["e"], dout_dev)
    torch.cuda.synchronize()
    again = (L.du, L.dcentroids, L.dz, *L.dw_routed, *L.dw_shared)
    for a, b in zip(first, again):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def _edge_workload(name, **kw):
    base = dict(I.WORKLOADS["mid_bf16"].__dict__)
    base.update(kw)
    base["name"] = name
    return I.Workload(**base)


BWD_EDGES = {
    "single_token": _edge_workload("bwd_single_token", T=1),
    "ragged_333": _edge_workload("bwd_ragged_333", T=333),
    "no_shared": _edge_workload("bwd_no_shared", T=300, d=1024, n_routed=32, top_k=4, n_shared=0, d_ff=512,
                                seed=2711),
}


@pytest.mark.parametrize("case", list(BWD_EDGES))
def test_backward_edge_cases(case):
    """One token, a ragged token count (partial row tiles in every backward launch) and no
    shared experts (no dx_shared, no shared weight gradients): du, dz, dgate and the centroid
    gradient in full, and the weight gradients of the most-loaded expert, against the oracle."""
    from mixture_experts_layer_26_amd.inputs import device as D
    w = BWD_EDGES[case]
    dev = D.upload(w, "cuda")
    L, dout, _ = _run(w, dev)
    u, e, b = I.make_u(w), I.make_e(w), I.make_b(w)
    idx_g = to_np(L.topk_idx)
    count = np.bincount(idx_g.ravel(), minlength=w.n_routed)
    hot = int(np.argmax(count))
    routed = {int(i): I.make_expert(w, False, int(i)) for i in np.unique(idx_g)}
    shared = [I.make_expert(w, True, j) for j in range(w.n_shared)]
    g = oracle.layer_backward(u, e, b, routed, shared, dout, top_k=w.top_k, d_ff=w.d_ff, act=w.act, ffn=w.ffn,
                              grad_routed=[hot], grad_shared=w.n_shared > 0)
    assert np.array_equal(idx_g, g["idx"])
    log(f"[bwd edge] {case}: T={w.T} N_s={w.n_shared}")
    _close("du", _f(L.du), g["du"])
    _close("dcentroids", _f(L.dcentroids), g["de"])
    _close("dgate", _f(L.dgate), g["dgate"])
    _close("dz", _f(L.dz), g["dz"])
    for m, name in enumerate(("dW1", "dW3", "dW2")):
        _close(f"{name}[{hot}] ({count[hot]} rows)", _f(L.dw_routed[m][hot]), g["dw_routed"][hot][m])
    for j in range(w.n_shared):
        for m, name in enumerate(("dW1", "dW3", "dW2")):
            _close(f"shared {name}[{j}]", _f(L.dw_shared[m][j]), g["dw_shared"][j][m])
    if w.n_shared == 0:
        assert L.dx_shared is None and L.dw_shared is None
