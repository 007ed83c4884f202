"""GPU parity of the softmax router (needs an MI355X).

Softmax scoring follows the DeepSeekMoE forward listing of "DeepSeek モデルアーキテクチャ
徹底解説": the K largest logits z = u . e_i are selected (no bias), and the gates are the
softmax of the selected logits. The ids must match the oracle bit for bit outside the
tie band (logit gap below 1e-5); gates within 4e-6. The gate tolerance: a logit error
dz moves a softmax gate g_k by at most 2 g_k max|dz|, and the fp32 logits (bf16
products, fp32 sums over d <= 7168) stay within about 1e-6 of the exact ones, so the
gates stay within about 2e-6; 4e-6 leaves a factor of two. The bias pointer is NULL
throughout: the softmax router must not read it. The whole layer step then runs on the
softmax routing and is checked on sampled tokens against the oracle's layer.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_26_amd import inputs as I
from mixture_experts_layer_26_amd.layer import MoeLayer
from tests.gpu_util import (FROB_TOL, MAXABS_TOL, check_routing, log, rel_errors, sample_tokens, to_np,
                            workload_on_device)

pytestmark = pytest.mark.gpu

GATE_TOL = 4e-6


def _layer(w):
    return MoeLayer(w.T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, w.ffn, score="softmax")


@pytest.mark.parametrize("name", ["tiny_f32", "mid_bf16", "v3_prefill_bf16", "v3_decode_skewed"])
def test_route_softmax_parity(name):
    w, dev = workload_on_device(name)
    L = _layer(w)
    L.route(dev["u"], dev["e"], None)
    torch.cuda.synchronize()
    u, e = I.make_u(w), I.make_e(w)
    idx, gate, gap, v = oracle.route(u, e, None, w.top_k, w.act, want_v=True, score="softmax")
    gate_gpu = to_np(L.topk_gate)
    diff, n_exempt = check_routing(to_np(L.topk_idx), gate_gpu, idx, gate, gap, v, w.top_k, GATE_TOL)
    same = np.setdiff1d(np.arange(w.T), diff)
    log(f"[route softmax] {name}: exempt {n_exempt}, differing (all exempt) {len(diff)}, "
        f"max gate error {np.max(np.abs(gate_gpu[same] - gate[same])):.2e}")


@pytest.mark.parametrize("name", ["tiny_f32", "mid_bf16"])
def test_layer_softmax_end_to_end(name):
    w, dev = workload_on_device(name)
    L = _layer(w)
    L.set_experts(dev["routed"], dev["shared"])
    bias = dev["b"].clone()
    L.step(dev["u"], dev["e"], bias, w.gamma)
    torch.cuda.synchronize()
    u, e, b = I.make_u(w), I.make_e(w), I.make_b(w)
    idx, gate, gap, v = oracle.route(u, e, None, w.top_k, w.act, want_v=True, score="softmax")
    idx_g = to_np(L.topk_idx)
    diff, _ = check_routing(idx_g, to_np(L.topk_gate), idx, gate, gap, v, w.top_k, GATE_TOL)
    # counts and the bias update follow the GPU's own (valid) selection
    count = oracle.dispatch(idx_g, w.n_routed)[0]
    assert np.array_equal(to_np(L.expert_count), count)
    assert np.array_equal(to_np(bias), oracle.bias_update(count, w.T, w.top_k, w.gamma, b))
    tok = np.setdiff1d(sample_tokens(w.T, 64), diff)
    sel = np.unique(idx[tok])
    routed = {int(i): I.make_expert(w, False, int(i)) for i in sel}
    shared = [I.make_expert(w, True, j) for j in range(w.n_shared)]
    res = oracle.layer(u[tok], e, None, routed, shared, top_k=w.top_k, d_ff=w.d_ff, act=w.act, ffn=w.ffn,
                       score="softmax")
    out = to_np(L.out[torch.from_numpy(tok).cuda()])
    out = I.bf16_bits_to_f32(out) if w.act == "bf16" else out
    frob, mx = rel_errors(out, res["out"])
    log(f"[e2e softmax] {name}: tokens {tok.size} frob {frob:.2e} maxabs {mx:.2e}")
    assert frob <= FROB_TOL and mx <= MAXABS_TOL
