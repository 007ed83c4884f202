"""Multi-step auxiliary-loss-free balancing on the GPU (needs an MI355X).

The end-of-step rule of the DeepSeek-V3 explainer (method section 2: b_i falls by gamma
when expert i is overloaded and rises by gamma when underloaded) applied over S steps
of fresh token batches, the bias carried on the device from step to step, through the
whole layer step (route, dispatch, grouped FFN, combine, bias update). Each step is
checked against the oracle given the same bias: routing (tie band exempt), counts and
the updated bias bit for bit. Over the run: every move is exactly +-gamma in fp32 (or
none at the mean load) with the sign of (mean - load), so |b_S - b_0| <= S * gamma.
The max/mean expert load of each step is logged.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_26_amd import inputs as I
from mixture_experts_layer_26_amd.layer import MoeLayer
from tests.gpu_util import check_routing, log, to_dev, to_np, workload_on_device

pytestmark = pytest.mark.gpu

STEPS = 6


def test_bias_loop_over_fresh_batches():
    w = I.WORKLOADS["mid_bf16"]
    _, dev = workload_on_device("mid_bf16")
    L = MoeLayer(w.T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, w.ffn)
    L.set_experts(dev["routed"], dev["shared"])
    e = I.make_e(w)
    b0 = I.make_b(w)
    bias = to_dev(b0.copy())
    mean = w.T * w.top_k / w.n_routed
    ratios = []
    for step in range(STEPS):
        u = I.make_u(w, batch=step + 1)
        u_dev = to_dev(u, bf16=True)
        b_before = to_np(bias).copy()
        L.step(u_dev, dev["e"], bias, w.gamma)
        torch.cuda.synchronize()
        # routing given the same bias, then counts and the update, bit for bit
        idx, gate, gap, v = oracle.route(u, e, b_before, w.top_k, w.act, want_v=True)
        idx_gpu = to_np(L.topk_idx)
        check_routing(idx_gpu, to_np(L.topk_gate), idx, gate, gap, v, w.top_k)
        count_gpu = to_np(L.expert_count)
        count_ref, _, _, _ = oracle.dispatch(idx_gpu, w.n_routed)
        assert np.array_equal(count_gpu, count_ref)
        b_after = to_np(bias)
        assert np.array_equal(b_after.view(np.uint32),
                              oracle.bias_update(count_gpu, w.T, w.top_k, w.gamma, b_before).view(np.uint32))
        # each move is +-gamma in fp32, towards the mean load
        load = count_gpu.astype(np.int64) * w.n_routed
        total = w.T * w.top_k
        want = np.where(load > total, np.float32(b_before - np.float32(w.gamma)),
                        np.where(load < total, np.float32(b_before + np.float32(w.gamma)), b_before))
        assert np.array_equal(b_after, want.astype(np.float32))
        ratios.append(count_gpu.max() / mean)
        log(f"[balance] step {step}: max/mean load {ratios[-1]:.3f}, min/mean {count_gpu.min() / mean:.3f}")
    drift = np.abs(to_np(bias).astype(np.float64) - b0.astype(np.float64))
    assert np.all(drift <= STEPS * w.gamma * (1 + 1e-5))
    log(f"[balance] max |b_S - b_0| = {drift.max():.6f} (bound {STEPS * w.gamma})")
