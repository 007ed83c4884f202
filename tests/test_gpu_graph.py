"""The layer step captured into a HIP graph and replayed (needs an MI355X).

A batch small enough to be bound by launch latency (the tiny layer, a decode batch) runs
its five calls from one graph launch. The calls allocate nothing, record no memset node
and never synchronise, so the capture holds exactly the step's kernels. Each case runs
one eager step from the workload's b, captures the step, then replays it three times;
between the replays the layer's buffers are overwritten and b restored by eager work
with a synchronisation, and every replay must reproduce the eager step bit for bit: the
routing, the dispatch arrays, the output and the updated bias. The kernels are
deterministic, so any difference is a capture or replay fault.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_26_amd import abi
from mixture_experts_layer_26_amd.layer import MoeLayer, pack_experts, quantize_experts
from tests.gpu_util import log, to_np, workload_on_device

pytestmark = pytest.mark.gpu

BUFS = ("topk_idx", "topk_gate", "expert_count", "expert_offset", "sorted_token", "pair_row", "out")
REPLAYS = 3


def _weights(dev, ffn, tiled, shape):
    routed, shared = dev["routed"], dev["shared"]
    if ffn == "fp8":
        routed = quantize_experts(routed)
        shared = quantize_experts(shared) if shared is not None else None
    lay = abi.MOE_LAYOUT_ROWS
    if tiled:
        routed = pack_experts(shape, routed)
        shared = pack_experts(shape, shared) if shared is not None else None
        lay = abi.MOE_LAYOUT_TILED
    return routed, shared, lay


@pytest.mark.parametrize("name,ffn,tiled", [("tiny_f32", "f32", False),
                                            ("mid_bf16", "bf16", True),
                                            ("mid_bf16", "fp8", False),
                                            ("v3_decode_skewed", "bf16", True)])
def test_graph_replays_match_the_eager_step(name, ffn, tiled):
    w, dev = workload_on_device(name)
    log(f"[graph] {name} ffn={ffn} tiled={tiled}")
    L = MoeLayer(w.T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, ffn)
    routed, shared, lay = _weights(dev, ffn, tiled, L.shape)
    L.set_experts(routed, shared, lay)
    b0 = dev["b"]
    bias = b0.clone()
    L.step(dev["u"], dev["e"], bias, w.gamma)
    torch.cuda.synchronize()
    ref = {k: to_np(getattr(L, k)).copy() for k in BUFS}
    ref_b = to_np(bias).copy()
    assert not np.array_equal(ref_b, to_np(b0)), "the step moved the bias"

    bias.copy_(b0)
    g = L.capture_step(dev["u"], dev["e"], bias, w.gamma)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for k in BUFS:  # eager work between replays: stale values a replay must overwrite
            getattr(L, k).fill_(-1)
        bias.copy_(b0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in BUFS:
            assert np.array_equal(to_np(getattr(L, k)), ref[k]), f"{name} replay {r}: {k}"
        assert np.array_equal(to_np(bias).view(np.uint32), ref_b.view(np.uint32)), f"{name} replay {r}: bias"
    log(f"[graph] {name} ffn={ffn}: {REPLAYS} replays bit-identical to the eager step")
