"""moe_grouped_ffn_noalloc against moe_grouped_ffn (needs an MI355X).

The entry point without a workspace runs the same kernels on the library's fixed scratch
array, so given the same routing its outputs must equal the workspace call's bit for bit.
Each case makes two calls in a row on one GPU, the second with fewer tokens, so the second
runs over the scratch contents the first left behind (tile-scheduling state and H). Cases:
the skewed decode batch in bf16 with the tiled weights the benchmark uses (128, then 40
tokens), the mid shape in FP8 (512, then 100 tokens: the FP8 scratch regions of u, H and
their scales), and the tiny fp32 layer (64, then 20 tokens). A shape past the scratch limit
is refused without touching the outputs.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_26_amd import abi
from mixture_experts_layer_26_amd.layer import MoeLayer, pack_experts, quantize_experts
from tests.gpu_util import log, to_np, workload_on_device

pytestmark = pytest.mark.gpu


def _weights(w, dev, ffn, tiled, shape):
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


@pytest.mark.parametrize("name,ffn,tiled,Ts", [("v3_decode_skewed", "bf16", True, (128, 40)),
                                               ("mid_bf16", "fp8", False, (512, 100)),
                                               ("tiny_f32", "f32", False, (64, 20))])
def test_noalloc_matches_workspace_call(name, ffn, tiled, Ts):
    w, dev = workload_on_device(name)
    weights = None
    for T in Ts:
        log(f"[noalloc] {name} ffn={ffn} T={T}")
        L = MoeLayer(T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, ffn)
        need = abi.moe_workspace_bytes(L.shape, abi.MOE_CALL_GROUPED_FFN)
        assert 0 < need <= abi.MOE_NOALLOC_SCRATCH_BYTES
        if weights is None:
            weights = _weights(w, dev, ffn, tiled, L.shape)
        L.set_experts(weights[0], weights[1], weights[2])
        u = dev["u"][:T]
        L.route(u, dev["e"], dev["b"])
        L.dispatch()
        L.grouped_ffn(u)
        torch.cuda.synchronize()
        y_ref = to_np(L.y_routed).copy()
        ysh_ref = to_np(L.y_shared).copy() if L.y_shared is not None else None
        L.y_routed.fill_(-7.0)
        if L.y_shared is not None:
            L.y_shared.fill_(-7.0)
        abi.moe_grouped_ffn_noalloc(L.shape, u, L.expert_offset, L.sorted_token, L.routed, L.shared, L.y_routed,
                                    L.y_shared)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(L.y_routed), y_ref), f"{name} T={T}: y_routed"
        if ysh_ref is not None:
            assert np.array_equal(to_np(L.y_shared), ysh_ref), f"{name} T={T}: y_shared"
        log(f"[noalloc] {name} T={T}: outputs bit-identical to the workspace call "
            f"(scratch used {need} of {abi.MOE_NOALLOC_SCRATCH_BYTES} bytes)")


def test_noalloc_refuses_shapes_past_the_limit():
    w, dev = workload_on_device("tiny_f32")
    T = 4096
    L = MoeLayer(T, 7168, 256, 8, 1, 2048, "bf16", "bf16")
    assert abi.moe_workspace_bytes(L.shape, abi.MOE_CALL_GROUPED_FFN) > abi.MOE_NOALLOC_SCRATCH_BYTES
    es = abi.make_expert_set(1 << 12, 1 << 12, 1 << 12)
    L.y_routed.fill_(3.0)
    with pytest.raises(abi.MoeError) as err:
        abi.moe_grouped_ffn_noalloc(L.shape, L.out, L.expert_offset, L.sorted_token, es, es, L.y_routed,
                                    L.y_shared)
    assert err.value.status == abi.MOE_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool((L.y_routed == 3.0).all())
