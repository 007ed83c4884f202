"""GPU tests of the tiled weight layout (needs an MI355X).

moe_pack_weights only reorders bytes: its output is compared bit for bit with torch's
reshape/permute of the same tensor. The grouped FFN must then give bit-identical
outputs from either layout: bf16 and FP8 on the mid shape (two shared experts, an odd
number of 128-wide K-steps in the FP8 down projection), the skewed decode batch at the
V3 shape, and the V3 prefill layer in bf16 and FP8 (the configurations the benchmark
times). The row-major path itself is checked against the oracle in test_gpu_parity.py
and test_gpu_fp8.py.
"""
import pytest
import torch

from mixture_experts_layer_26_amd import abi
from mixture_experts_layer_26_amd import inputs as I
from mixture_experts_layer_26_amd.layer import MoeLayer, pack_experts, quantize_experts
from tests.gpu_util import log, workload_on_device

pytestmark = pytest.mark.gpu


def _tiled_ref(x: torch.Tensor, R: int, ks: int) -> torch.Tensor:
    """[E, N, K] -> [E][N/R][K/ks][R][ks], flattened back to [E, N, K]."""
    E, N, K = x.shape
    return x.view(E, N // R, R, K // ks, ks).permute(0, 1, 3, 2, 4).contiguous().view(E, N, K)


@pytest.mark.parametrize("ffn", ["bf16", "fp8"])
def test_pack_matches_permute(ffn):
    d, d_ff, E = 512, 384, 3
    shape = abi.make_shape(T=16, d=d, n_routed=4, top_k=2, n_shared=1, d_ff=d_ff, act="bf16", ffn=ffn)
    ks = 64 if ffn == "bf16" else 128  # 128 bytes of K
    gen = torch.Generator(device="cuda").manual_seed(7)
    for m, (N, K, R) in [(abi.MOE_W1, (d_ff, d, 128)), (abi.MOE_W3, (d_ff, d, 128)), (abi.MOE_W2, (d, d_ff, 256))]:
        bits = torch.randint(-32768, 32767, (E, N, K), device="cuda", generator=gen, dtype=torch.int32)
        x = bits.to(torch.int16) if ffn == "bf16" else (bits & 0xFF).to(torch.uint8)
        y = torch.empty_like(x)
        abi.moe_pack_weights(shape, m, E, x, y)
        torch.cuda.synchronize()
        assert torch.equal(y, _tiled_ref(x, R, ks)), (ffn, m)


@pytest.mark.parametrize("base,T,ffn", [("mid_bf16", 512, "bf16"), ("mid_bf16", 512, "fp8"),
                                        ("v3_decode_skewed", None, "bf16"), ("v3_prefill_bf16", None, "bf16"),
                                        ("v3_prefill_bf16", None, "fp8")])
def test_tiled_layout_bit_identical(base, T, ffn):
    wb = I.WORKLOADS[base]
    w = wb.with_tokens(T) if T is not None else wb
    _, dev = workload_on_device(base, T)
    L = MoeLayer(w.T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, ffn)
    if ffn == "fp8":
        routed = quantize_experts(dev["routed"])
        shared = quantize_experts(dev["shared"]) if dev["shared"] is not None else None
    else:
        routed, shared = dev["routed"], dev["shared"]
    L.set_experts(routed, shared)
    bias = dev["b"].clone()
    L.route(dev["u"], dev["e"], bias)
    L.dispatch()
    L.grouped_ffn(dev["u"])
    torch.cuda.synchronize()
    y_rows, s_rows = L.y_routed.clone(), L.y_shared.clone()
    L.set_experts(pack_experts(L.shape, routed), pack_experts(L.shape, shared) if shared is not None else None,
                  layout=abi.MOE_LAYOUT_TILED)
    L.y_routed.fill_(0)
    L.y_shared.fill_(0)
    L.grouped_ffn(dev["u"])
    torch.cuda.synchronize()
    same_r = torch.equal(L.y_routed.view(torch.int16) if L.y_routed.dtype == torch.bfloat16 else L.y_routed,
                         y_rows.view(torch.int16) if y_rows.dtype == torch.bfloat16 else y_rows)
    same_s = torch.equal(L.y_shared, s_rows)
    log(f"[layout] {w.name} {ffn}: tiled == rows: routed {same_r}, shared {same_s}")
    assert same_r and same_s
