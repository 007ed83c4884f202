"""The layer backward with TILED weights against the same backward with row-major weights
(needs an MI355X).

moe_grouped_ffn_backward accepts either weight layout and writes the weight gradients in
the weights' own layout. Only the addresses differ between the two (the same values reach
LDS in the same places and the MFMAs run in the same order), so every output must be bit
for bit the row-major run's, and the tiled weight gradients must equal the row-major ones
packed with moe_pack_weights. Two shapes: the mid workload's (d_ff = 1408, whose dh launch
takes 128-column tiles) and a small one with d_ff a multiple of 256 (256-column dh tiles).
The row-major backward itself is checked against the oracle in test_gpu_backward.py.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_26_amd import abi
from mixture_experts_layer_26_amd import inputs as I
from mixture_experts_layer_26_amd.inputs import device as D
from mixture_experts_layer_26_amd.layer import MoeLayer, pack_experts
from tests.gpu_util import log, to_dev, to_np, workload_on_device

pytestmark = pytest.mark.gpu

SMALL = I.Workload("bwd_tiled_small", T=300, d=512, n_routed=8, top_k=2, n_shared=1, d_ff=512, act="bf16",
                   ffn="bf16", seed=2711, bias_range=0.01)


def _step_and_backward(w, dev, routed, shared, layout, dout_dev):
    L = MoeLayer(w.T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, w.ffn)
    L.set_experts(routed, shared, layout=layout)
    L.route(dev["u"], dev["e"], dev["b"].clone())
    L.dispatch()
    L.grouped_ffn(dev["u"])
    L.combine(dev["u"])
    L.backward(dev["u"], dev["e"], dout_dev)
    torch.cuda.synchronize()
    return L


def _same(name, a, b):
    assert np.array_equal(to_np(a), to_np(b)), f"{name} differs between the layouts"


@pytest.mark.parametrize("case", ["mid", "small"])
def test_backward_tiled_bit_identical(case):
    if case == "mid":
        w, dev = workload_on_device("mid_bf16", 256)
    else:
        w, dev = SMALL, D.upload(SMALL, "cuda")
    log(f"[bwd tiled] {case}: T={w.T} d={w.d} N_r={w.n_routed} K={w.top_k} N_s={w.n_shared} d_ff={w.d_ff}")
    dout_dev = to_dev(I.make_u(w, batch=99), bf16=True)
    rows = _step_and_backward(w, dev, dev["routed"], dev["shared"], abi.MOE_LAYOUT_ROWS, dout_dev)
    shape = rows.shape
    tr, ts = pack_experts(shape, dev["routed"]), pack_experts(shape, dev["shared"])
    tiled = _step_and_backward(w, dev, tr, ts, abi.MOE_LAYOUT_TILED, dout_dev)
    for name in ("out", "du", "dcentroids", "dz", "dgate", "dx_routed", "dx_shared", "dy_routed"):
        _same(name, getattr(rows, name), getattr(tiled, name))
    for kind, g_rows, g_tiled in (("routed", rows.dw_routed, tiled.dw_routed), ("shared", rows.dw_shared, tiled.dw_shared)):
        packed = pack_experts(shape, g_rows)
        torch.cuda.synchronize()
        for m, name in enumerate(("dW1", "dW3", "dW2")):
            _same(f"{kind} {name}", packed[m], g_tiled[m])
    log(f"[bwd tiled] {case}: every output and weight gradient bit-identical")
