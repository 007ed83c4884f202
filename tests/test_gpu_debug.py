"""MOE_DEBUG=1 index validation (needs an MI355X).

With MOE_DEBUG=1 the calls that take index arrays from earlier calls check them on the
device first and return MOE_ERR_INVALID_ARG, launching nothing else, when one is out of
range. Each corrupted case below is built so that even an unchecked launch would stay
inside allocated memory: the buffers a bad index would reach get spare rows, and the
offsets case only shortens the total.
"""
import pytest
import torch

from mixture_experts_layer_26_amd import abi
from mixture_experts_layer_26_amd.layer import MoeLayer
from tests.gpu_util import log, workload_on_device

pytestmark = pytest.mark.gpu


def _run_step(w, dev):
    L = MoeLayer(w.T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, w.ffn)
    L.set_experts(dev["routed"], dev["shared"])
    bias = dev["b"].clone()
    L.step(dev["u"], dev["e"], bias, w.gamma)
    torch.cuda.synchronize()
    return L


def _expect_invalid(fn):
    with pytest.raises(abi.MoeError) as ex:
        fn()
    assert ex.value.status == abi.MOE_ERR_INVALID_ARG


def test_debug_checks(monkeypatch):
    w, dev = workload_on_device("mid_bf16", 256)
    L0 = _run_step(w, dev)
    ref = L0.out.view(torch.int16).clone()
    monkeypatch.setenv("MOE_DEBUG", "1")
    L = _run_step(w, dev)  # valid inputs pass every check and give the same result
    assert torch.equal(L.out.view(torch.int16), ref)
    P, T, d, n_r = w.T * w.top_k, w.T, w.d, w.n_routed

    # combine: pair_row past the routed rows (y_routed has 8 spare rows)
    y_pad = torch.zeros((P + 8, d), dtype=torch.bfloat16, device="cuda")
    y_pad[:P].copy_(L.y_routed)
    bad_pr = L.pair_row.clone()
    bad_pr.view(-1)[5] = P + 3
    out = torch.full((T, d), 7.0, dtype=torch.bfloat16, device="cuda")
    _expect_invalid(lambda: abi.moe_combine(L.shape, dev["u"], y_pad, L.y_shared, bad_pr, L.topk_gate, out))
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0)), "nothing may be written after a failed check"

    # dispatch: an expert id of n_r (the outputs have spare entries)
    bad_idx = L.topk_idx.clone()
    bad_idx.view(-1)[7] = n_r
    count = torch.zeros(n_r + 8, dtype=torch.int32, device="cuda")
    offs = torch.zeros(n_r + 8, dtype=torch.int32, device="cuda")
    st = torch.zeros(P + 64, dtype=torch.int32, device="cuda")
    pr = torch.zeros(P + 64, dtype=torch.int32, device="cuda")
    _expect_invalid(lambda: abi.moe_dispatch(L.shape, bad_idx, count, offs, st, pr, L.ws_dispatch,
                                             L.ws_dispatch_bytes))

    # grouped FFN: a sorted token of T (u has a spare row) and a short offset total
    u_pad = torch.zeros((T + 1, d), dtype=torch.bfloat16, device="cuda")
    u_pad[:T].copy_(dev["u"])
    bad_st = L.sorted_token.clone()
    bad_st[3] = T
    _expect_invalid(lambda: abi.moe_grouped_ffn(L.shape, u_pad, L.expert_offset, bad_st, L.routed, L.shared,
                                                L.y_routed, L.y_shared, L.ws_ffn, L.ws_ffn_bytes))
    bad_off = L.expert_offset.clone()
    bad_off[n_r] = P - 1
    _expect_invalid(lambda: abi.moe_grouped_ffn(L.shape, dev["u"], bad_off, L.sorted_token, L.routed, L.shared,
                                                L.y_routed, L.y_shared, L.ws_ffn, L.ws_ffn_bytes))
    torch.cuda.synchronize()

    # and the valid arrays still pass afterwards
    abi.moe_grouped_ffn(L.shape, dev["u"], L.expert_offset, L.sorted_token, L.routed, L.shared, L.y_routed,
                        L.y_shared, L.ws_ffn, L.ws_ffn_bytes)
    abi.moe_combine(L.shape, dev["u"], L.y_routed, L.y_shared, L.pair_row, L.topk_gate, L.out)
    torch.cuda.synchronize()
    assert torch.equal(L.out.view(torch.int16), ref)
    log("[debug] bad pair_row, topk_idx, sorted_token and offsets rejected; valid arrays pass")
