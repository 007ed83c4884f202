"""Device buffers for one layer shape and the five-call step of the C ABI.

A step is: moe_route -> moe_dispatch -> moe_grouped_ffn -> moe_combine ->
moe_bias_update, all enqueued on one stream with no host synchronisation. The
bias is the caller's persistent state; the update feeds the next step's routing
(DeepSeek-V3 explainer, method section 2: the bias moves at the end of each step).
`backward` runs the three backward calls for the step just taken.
"""
from __future__ import annotations

import torch

from . import abi

_TORCH_ACT = {"f32": torch.float32, "bf16": torch.bfloat16}


class MoeLayer:
    def __init__(self, T: int, d: int, n_routed: int, top_k: int, n_shared: int, d_ff: int,
                 act: str = "bf16", ffn: str = "bf16", device: str = "cuda", score: str = "sigmoid"):
        self.T, self.d, self.n_routed, self.top_k = T, d, n_routed, top_k
        self.n_shared, self.d_ff, self.act, self.ffn = n_shared, d_ff, act, ffn
        self.score = score
        self.device = torch.device(device)
        self.shape = abi.make_shape(T, d, n_routed, top_k, n_shared, d_ff, act, ffn, score)
        adt = _TORCH_ACT[act]
        dev = self.device
        i32 = torch.int32
        self.topk_idx = torch.empty((T, top_k), dtype=i32, device=dev)
        self.topk_gate = torch.empty((T, top_k), dtype=torch.float32, device=dev)
        self.expert_count = torch.empty(n_routed, dtype=i32, device=dev)
        self.expert_offset = torch.empty(n_routed + 1, dtype=i32, device=dev)
        self.sorted_token = torch.empty(T * top_k, dtype=i32, device=dev)
        self.pair_row = torch.empty((T, top_k), dtype=i32, device=dev)
        self.y_routed = torch.empty((T * top_k, d), dtype=adt, device=dev)
        self.y_shared = torch.empty((T, d), dtype=torch.float32, device=dev) if n_shared > 0 else None
        self.out = torch.empty((T, d), dtype=adt, device=dev)
        self.ws_route_bytes = abi.moe_workspace_bytes(self.shape, abi.MOE_CALL_ROUTE)
        self.ws_dispatch_bytes = abi.moe_workspace_bytes(self.shape, abi.MOE_CALL_DISPATCH)
        self.ws_ffn_bytes = abi.moe_workspace_bytes(self.shape, abi.MOE_CALL_GROUPED_FFN)
        self.ws_route = torch.empty(max(1, self.ws_route_bytes), dtype=torch.uint8, device=dev)
        self.ws_dispatch = torch.empty(max(1, self.ws_dispatch_bytes), dtype=torch.uint8, device=dev)
        self.ws_ffn = torch.empty(max(1, self.ws_ffn_bytes), dtype=torch.uint8, device=dev)
        self.routed = None
        self.shared = None
        self._keep = []

    def set_experts(self, routed: tuple, shared: tuple | None, layout: int = abi.MOE_LAYOUT_ROWS):
        """routed/shared: (w1, w3, w2) device tensors, or (w1, w3, w2, s1, s3, s2) for FP8, in
        the given weight layout (ROWS, or TILED as made by pack_experts)."""
        self._keep = [routed, shared]
        w = lambda t: tuple(t) + (None,) * (6 - len(t))
        self.routed = abi.make_expert_set(*w(routed), layout=layout)
        self.shared = abi.make_expert_set(*w(shared), layout=layout) if shared is not None else None

    # -- the five calls ----------------------------------------------------------
    def route(self, u, centroids, bias, stream=None):
        abi.moe_route(self.shape, u, centroids, bias, self.topk_idx, self.topk_gate, self.ws_route,
                      self.ws_route_bytes, stream)

    def dispatch(self, stream=None):
        abi.moe_dispatch(self.shape, self.topk_idx, self.expert_count, self.expert_offset,
                         self.sorted_token, self.pair_row, self.ws_dispatch, self.ws_dispatch_bytes, stream)

    def grouped_ffn(self, u, stream=None):
        abi.moe_grouped_ffn(self.shape, u, self.expert_offset, self.sorted_token, self.routed, self.shared,
                            self.y_routed, self.y_shared, self.ws_ffn, self.ws_ffn_bytes, stream)

    def combine(self, u, stream=None):
        abi.moe_combine(self.shape, u, self.y_routed, self.y_shared, self.pair_row, self.topk_gate, self.out,
                        stream)

    def bias_update(self, bias, gamma: float, stream=None):
        abi.moe_bias_update(self.shape, self.expert_count, gamma, bias, stream)

    # -- backward ----------------------------------------------------------------
    def alloc_backward(self):
        """Buffers of the three backward calls (bf16 layer, row-major weights)."""
        dev, T, d, K, F = self.device, self.T, self.d, self.top_k, self.d_ff
        bf = torch.bfloat16
        self.dy_routed = torch.empty((T * K, d), dtype=bf, device=dev)
        self.dgate = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.dx_routed = torch.empty((T * K, d), dtype=bf, device=dev)
        self.dx_shared = torch.empty((T, d), dtype=torch.float32, device=dev) if self.n_shared > 0 else None
        self.du = torch.empty((T, d), dtype=bf, device=dev)
        self.dcentroids = torch.empty((self.n_routed, d), dtype=bf, device=dev)
        self.dz = torch.empty((T, K), dtype=torch.float32, device=dev)
        mk = lambda E: (torch.empty((E, F, d), dtype=bf, device=dev), torch.empty((E, F, d), dtype=bf, device=dev),
                        torch.empty((E, d, F), dtype=bf, device=dev))
        self.dw_routed = mk(self.n_routed)
        self.dw_shared = mk(self.n_shared) if self.n_shared > 0 else None
        self.g_routed = abi.make_expert_grads(*self.dw_routed)
        self.g_shared = abi.make_expert_grads(*self.dw_shared) if self.dw_shared is not None else None
        self.ws_bwd_bytes = abi.moe_workspace_bytes(self.shape, abi.MOE_CALL_GROUPED_FFN_BACKWARD)
        self.ws_rbwd_bytes = abi.moe_workspace_bytes(self.shape, abi.MOE_CALL_ROUTE_BACKWARD)
        self.ws_bwd = torch.empty(max(1, self.ws_bwd_bytes), dtype=torch.uint8, device=dev)
        self.ws_rbwd = torch.empty(max(1, self.ws_rbwd_bytes), dtype=torch.uint8, device=dev)

    def backward(self, u, centroids, dout, stream=None):
        """Gradients of sum(dout * out) for the step just run (routing held fixed): fills du,
        dcentroids, dz, the weight gradients dw_routed / dw_shared and the intermediates."""
        if not hasattr(self, "du"):
            self.alloc_backward()
        abi.moe_combine_backward(self.shape, dout, self.y_routed, self.pair_row, self.topk_gate, self.dy_routed,
                                 self.dgate, stream)
        abi.moe_grouped_ffn_backward(self.shape, u, dout, self.expert_offset, self.sorted_token, self.routed,
                                     self.shared, self.dy_routed, self.dx_routed, self.dx_shared, self.g_routed,
                                     self.g_shared, self.ws_bwd, self.ws_bwd_bytes, stream)
        abi.moe_route_backward(self.shape, u, centroids, self.topk_idx, self.topk_gate, self.dgate,
                               self.expert_offset, self.sorted_token, self.pair_row, dout, self.dx_routed,
                               self.dx_shared, self.du, self.dcentroids, self.dz, self.ws_rbwd, self.ws_rbwd_bytes,
                               stream)

    def step(self, u, centroids, bias, gamma: float = 0.001, stream=None):
        """One pass of the whole layer; returns the output buffer (overwritten next step)."""
        self.route(u, centroids, bias, stream)
        self.dispatch(stream)
        self.grouped_ffn(u, stream)
        self.combine(u, stream)
        self.bias_update(bias, gamma, stream)
        return self.out

    def capture_step(self, u, centroids, bias, gamma: float = 0.001):
        """The five calls of `step` recorded once into a HIP graph (torch.cuda.CUDAGraph) on
        these tensors; `replay()` then runs a whole step with one launch from the host,
        which is what a batch small enough to be bound by launch latency needs. The calls
        allocate nothing, record no memset and never synchronise, so they can be captured;
        every replay reads u, centroids and bias and writes the layer's buffers and bias as
        an eager step would (bias moves by the update each replay)."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()  # default priority
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                self.step(u, centroids, bias, gamma)
        torch.cuda.current_stream().wait_stream(side)
        return g


def quantize_experts(ws: tuple, stream=None) -> tuple:
    """E4M3 codes and 128x128 block scales of stacked expert weights (w1, w3, w2) ->
    (q1, q3, q2, s1, s3, s2), made by moe_quantize_fp8 on the device."""
    outs_q, outs_s = [], []
    for w in ws:
        E, R, C = w.shape
        q = torch.empty((E, R, C), dtype=torch.uint8, device=w.device)
        s = torch.empty((E, R // 128, C // 128), dtype=torch.float32, device=w.device)
        xt = abi.MOE_BF16 if w.dtype == torch.bfloat16 else abi.MOE_F32
        abi.moe_quantize_fp8(w, xt, E * R, C, 128, 128, q, s, stream)
        outs_q.append(q)
        outs_s.append(s)
    return tuple(outs_q) + tuple(outs_s)


def pack_experts(shape, ws: tuple, stream=None) -> tuple:
    """The TILED layout of stacked expert weights (w1, w3, w2[, s1, s3, s2]) made by
    moe_pack_weights; scales are passed through unchanged."""
    out = []
    for m, w in zip((abi.MOE_W1, abi.MOE_W3, abi.MOE_W2), ws[:3]):
        t = torch.empty_like(w)
        abi.moe_pack_weights(shape, m, w.shape[0], w, t, stream)
        out.append(t)
    return tuple(out) + tuple(ws[3:])
