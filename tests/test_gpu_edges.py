"""Edge cases of the whole layer step on the GPU (needs an MI355X).

Each case runs the five calls (route, dispatch, grouped FFN, combine, bias update) through
the C ABI on a shape or routing that the main workloads do not reach, and checks them as
test_gpu_parity.py does: routing bit for bit outside the tie band, counts, permutation and
bias bit for bit, and the output on sampled tokens against the oracle within the output
tolerances (relative Frobenius 5e-3, max-abs 2e-2 of the largest reference magnitude).

- a single token; a ragged token count (333: partial router, GEMM and shared-expert tiles);
- no shared experts (the y_shared-free paths);
- K = N_r (every expert on every token) and the largest K (16 of 256 experts);
- every token on the same K experts (bias +10 on experts 0..K-1, which the sigmoid scores in
  (0, 1) cannot overturn): K groups of T rows, many row blocks each, every other expert empty;
- FP8 experts with a ragged token count; fp32 with a ragged token count;
- the largest number of shared experts (8), in bf16 and FP8: the shared down-projection's K
  range runs over eight weight matrices;
- FP8 with d_ff = 128: the routed down-projection has a single 128-wide K-step, and the
  shared one (two experts) two K segments of one step each;
- fp32 without shared experts (no y_shared buffer).
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_26_amd import inputs as I
from mixture_experts_layer_26_amd.inputs import device as D
from mixture_experts_layer_26_amd.layer import MoeLayer, quantize_experts
from tests.gpu_util import FROB_TOL, MAXABS_TOL, check_routing, log, rel_errors, sample_tokens, to_dev, to_np

pytestmark = pytest.mark.gpu

MID = I.WORKLOADS["mid_bf16"]


def _w(name, base=MID, **kw):
    d = dict(base.__dict__)
    d.update(kw)
    d["name"] = name
    return I.Workload(**d)


CASES = {
    "single_token": _w("single_token", T=1),
    "ragged_333": _w("ragged_333", T=333),
    "no_shared": _w("no_shared", T=300, d=1024, n_routed=32, top_k=4, n_shared=0, d_ff=512, seed=2701),
    "k_equals_n": _w("k_equals_n", T=100, d=256, n_routed=16, top_k=16, n_shared=1, d_ff=128, seed=2702),
    "max_top_k": _w("max_top_k", T=200, d=512, n_routed=256, top_k=16, n_shared=1, d_ff=256, seed=2703),
    "all_on_k_experts": _w("all_on_k_experts", T=2048, seed=2704),
    "fp8_ragged_333": _w("fp8_ragged_333", T=333, ffn="fp8"),
    "max_shared_8": _w("max_shared_8", T=200, d=512, n_routed=32, top_k=4, n_shared=8, d_ff=256, seed=2705),
    "fp8_max_shared_8": _w("fp8_max_shared_8", T=200, d=512, n_routed=32, top_k=4, n_shared=8, d_ff=256,
                           seed=2705, ffn="fp8"),
    "f32_ragged_77": _w("f32_ragged_77", base=I.WORKLOADS["tiny_f32"], T=77),
    "f32_no_shared": _w("f32_no_shared", base=I.WORKLOADS["tiny_f32"], T=100, d=128, n_routed=8, top_k=2,
                        n_shared=0, d_ff=64, seed=2708),
    "fp8_dff_128": _w("fp8_dff_128", T=300, d=256, n_routed=16, top_k=4, n_shared=2, d_ff=128, seed=2706,
                      ffn="fp8"),
}


def _q_host(tup):
    out = [oracle.quantize(a, "bf16", 128, 128) for a in tup]
    return (out[0][0], out[1][0], out[2][0], out[0][1], out[1][1], out[2][1])


@pytest.mark.parametrize("case", list(CASES))
def test_layer_edge_case(case):
    w = CASES[case]
    b = I.make_b(w)
    if case == "all_on_k_experts":
        b = b.copy()
        b[:w.top_k] += 10.0
    run_layer_case(w, b, case)
    if case == "all_on_k_experts":
        counts = np.bincount(oracle.route(I.make_u(w), I.make_e(w), b, w.top_k, w.act)[0].ravel(),
                             minlength=w.n_routed)
        assert np.all(counts[:w.top_k] == w.T) and not np.any(counts[w.top_k:])


def run_layer_case(w, b, case):
    """One layer step on the GPU against the oracle: routing, dispatch and bias bit for bit
    (outside the tie band), the output on sampled tokens within the output tolerances."""
    log(f"[edge] {case}: T={w.T} d={w.d} N_r={w.n_routed} K={w.top_k} N_s={w.n_shared} d_ff={w.d_ff} "
        f"ffn={w.ffn}")
    bw = w if w.ffn != "fp8" else _w(w.name, base=w, ffn="bf16")  # FP8 codes come from the bf16 tensors
    dev = D.upload(bw, "cuda")
    routed, shared = dev["routed"], dev["shared"]
    if w.ffn == "fp8":
        routed = quantize_experts(routed)
        shared = quantize_experts(shared) if shared is not None else None
    L = MoeLayer(w.T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, w.ffn)
    L.set_experts(routed, shared)
    bias = to_dev(b.copy())
    L.step(dev["u"], dev["e"], bias, w.gamma)
    torch.cuda.synchronize()

    u, e = I.make_u(w), I.make_e(w)
    idx, gate, gap, v = oracle.route(u, e, b, w.top_k, w.act, want_v=True)
    idx_g = to_np(L.topk_idx)
    diff, n_exempt = check_routing(idx_g, to_np(L.topk_gate), idx, gate, gap, v, w.top_k)
    want = oracle.dispatch(idx_g, w.n_routed)
    got = [to_np(t) for t in (L.expert_count, L.expert_offset, L.sorted_token, L.pair_row)]
    for g, r, what in zip(got, want, ("count", "offset", "sorted_token", "pair_row")):
        assert np.array_equal(g.reshape(r.shape), r), what
    assert np.array_equal(to_np(bias), oracle.bias_update(want[0], w.T, w.top_k, w.gamma, b))

    tok = np.setdiff1d(sample_tokens(w.T, 48), diff)
    need = sorted(set(idx[tok].ravel().tolist()))
    mk = (lambda t: _q_host(t)) if w.ffn == "fp8" else (lambda t: t)
    r_host = {i: mk(I.make_expert(bw, False, i)) for i in need}
    s_host = [mk(I.make_expert(bw, True, j)) for j in range(w.n_shared)]
    res = oracle.layer(u[tok], e, b, r_host, s_host, top_k=w.top_k, d_ff=w.d_ff, act=w.act, ffn=w.ffn)
    out = to_np(L.out[torch.from_numpy(tok).cuda()])
    out = I.bf16_bits_to_f32(out) if w.act == "bf16" else out
    frob, mx = rel_errors(out, res["out"])
    log(f"[edge] {case}: tokens {tok.size} exempt {n_exempt} differing {len(diff)} frob {frob:.2e} "
        f"maxabs {mx:.2e}")
    assert frob <= FROB_TOL and mx <= MAXABS_TOL


def test_empty_batch():
    """T = 0 through the forward and backward calls: counts and offsets zero, the bias
    unchanged (every count equals the mean, 0), zero weight and centroid gradients, MOE_OK
    everywhere, with NULL pointers for the empty token arrays."""
    w = _w("empty", T=0, d=512, n_routed=16, top_k=4, n_shared=2, d_ff=256, seed=2707)
    ws = _w("empty_weights", base=w, T=4)  # the same tensors' generator needs a token count
    dev = D.upload(ws, "cuda")
    log(f"[edge] empty batch: d={w.d} N_r={w.n_routed} K={w.top_k} N_s={w.n_shared} d_ff={w.d_ff}")
    L = MoeLayer(0, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, w.ffn)
    L.set_experts(dev["routed"], dev["shared"])
    L.expert_count.fill_(7)
    L.expert_offset.fill_(7)
    u = torch.empty((0, w.d), dtype=torch.bfloat16, device="cuda")
    bias = to_dev(I.make_b(w).copy())
    b0 = bias.clone()
    L.step(u, dev["e"], bias, w.gamma)
    torch.cuda.synchronize()
    assert not torch.any(L.expert_count != 0) and not torch.any(L.expert_offset != 0)
    assert torch.equal(bias, b0)
    L.alloc_backward()
    for t in (*L.dw_routed, *L.dw_shared, L.dcentroids):
        t.fill_(3.0)
    L.backward(u, dev["e"], torch.empty((0, w.d), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    for t in (*L.dw_routed, *L.dw_shared, L.dcentroids):
        assert not torch.any(t.float() != 0)
