"""GPU parity of every C ABI call against the CPU oracle (needs an MI355X).

Per-call tests feed each call the oracle's upstream results (uploaded), so a
mismatch names the call; the end-to-end tests run the five calls back to back as
the benchmark does. Small workloads are checked on every output; the V3-shaped
ones on all routing/dispatch results and on sampled output rows (including each
expert group's ragged tail), with the oracle computing those rows one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_26_amd import inputs as I
from mixture_experts_layer_26_amd.layer import MoeLayer
from tests.gpu_util import (FROB_TOL, MAXABS_TOL, ROW_TOL, check_routing, host_expert, log, rel_errors,
                            row_errors, sample_tokens, to_dev, to_np, workload_on_device)

pytestmark = pytest.mark.gpu

BF16_CONFIGS = ["mid_bf16", "v3_prefill_bf16", "v3_decode_skewed", "v3_ep8_share_bf16"]
ALL_CONFIGS = ["tiny_f32"] + BF16_CONFIGS


def _layer(w):
    return MoeLayer(w.T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, w.ffn)


def _host_inputs(w):
    return I.make_u(w), I.make_e(w), I.make_b(w)


# ------------------------------------------------------------------------ route

@pytest.mark.parametrize("name", ALL_CONFIGS)
def test_route_parity(name):
    w, dev = workload_on_device(name)
    L = _layer(w)
    L.route(dev["u"], dev["e"], dev["b"])
    torch.cuda.synchronize()
    u, e, b = _host_inputs(w)
    idx, gate, gap, v = oracle.route(u, e, b, w.top_k, w.act, want_v=True)
    diff, n_exempt = check_routing(to_np(L.topk_idx), to_np(L.topk_gate), idx, gate, gap, v, w.top_k)
    log(f"[route] {name}: exempt tokens {n_exempt}, differing (all exempt) {len(diff)}")


# --------------------------------------------------------------------- dispatch

def _random_topk(rng, T, n_r, K, p=None):
    idx = np.empty((T, K), np.int32)
    for t in range(T):
        idx[t] = np.sort(rng.choice(n_r, K, replace=False, p=p))
    return idx


def _dispatch_cases():
    rng = np.random.default_rng(7)
    return {
        "single_token": (_random_topk(rng, 1, 256, 8), 256),
        "ragged_1000": (_random_topk(rng, 1000, 64, 6), 64),
        "all_on_few": (np.tile(np.arange(8, dtype=np.int32), (5000, 1)), 256),
        "many_chunks_70000": (_random_topk(rng, 70000, 16, 2), 16),
        "k_equals_n": (np.tile(np.arange(16, dtype=np.int32), (300, 1)), 16),
        "skewed": (_random_topk(rng, 4096, 256, 8, p=np.r_[np.full(8, 0.05), np.full(248, 0.6 / 248)]), 256),
    }


def _gpu_dispatch(idx, n_r):
    T, K = idx.shape
    L = MoeLayer(T, 256, n_r, K, 0, 128, "bf16", "bf16")
    L.topk_idx.copy_(to_dev(idx))
    L.dispatch()
    torch.cuda.synchronize()
    return L, [to_np(t) for t in (L.expert_count, L.expert_offset, L.sorted_token, L.pair_row)]


@pytest.mark.parametrize("case", list(_dispatch_cases().keys()))
def test_dispatch_parity_edge_cases(case):
    idx, n_r = _dispatch_cases()[case]
    _, got = _gpu_dispatch(idx, n_r)
    want = oracle.dispatch(idx, n_r)
    for g, r, what in zip(got, want, ("count", "offset", "sorted_token", "pair_row")):
        assert np.array_equal(g.reshape(r.shape), r), f"{case}: {what}"


@pytest.mark.parametrize("name", ALL_CONFIGS)
def test_dispatch_and_bias_parity(name):
    """Dispatch of the oracle's routing, and the bias update from those counts."""
    w = I.WORKLOADS[name]
    u, e, b = _host_inputs(w)
    idx, _, _, _ = oracle.route(u, e, b, w.top_k, w.act)
    L, got = _gpu_dispatch(idx, w.n_routed)
    want = oracle.dispatch(idx, w.n_routed)
    for g, r, what in zip(got, want, ("count", "offset", "sorted_token", "pair_row")):
        assert np.array_equal(g.reshape(r.shape), r), what
    bias = to_dev(b)
    shape_layer = _layer(w)
    shape_layer.expert_count.copy_(L.expert_count)
    shape_layer.bias_update(bias, w.gamma)
    torch.cuda.synchronize()
    want_b = oracle.bias_update(want[0], w.T, w.top_k, w.gamma, b)
    assert np.array_equal(to_np(bias), want_b)
    mean = w.T * w.top_k / w.n_routed
    log(f"[dispatch] {name}: load min {want[0].min()} max {want[0].max()} mean {mean:g}; "
        f"at mean {int(np.sum(want[0] == mean))}")


# --------------------------------------------------------------------- combine

@pytest.mark.parametrize("name", ALL_CONFIGS)
def test_combine_parity(name):
    w = I.WORKLOADS[name]
    u, e, b = _host_inputs(w)
    idx, gate, _, _ = oracle.route(u, e, b, w.top_k, w.act)
    _, _, _, pair_row = oracle.dispatch(idx, w.n_routed)
    rng_y = I.normal(w.seed + 77, 1, 0, w.pairs * w.d, 0.5, w.act).reshape(w.pairs, w.d)
    ysh = I.normal(w.seed + 77, 2, 0, w.T * w.d, 0.7, "f32").reshape(w.T, w.d) if w.n_shared else None
    g32 = gate.astype(np.float32)
    L = _layer(w)
    bf = w.act == "bf16"
    L.y_routed.copy_(to_dev(rng_y, bf16=bf))
    if ysh is not None:
        L.y_shared.copy_(to_dev(ysh))
    L.pair_row.copy_(to_dev(pair_row))
    L.topk_gate.copy_(to_dev(g32))
    ud = to_dev(u, bf16=bf)
    L.combine(ud)
    torch.cuda.synchronize()
    out = to_np(L.out)
    out = I.bf16_bits_to_f32(out) if bf else out
    ref = oracle.combine(u, ysh, rng_y, pair_row, g32, w.act)
    frob, mx = rel_errors(out, ref)
    assert frob <= FROB_TOL and mx <= MAXABS_TOL
    # one rounding to the output type, plus fp32 sums
    ulp_rel = 2.0 ** -8 if bf else 2.0 ** -20
    assert np.all(np.abs(out - ref) <= ulp_rel * np.abs(ref) + 1e-5 * np.max(np.abs(ref)))
    log(f"[combine] {name}: frob {frob:.2e} maxabs {mx:.2e}")


# ------------------------------------------------------------------ grouped FFN

def _ffn_sample(w, count, offset, rng):
    """Sorted rows to check: every row for small workloads; else the first and last rows
    (the ragged tail tile) of a few experts, including the busiest and the least busy."""
    if w.pairs * w.d * w.d_ff <= 2 * 10 ** 9:
        return np.arange(w.pairs)
    act = np.nonzero(count > 0)[0]
    pick = {int(act[0]), int(act[-1]), int(np.argmax(count)), int(act[np.argmin(count[act])])}
    pick |= set(rng.choice(act, 3, replace=False).tolist())
    rows = []
    for i in sorted(pick):
        r = np.arange(offset[i], offset[i + 1])
        rows.append(r if r.size <= 12 else np.r_[r[:6], r[-6:]])
    return np.concatenate(rows)


@pytest.mark.parametrize("name", ALL_CONFIGS)
def test_grouped_ffn_parity(name):
    w, dev = workload_on_device(name)
    u, e, b = _host_inputs(w)
    idx, _, _, _ = oracle.route(u, e, b, w.top_k, w.act)
    count, offset, sorted_token, pair_row = oracle.dispatch(idx, w.n_routed)
    L = _layer(w)
    L.expert_offset.copy_(to_dev(offset))
    L.sorted_token.copy_(to_dev(sorted_token))
    L.set_experts(dev["routed"], dev["shared"])
    L.grouped_ffn(dev["u"])
    torch.cuda.synchronize()
    bf = w.act == "bf16"
    rows = _ffn_sample(w, count, offset, np.random.default_rng(3))
    y_gpu = to_np(L.y_routed[torch.from_numpy(rows).cuda()])
    y_gpu = I.bf16_bits_to_f32(y_gpu) if bf else y_gpu
    expert_of_row = np.searchsorted(offset, rows, side="right") - 1
    ref = np.empty((rows.size, w.d))
    for i in np.unique(expert_of_row):
        sel = expert_of_row == i
        w1, w3, w2 = host_expert(w, False, int(i))
        _, ref[sel] = oracle.expert_rows(u[sorted_token[rows[sel]]], w1, w3, w2, w.ffn)
    frob, mx = rel_errors(y_gpu, ref)
    err = row_errors(y_gpu, ref)
    log(f"[ffn] {name}: routed rows {rows.size} frob {frob:.2e} maxabs {mx:.2e}; worst row {err.max():.2e}")
    assert frob <= FROB_TOL and mx <= MAXABS_TOL
    assert err.max() <= ROW_TOL, f"routed sorted row {rows[np.argmax(err)]}: {err.max():.2e}"
    # shared experts: sum over N_s of FFN_j(u_t) on sampled tokens
    tok = sample_tokens(w.T, 16)
    ysh = to_np(L.y_shared[torch.from_numpy(tok).cuda()])
    ref_s = np.zeros((tok.size, w.d))
    for j in range(w.n_shared):
        w1, w3, w2 = host_expert(w, True, j)
        ref_s += oracle.expert_rows(u[tok], w1, w3, w2, w.ffn)[1]
    frob, mx = rel_errors(ysh, ref_s)
    err = row_errors(ysh, ref_s)
    log(f"[ffn] {name}: shared tokens {tok.size} frob {frob:.2e} maxabs {mx:.2e}; worst row {err.max():.2e}")
    assert frob <= FROB_TOL and mx <= MAXABS_TOL
    assert err.max() <= ROW_TOL, f"shared row of token {tok[np.argmax(err)]}: {err.max():.2e}"


# ------------------------------------------------------------------ end to end

def _oracle_layer_for(w, u_rows, e, b):
    idx, _, _, _ = oracle.route(u_rows, e, b, w.top_k, w.act)
    need = sorted(set(idx.ravel().tolist()))
    routed = {i: host_expert(w, False, i) for i in need}
    shared = [host_expert(w, True, j) for j in range(w.n_shared)]
    return oracle.layer(u_rows, e, b, routed, shared, top_k=w.top_k, d_ff=w.d_ff, act=w.act, ffn=w.ffn,
                        want_components=True)


SAMPLES = {"tiny_f32": 64, "mid_bf16": 96, "v3_prefill_bf16": 64, "v3_decode_skewed": 64, "v3_ep8_share_bf16": 64}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ALL_CONFIGS)
def test_layer_end_to_end(name):
    w, dev = workload_on_device(name)
    L = _layer(w)
    L.set_experts(dev["routed"], dev["shared"])
    bias = dev["b"].clone()
    L.step(dev["u"], dev["e"], bias, w.gamma)
    torch.cuda.synchronize()
    u, e, b = _host_inputs(w)
    idx, gate, gap, v = oracle.route(u, e, b, w.top_k, w.act, want_v=True)
    idx_g = to_np(L.topk_idx)
    diff, n_exempt = check_routing(idx_g, to_np(L.topk_gate), idx, gate, gap, v, w.top_k)
    got = [to_np(t) for t in (L.expert_count, L.expert_offset, L.sorted_token, L.pair_row)]
    if len(diff) == 0:
        want = oracle.dispatch(idx, w.n_routed)
        for g, r, what in zip(got, want, ("count", "offset", "sorted_token", "pair_row")):
            assert np.array_equal(g.reshape(r.shape), r), what
        assert np.array_equal(to_np(bias), oracle.bias_update(want[0], w.T, w.top_k, w.gamma, b))
    else:
        # the GPU's own (valid) routing: dispatch must be the stable sort of it
        want = oracle.dispatch(idx_g, w.n_routed)
        for g, r in zip(got, want):
            assert np.array_equal(g.reshape(r.shape), r)
        assert np.array_equal(to_np(bias), oracle.bias_update(want[0], w.T, w.top_k, w.gamma, b))
    tok = sample_tokens(w.T, SAMPLES[name])
    tok = np.setdiff1d(tok, diff)
    res = _oracle_layer_for(w, u[tok], e, b)
    out = to_np(L.out[torch.from_numpy(tok).cuda()])
    out = I.bf16_bits_to_f32(out) if w.act == "bf16" else out
    frob, mx = rel_errors(out, res["out"])
    err = row_errors(out, res["out"])
    log(f"[e2e] {name}: tokens {tok.size} exempt {n_exempt} differing {len(diff)} "
        f"frob {frob:.2e} maxabs {mx:.2e}; worst token {err.max():.2e}")
    assert frob <= FROB_TOL and mx <= MAXABS_TOL
    assert err.max() <= ROW_TOL, f"token {tok[np.argmax(err)]}: {err.max():.2e}"
    # the routed and shared parts on their own: the residual dominates the output's norm
    ysh = to_np(L.y_shared[torch.from_numpy(tok).cuda()]) if w.n_shared else None
    if w.n_shared:
        f2, m2 = rel_errors(ysh, res["shared_sum"])
        e2 = row_errors(ysh, res["shared_sum"])
        assert f2 <= FROB_TOL and m2 <= MAXABS_TOL and e2.max() <= ROW_TOL
    routed = out.astype(np.float64) - I.bf16_bits_to_f32(to_np(dev["u"][torch.from_numpy(tok).cuda()])) \
        if w.act == "bf16" else out.astype(np.float64) - to_np(dev["u"][torch.from_numpy(tok).cuda()])
    if w.n_shared:
        routed -= ysh
    # out - u - y_shared recovers the gate-weighted routed sum up to the one rounding of out
    # to the act dtype (at most half an ulp per element: 2^-9 of |out| in bf16, 2^-24 in fp32)
    rnd = 2.0 ** -9 if w.act == "bf16" else 2.0 ** -24
    dr = np.linalg.norm(routed - res["routed_sum"], axis=1)
    bound = ROW_TOL * np.linalg.norm(res["routed_sum"], axis=1) + rnd * np.linalg.norm(res["out"], axis=1)
    log(f"[e2e] {name}: routed part of the output, worst token at {(dr / bound).max():.2f} of its bound")
    assert np.all(dr <= bound), f"routed part of token {tok[np.argmax(dr / bound)]}"


@pytest.mark.parametrize("name", ["mid_bf16", "v3_decode_skewed"])
def test_step_is_deterministic(name):
    w, dev = workload_on_device(name)
    L = _layer(w)
    L.set_experts(dev["routed"], dev["shared"])
    outs = []
    for _ in range(2):
        bias = dev["b"].clone()
        L.step(dev["u"], dev["e"], bias, w.gamma)
        torch.cuda.synchronize()
        outs.append([to_np(t).copy() for t in (L.out, L.topk_idx, L.topk_gate, L.expert_count,
                                               L.sorted_token, L.pair_row, L.y_routed, bias)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
