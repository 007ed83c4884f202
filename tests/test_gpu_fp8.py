"""GPU parity of the FP8 E4M3 path against the CPU oracle (needs an MI355X).

Quantisation of inputs (weights in 128x128 blocks, activations in 1x128 tiles) is
deterministic, so the GPU's codes and scales must equal the oracle's bit for bit.
The FP8 layer output is compared with the oracle applying the identical
quantisation, within the layer tolerance. On the sampled rows the GPU's H codes and scales
are also checked against the oracle's H, and the fp32 shared rows against the exact product
of the GPU's own shared H (the checks and their bounds are those of test_gpu_tile_edges.py).
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_26_amd import abi
from mixture_experts_layer_26_amd import inputs as I
from mixture_experts_layer_26_amd.layer import MoeLayer, quantize_experts
from tests.gpu_util import (FROB_TOL, MAXABS_TOL, ROW_TOL, check_routing, host_expert, log, rel_errors,
                            row_errors, sample_tokens, to_dev, to_np, workload_on_device)
from tests.test_gpu_tile_edges import (SHARED_FP8_TOL, _check_h_codes, _check_layout_reading, _down, _fp8_h,
                                      _row_errors)

pytestmark = pytest.mark.gpu


def _gpu_quantize(x: np.ndarray, xt: str, tr: int, tc: int):
    rows, cols = x.shape
    xd = to_dev(x, bf16=(xt == "bf16"))
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows // tr, cols // tc), dtype=torch.float32, device="cuda")
    abi.moe_quantize_fp8(xd, abi.MOE_BF16 if xt == "bf16" else abi.MOE_F32, rows, cols, tr, tc, q, s)
    torch.cuda.synchronize()
    return to_np(q), to_np(s)


@pytest.mark.parametrize("tiles", [(128, 128), (1, 128)])
@pytest.mark.parametrize("xt", ["bf16", "f32"])
def test_quantize_parity(tiles, xt):
    tr, tc = tiles
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((384, 640)) * np.exp2(rng.integers(-12, 6, (384, 1)))).astype(np.float32)
    x[0:128, 0:128] = 0.0                                  # an all-zero tile
    x[200, 300] = 3.0e-40                                   # a subnormal input
    x[130:140, 256:384] = np.float32(448.0) * 2.0 ** -20   # flat tile
    if xt == "bf16":
        x = oracle.bf16_from_double(x.astype(np.float64))
    q, s = _gpu_quantize(x, xt, tr, tc)
    qr, sr = oracle.quantize(x, xt, tr, tc)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q, qr)


@pytest.mark.slow
def test_e4m3_conversion_exhaustive():
    """Every non-negative float32 up to 448 (and its negative) through the GPU
    quantiser with a unit scale: rows of 127 values plus one 448, so amax / 448 = 1
    and the codes are the plain E4M3 rounding, compared with the oracle's encoder."""
    top = int(np.float32(448.0).view(np.uint32))
    per_row = 127
    chunk_rows = 1 << 19
    start = 0
    checked = 0
    while start <= top:
        n = min(chunk_rows * per_row, top + 1 - start)
        bits = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32)
        rows = (n + per_row - 1) // per_row
        vals = np.zeros(rows * per_row, np.float32)
        vals[:n] = bits.view(np.float32)
        for sign in (1.0, -1.0):
            x = np.empty((rows, 128), np.float32)
            x[:, 0] = 448.0
            x[:, 1:] = sign * vals.reshape(rows, per_row)
            q, s = _gpu_quantize(x, "f32", 1, 128)
            assert np.all(s == 1.0)
            want = oracle.e4m3_from_float(x[:, 1:].ravel()[:n])
            got = q[:, 1:].ravel()[:n]
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (sign, hex(int(bits[bad[0]])), got[bad[0]], want[bad[0]])
        checked += n
        start += n
    log(f"[e4m3] {checked} magnitudes, both signs: GPU conversion equals the oracle")


def _fp8_setup(base: str, T=None):
    """Device FP8 weights made by the library from the bf16 tensors of workload `base`
    (the FP8 workloads share their tensors with a bf16 one)."""
    _, dev = workload_on_device(base, T)
    key = "_fp8_"
    if key not in dev:
        routed = quantize_experts(dev["routed"])
        shared = quantize_experts(dev["shared"]) if dev["shared"] is not None else None
        torch.cuda.synchronize()
        dev[key] = (routed, shared)
    return dev, dev[key]


def _q_host(tup):
    out = [oracle.quantize(a, "bf16", 128, 128) for a in tup]
    return (out[0][0], out[1][0], out[2][0], out[0][1], out[1][1], out[2][1])


_q_cache = {}


def _q_expert(w, shared: bool, i: int):
    """The oracle's 128x128 E4M3 codes and scales of one expert's generated weights (cached)."""
    key = (w.seed, w.d, w.d_ff, shared, int(i))
    if key not in _q_cache:
        if len(_q_cache) >= 320:
            _q_cache.pop(next(iter(_q_cache)))
        _q_cache[key] = _q_host(host_expert(w, shared, int(i)))
    return _q_cache[key]


def test_fp8_weight_codes_match_oracle():
    w = I.WORKLOADS["v3_prefill_fp8"]
    dev, (routed, shared) = _fp8_setup("v3_prefill_bf16")
    for i in (0, 77, 255):
        want = _q_host(I.make_expert(w, False, i))
        for j in range(6):
            assert np.array_equal(to_np(routed[j][i]), want[j]), (i, j)
    want = _q_host(I.make_expert(w, True, 0))
    for j in range(6):
        assert np.array_equal(to_np(shared[j][0]), want[j])


def _layer(w):
    return MoeLayer(w.T, w.d, w.n_routed, w.top_k, w.n_shared, w.d_ff, w.act, w.ffn)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("base,T", [("mid_bf16", 512), ("v3_prefill_bf16", None), ("v3_ep8_share_bf16", None)])
def test_fp8_layer_end_to_end(base, T):
    """The V3 prefill workload in FP8, and the mid shape in FP8 (d = 2048, d_ff = 1408,
    two shared experts, ragged 11-block d_ff), on the tensors of the bf16 workloads. 64
    sampled tokens at V3 (48 at the mid shape), each bounded on its own; their routed rows
    against the oracle's FP8 FFN (pooled) and, row by row, against the exact product of the
    GPU's own H codes (an H code may round to the other side of a midpoint, which moves its
    row by up to a few percent)."""
    wb = I.WORKLOADS[base]
    w = I.Workload(wb.name.replace("bf16", "fp8"), T=wb.T, d=wb.d, n_routed=wb.n_routed, top_k=wb.top_k,
                   n_shared=wb.n_shared, d_ff=wb.d_ff, act="bf16", ffn="fp8", seed=wb.seed,
                   bias_range=wb.bias_range)
    if T is not None:
        w = w.with_tokens(T)
    dev, (routed, shared) = _fp8_setup(base, T)
    L = _layer(w)
    L.set_experts(routed, shared)
    bias = dev["b"].clone()
    L.step(dev["u"], dev["e"], bias, w.gamma)
    torch.cuda.synchronize()
    u = I.make_u(w)
    e, b = I.make_e(w), I.make_b(w)
    idx, gate, gap, v = oracle.route(u, e, b, w.top_k, w.act, want_v=True)
    diff, n_exempt = check_routing(to_np(L.topk_idx), to_np(L.topk_gate), idx, gate, gap, v, w.top_k)
    tok = np.setdiff1d(sample_tokens(w.T, 64 if w.d > 4096 else 48), diff)
    idx_s, _, _, _ = oracle.route(u[tok], e, b, w.top_k, w.act)
    need = sorted(set(idx_s.ravel().tolist()))
    r_host = {i: _q_expert(w, False, i) for i in need}
    s_host = [_q_expert(w, True, j) for j in range(w.n_shared)]
    log(f"[fp8 e2e] {w.name}: oracle weights of {len(need)} experts ready")
    res = oracle.layer(u[tok], e, b, r_host, s_host, top_k=w.top_k, d_ff=w.d_ff, act="bf16", ffn="fp8",
                       want_components=True)
    out = I.bf16_bits_to_f32(to_np(L.out[torch.from_numpy(tok).cuda()]))
    frob, mx = rel_errors(out, res["out"])
    err = row_errors(out, res["out"])
    ysh = to_np(L.y_shared[torch.from_numpy(tok).cuda()])
    f2, m2 = rel_errors(ysh, res["shared_sum"])
    log(f"[fp8 e2e] {w.name}: tokens {tok.size} exempt {n_exempt} out frob {frob:.2e} maxabs {mx:.2e}, "
        f"worst token against the oracle {err.max():.2e}; shared frob {f2:.2e}")
    assert frob <= FROB_TOL and mx <= MAXABS_TOL
    assert f2 <= FROB_TOL and m2 <= MAXABS_TOL
    # routed rows of the sampled tokens, grouped by expert, against the oracle's FP8 FFN
    pr = to_np(L.pair_row)[tok].ravel()
    sel = to_np(L.topk_idx)[tok].ravel()
    src = np.repeat(tok, w.top_k)
    y_gpu = I.bf16_bits_to_f32(to_np(L.y_routed[torch.from_numpy(pr).cuda()]))
    y_ref = np.empty_like(y_gpu, dtype=np.float64)
    h_ref = np.empty((y_gpu.shape[0], w.d_ff))
    for i in np.unique(sel):
        m = sel == i
        h1, y1 = oracle.expert_rows(u[src[m]], *r_host[int(i)][:3], "fp8", *r_host[int(i)][3:])
        h_ref[m], y_ref[m] = h1, y1
    f3, m3 = rel_errors(y_gpu, y_ref)
    log(f"[fp8 ffn] {w.name}: routed rows {y_gpu.shape[0]} frob {f3:.2e} maxabs {m3:.2e}")
    assert f3 <= FROB_TOL and m3 <= MAXABS_TOL
    # H of those rows and of the sampled tokens' shared rows, against the oracle's H
    tab = oracle.e4m3_table()
    h_r, s_r, h_s, s_s, q_u = _fp8_h(L, w)
    tok_dev = torch.from_numpy(tok.astype(np.int64)).cuda()
    _check_layout_reading(to_np(q_u[tok_dev]), u[tok], w.name)
    rows_dev = torch.from_numpy(pr.astype(np.int64)).cuda()
    hr, sr = to_np(h_r[rows_dev]), to_np(s_r[rows_dev])
    _check_h_codes(h_ref, hr, sr, tab, f"{w.name} routed rows")
    # each routed row against the exact product of the GPU's own H codes and scales with W2
    y_routed_adopt = np.empty_like(y_ref)
    for i in np.unique(sel):
        m = sel == i
        y_routed_adopt[m] = _down(hr[m], sr[m], r_host[int(i)], tab)
    er = _row_errors(y_gpu.astype(np.float64), y_routed_adopt)
    log(f"[fp8 ffn] {w.name}: routed rows against the product of the GPU's H: worst {er.max():.2e}")
    assert er.max() <= ROW_TOL, f"routed row {pr[np.argmax(er)]}: {er.max():.2e}"
    hs, ss = to_np(h_s[tok_dev]), to_np(s_s[tok_dev])
    F, nb = w.d_ff, w.d_ff // 128
    y_adopt = np.zeros((tok.size, w.d))
    for j in range(w.n_shared):
        h_o, _ = oracle.expert_rows(u[tok], *s_host[j][:3], "fp8", *s_host[j][3:])
        _check_h_codes(h_o, hs[:, j * F:(j + 1) * F], ss[:, j * nb:(j + 1) * nb], tab, f"{w.name} shared {j}")
        y_adopt += _down(hs[:, j * F:(j + 1) * F], ss[:, j * nb:(j + 1) * nb], s_host[j], tab)
    err = _row_errors(ysh.astype(np.float64), y_adopt)
    log(f"[fp8 ffn] {w.name}: shared rows against the product of the GPU's H: worst {err.max():.2e}")
    assert err.max() <= SHARED_FP8_TOL
    # each sampled token's output against the layer formed from the GPU's own H codes (checked
    # above as correct roundings of the oracle's H): u + shared product + gated routed products.
    # Against the oracle itself one shared H code on the other side of a midpoint can move a
    # token by up to about 8e-3 at this shape, which the pooled check above absorbs.
    g = to_np(L.topk_gate)[tok].astype(np.float64)
    y_tok = np.zeros((tok.size, w.d))
    for j in range(w.top_k):
        y_tok += g[:, j:j + 1] * y_routed_adopt[j::w.top_k]
    out_adopt = I.bf16_bits_to_f32(u[tok]).astype(np.float64) + y_adopt + y_tok
    et = _row_errors(out.astype(np.float64), out_adopt)
    log(f"[fp8 e2e] {w.name}: tokens against the layer of the GPU's own H codes: worst {et.max():.2e}")
    assert et.max() <= ROW_TOL, f"token {tok[np.argmax(et)]}: {et.max():.2e}"
