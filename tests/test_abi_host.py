"""C ABI checks that need no GPU: the library loads, exports every entry point the
header declares, sizes workspaces, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_26_amd import abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|size_t|const char\*|int32_t)\s+(moe_\w+)\s*\(",
                                 text, re.M)))


def test_exports_every_declared_symbol():
    lib = abi.load()
    names = _declared()
    assert {"moe_route", "moe_dispatch", "moe_grouped_ffn", "moe_combine", "moe_bias_update"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.moe_abi_version() == abi.ABI_VERSION == 5
    assert lib.moe_status_string(0) == b"ok"


def _shape(**kw):
    base = dict(T=64, d=256, n_routed=16, top_k=2, n_shared=1, d_ff=128, act="f32", ffn="f32")
    base.update(kw)
    return abi.make_shape(**base)


FAKE = 0x1000  # never dereferenced: every call below is rejected on the host


@pytest.mark.parametrize("kw", [dict(T=-1), dict(top_k=0), dict(top_k=17, n_routed=32), dict(top_k=20),
                                dict(n_routed=0), dict(n_routed=257), dict(d=100), dict(d_ff=100),
                                dict(n_shared=9), dict(act="f32", ffn="bf16"), dict(act="bf16", ffn="f32"),
                                dict(act="f32", ffn="fp8")])
def test_bad_shapes_rejected(kw):
    s = _shape(**kw)
    lib = abi.load()
    st = lib.moe_route(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == abi.MOE_ERR_INVALID_ARG
    assert abi.moe_workspace_bytes(s, abi.MOE_CALL_DISPATCH) == 0


def test_null_pointers_rejected():
    s = _shape()
    lib = abi.load()
    assert lib.moe_route(ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == \
        abi.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == \
        abi.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == \
        abi.MOE_ERR_INVALID_ARG  # n_shared = 1 needs y_shared
    u = FAKE
    assert lib.moe_combine(ctypes.byref(s), u, FAKE, FAKE, FAKE, FAKE, u, None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_bias_update(ctypes.byref(s), None, ctypes.c_float(0.001), FAKE, None) == \
        abi.MOE_ERR_INVALID_ARG
    assert lib.moe_bias_update(ctypes.byref(s), FAKE, ctypes.c_float(-1.0), FAKE, None) == \
        abi.MOE_ERR_INVALID_ARG


def test_empty_batch_host_calls():
    """T = 0: the arrays that scale with T may be NULL; the calls that own no T-free output
    return MOE_OK without touching the device (the ones that zero outputs are GPU tests)."""
    lib = abi.load()
    s = _shape(T=0)
    assert lib.moe_route(ctypes.byref(s), None, FAKE, FAKE, None, None, None, 0, None) == abi.MOE_OK
    assert lib.moe_route(ctypes.byref(s), None, None, FAKE, None, None, None, 0, None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(s), None, None, None, None, None, None, None) == abi.MOE_OK
    ex = abi.moe_expert_set()
    ex.w1 = ex.w3 = ex.w2 = FAKE
    ex.layout = abi.MOE_LAYOUT_ROWS
    assert lib.moe_grouped_ffn(ctypes.byref(s), None, FAKE, None, ctypes.byref(ex), ctypes.byref(ex), None, None,
                               None, 0, None) == abi.MOE_OK
    assert lib.moe_grouped_ffn(ctypes.byref(s), None, None, None, ctypes.byref(ex), ctypes.byref(ex), None, None,
                               None, 0, None) == abi.MOE_ERR_INVALID_ARG  # expert_offset does not scale with T
    sb = _shape(T=0, act="bf16", ffn="bf16")
    assert lib.moe_combine_backward(ctypes.byref(sb), None, None, None, None, None, None, None) == abi.MOE_OK


def test_workspace_checks():
    s = _shape()
    lib = abi.load()
    need = abi.moe_workspace_bytes(s, abi.MOE_CALL_DISPATCH)
    assert need >= 16 * 4
    assert lib.moe_dispatch(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == \
        abi.MOE_ERR_WORKSPACE
    assert lib.moe_dispatch(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None) == \
        abi.MOE_ERR_WORKSPACE
    es = abi.make_expert_set(FAKE, FAKE, FAKE)
    ffn_need = abi.moe_workspace_bytes(s, abi.MOE_CALL_GROUPED_FFN)
    # H routed + H shared in fp32
    assert ffn_need >= (64 * 2 + 64) * 128 * 4
    assert lib.moe_grouped_ffn(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(es), ctypes.byref(es), FAKE,
                               FAKE, FAKE, ffn_need - 1, None) == abi.MOE_ERR_WORKSPACE
    # FP8 needs the block scales
    s8 = _shape(d=256, d_ff=128, act="bf16", ffn="fp8")
    assert lib.moe_grouped_ffn(ctypes.byref(s8), FAKE, FAKE, FAKE, ctypes.byref(es), ctypes.byref(es), FAKE,
                               FAKE, FAKE, 1 << 30, None) == abi.MOE_ERR_INVALID_ARG
    # bf16 MFMA tiles need d % 256 == 0 and d_ff % 128 == 0
    sb = _shape(d=320, d_ff=128, act="bf16", ffn="bf16")
    assert lib.moe_grouped_ffn(ctypes.byref(sb), FAKE, FAKE, FAKE, ctypes.byref(es), ctypes.byref(es), FAKE,
                               FAKE, FAKE, 1 << 30, None) == abi.MOE_ERR_UNSUPPORTED


def test_route_workspace():
    lib = abi.load()
    s32 = _shape()  # fp32 activations need no workspace
    assert abi.moe_workspace_bytes(s32, abi.MOE_CALL_ROUTE) == 0
    sb = _shape(T=8192, d=7168, n_routed=256, top_k=8, d_ff=2048, act="bf16", ffn="bf16")
    need = abi.moe_workspace_bytes(sb, abi.MOE_CALL_ROUTE)
    # partial logits of the K chunks: [chunks][T][N_r] fp32, 1 <= chunks <= 32
    assert 8192 * 256 * 4 <= need <= 32 * 8192 * 256 * 4 + 4096
    assert lib.moe_route(ctypes.byref(sb), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == \
        abi.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(sb), FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None) == \
        abi.MOE_ERR_WORKSPACE


def test_route_score_modes():
    """score is SIGMOID or SOFTMAX; only SOFTMAX may go without a bias. Every call here is
    stopped on the host (the workspace is one byte short)."""
    lib = abi.load()
    assert ctypes.sizeof(abi.moe_shape) == 40
    bad = _shape()
    bad.score = 2
    assert lib.moe_route(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == \
        abi.MOE_ERR_INVALID_ARG
    assert abi.moe_workspace_bytes(bad, abi.MOE_CALL_ROUTE) == 0
    sig = _shape(T=256, d=256, act="bf16", ffn="bf16")
    soft = _shape(T=256, d=256, act="bf16", ffn="bf16", score="softmax")
    need = abi.moe_workspace_bytes(soft, abi.MOE_CALL_ROUTE)
    assert need == abi.moe_workspace_bytes(sig, abi.MOE_CALL_ROUTE) > 0
    assert lib.moe_route(ctypes.byref(sig), FAKE, FAKE, None, FAKE, FAKE, FAKE, need, None) == \
        abi.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(soft), FAKE, FAKE, None, FAKE, FAKE, FAKE, need - 1, None) == \
        abi.MOE_ERR_WORKSPACE


def test_quantize_args_rejected():
    lib = abi.load()
    q = lib.moe_quantize_fp8
    assert q(FAKE, abi.MOE_F32, 128, 100, 1, 128, FAKE, FAKE, None) == abi.MOE_ERR_INVALID_ARG
    assert q(FAKE, abi.MOE_F32, 100, 128, 128, 128, FAKE, FAKE, None) == abi.MOE_ERR_INVALID_ARG
    assert q(FAKE, abi.MOE_F32, 128, 128, 64, 64, FAKE, FAKE, None) == abi.MOE_ERR_UNSUPPORTED
    assert q(FAKE, 7, 128, 128, 1, 128, FAKE, FAKE, None) == abi.MOE_ERR_INVALID_ARG
    assert q(None, abi.MOE_F32, 128, 128, 1, 128, FAKE, FAKE, None) == abi.MOE_ERR_INVALID_ARG


def test_weight_layout_checks():
    lib = abi.load()
    sb = _shape(d=256, d_ff=128, act="bf16", ffn="bf16")
    rows = abi.make_expert_set(FAKE, FAKE, FAKE)
    tiled = abi.make_expert_set(FAKE, FAKE, FAKE, layout=abi.MOE_LAYOUT_TILED)
    bad = abi.make_expert_set(FAKE, FAKE, FAKE, layout=7)
    ffn = lambda s, r, sh: lib.moe_grouped_ffn(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(r), ctypes.byref(sh),
                                               FAKE, FAKE, FAKE, 1 << 30, None)
    assert ffn(sb, bad, bad) == abi.MOE_ERR_INVALID_ARG
    assert ffn(sb, tiled, rows) == abi.MOE_ERR_INVALID_ARG  # routed and shared must agree
    s32 = _shape()  # fp32 expert GEMMs read only the row-major layout
    assert ffn(s32, tiled, tiled) == abi.MOE_ERR_UNSUPPORTED


def test_pack_weights_args_rejected():
    lib = abi.load()
    p = lambda s, m, e, a, b: lib.moe_pack_weights(ctypes.byref(s), m, e, a, b, None)
    sb = _shape(d=256, d_ff=128, act="bf16", ffn="bf16")
    other = FAKE + (1 << 30)
    assert p(sb, 3, 1, FAKE, other) == abi.MOE_ERR_INVALID_ARG            # no such matrix
    assert p(sb, abi.MOE_W1, 0, FAKE, other) == abi.MOE_ERR_INVALID_ARG   # no experts
    assert p(sb, abi.MOE_W1, 1, None, other) == abi.MOE_ERR_INVALID_ARG
    assert p(sb, abi.MOE_W2, 2, FAKE, FAKE + 1024) == abi.MOE_ERR_INVALID_ARG  # overlapping
    assert p(_shape(), abi.MOE_W1, 1, FAKE, other) == abi.MOE_ERR_UNSUPPORTED  # fp32 is never tiled
    assert p(_shape(d=320, d_ff=128, act="bf16", ffn="bf16"), abi.MOE_W1, 1, FAKE, other) == \
        abi.MOE_ERR_UNSUPPORTED


def test_backward_args_rejected():
    """The backward runs bf16 layers with either weight layout (the same for both expert kinds),
    d % 256 == 0, d_ff % 128 == 0; every call below is stopped on the host before any HIP call."""
    lib = abi.load()
    fp32 = _shape()
    bf = _shape(act="bf16", ffn="bf16")
    odd = _shape(act="bf16", ffn="bf16", d=384)  # d % 256 != 0
    fp8 = _shape(act="bf16", ffn="fp8")
    for s in (fp32, odd, fp8):
        assert abi.moe_workspace_bytes(s, abi.MOE_CALL_GROUPED_FFN_BACKWARD) == 0
        assert abi.moe_workspace_bytes(s, abi.MOE_CALL_ROUTE_BACKWARD) == 0
        assert lib.moe_combine_backward(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == \
            abi.MOE_ERR_UNSUPPORTED
    need = abi.moe_workspace_bytes(bf, abi.MOE_CALL_GROUPED_FFN_BACKWARD)
    # h, da, dv for the routed rows and the shared experts' rows, bf16
    assert need >= 3 * 2 * (64 * 2 + 64 * 1) * 128
    assert abi.moe_workspace_bytes(bf, abi.MOE_CALL_ROUTE_BACKWARD) >= 64 * 2 * 4
    es = abi.make_expert_set(FAKE, FAKE, FAKE)
    tiled = abi.make_expert_set(FAKE, FAKE, FAKE, layout=abi.MOE_LAYOUT_TILED)
    bad = abi.make_expert_set(FAKE, FAKE, FAKE, layout=7)
    gr = abi.make_expert_grads(FAKE, FAKE, FAKE)
    nullg = abi.make_expert_grads(FAKE, None, FAKE)
    call = lambda s, r, sh, g, gs, dxs, ws, n: lib.moe_grouped_ffn_backward(
        ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, ctypes.byref(r), None if sh is None else ctypes.byref(sh),
        FAKE, FAKE, dxs, ctypes.byref(g), None if gs is None else ctypes.byref(gs), ws, n, None)
    assert call(bf, es, es, gr, gr, FAKE, FAKE, need - 1) == abi.MOE_ERR_WORKSPACE
    assert call(bf, es, es, gr, gr, FAKE, None, need) == abi.MOE_ERR_WORKSPACE
    assert call(bf, tiled, es, gr, gr, FAKE, FAKE, need) == abi.MOE_ERR_INVALID_ARG  # mixed layouts
    assert call(bf, bad, bad, gr, gr, FAKE, FAKE, need) == abi.MOE_ERR_INVALID_ARG
    assert call(bf, es, es, nullg, gr, FAKE, FAKE, need) == abi.MOE_ERR_INVALID_ARG
    assert call(bf, es, None, gr, gr, FAKE, FAKE, need) == abi.MOE_ERR_INVALID_ARG   # n_shared = 1
    assert call(bf, es, es, gr, None, FAKE, FAKE, need) == abi.MOE_ERR_INVALID_ARG
    assert call(bf, es, es, gr, gr, None, FAKE, need) == abi.MOE_ERR_INVALID_ARG     # dx_shared
    rneed = abi.moe_workspace_bytes(bf, abi.MOE_CALL_ROUTE_BACKWARD)
    args = [FAKE] * 14
    assert lib.moe_route_backward(ctypes.byref(bf), *args, FAKE, rneed - 1, None) == abi.MOE_ERR_WORKSPACE
    args[10] = None  # dx_shared with a shared expert
    assert lib.moe_route_backward(ctypes.byref(bf), *args, FAKE, rneed, None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_backward(ctypes.byref(bf), FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == \
        abi.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,fits", [
    (dict(T=299_594, d=7168, d_ff=256), dict(T=299_593)),                 # u: T*d < 2^31
    (dict(T=4, d=1 << 22, d_ff=128), dict(d=(1 << 22) - 256)),             # row length d
    (dict(T=4, d=256, d_ff=1 << 22), dict(d_ff=(1 << 22) - 128)),          # row length d_ff
    (dict(T=4, n_shared=2, d=256, d_ff=1 << 21), dict(n_shared=1)),       # shared H row N_s*d_ff
    (dict(T=599_187, d=7168, d_ff=256, ffn="fp8"), dict(T=599_186))])      # FP8 codes of u: T*d < 2^32
def test_bf16_ffn_rejects_operands_past_32_bit_offsets(kw, fits):
    """The bf16 grouped GEMMs address loaded rows with a wave-uniform base and a 32-bit byte
    offset: the gathered rows of u are offsets from u itself (u must have fewer than 2^31
    elements), every other offset stays within one tile's rows (row lengths below 2^22
    elements). Larger shapes are refused on the host, before any launch; the same shape just
    inside the limit passes the check (and stops at the workspace check)."""
    base = dict(n_routed=16, top_k=2, n_shared=1, act="bf16", ffn="bf16")
    base.update(kw)
    lib = abi.load()
    es = abi.make_expert_set(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)  # scales are read for FP8 only
    s = _shape(**base)
    assert lib.moe_grouped_ffn(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(es), ctypes.byref(es), FAKE, FAKE,
                               FAKE, 1 << 62, None) == abi.MOE_ERR_UNSUPPORTED
    ok = _shape(**dict(base, **fits))
    assert lib.moe_grouped_ffn(ctypes.byref(ok), FAKE, FAKE, FAKE, ctypes.byref(es), ctypes.byref(es), FAKE, FAKE,
                               FAKE, 0, None) == abi.MOE_ERR_WORKSPACE


def test_noalloc_ffn_checks_on_the_host():
    """moe_grouped_ffn_noalloc takes moe_grouped_ffn's arguments without a workspace: the same
    argument checks, an empty batch does nothing, and a shape whose workspace exceeds the fixed
    scratch is refused with MOE_ERR_SCRATCH_LIMIT before any HIP call."""
    lib = abi.load()
    es = abi.make_expert_set(FAKE, FAKE, FAKE, layout=abi.MOE_LAYOUT_TILED)
    call = lambda s: lib.moe_grouped_ffn_noalloc(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(es),
                                                 ctypes.byref(es), FAKE, FAKE, None)
    v3 = dict(d=7168, n_routed=256, top_k=8, n_shared=1, d_ff=2048, act="bf16", ffn="bf16")
    big = _shape(T=8192, **v3)
    assert abi.moe_workspace_bytes(big, abi.MOE_CALL_GROUPED_FFN) > abi.MOE_NOALLOC_SCRATCH_BYTES
    assert call(big) == abi.MOE_ERR_SCRATCH_LIMIT
    assert b"scratch" in lib.moe_status_string(abi.MOE_ERR_SCRATCH_LIMIT)
    # the largest V3 batch that fits, and the next one
    fit = max(T for T in range(1, 4096) if abi.moe_workspace_bytes(_shape(T=T, **v3), abi.MOE_CALL_GROUPED_FFN)
              <= abi.MOE_NOALLOC_SCRATCH_BYTES)
    assert 1700 <= fit < 1900
    assert call(_shape(T=fit + 1, **v3)) == abi.MOE_ERR_SCRATCH_LIMIT
    assert call(_shape(T=0, **v3)) == abi.MOE_OK
    assert call(_shape(T=16, d=100, **{k: v for k, v in v3.items() if k != "d"})) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_grouped_ffn_noalloc(ctypes.byref(_shape(T=16, **v3)), FAKE, FAKE, FAKE, None, None, FAKE,
                                       FAKE, None) == abi.MOE_ERR_INVALID_ARG
    fp8 = dict(v3, ffn="fp8")  # FP8 needs its block scales
    assert call(_shape(T=16, **fp8)) == abi.MOE_ERR_INVALID_ARG
