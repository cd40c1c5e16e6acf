"""The C ABI without a GPU: the library loads, exports every declared entry
point, and refuses bad arguments with its named codes before touching the
device."""
import ctypes
import os
import re

import pytest

import block_fp8_mixture_router_amd as moe
from block_fp8_mixture_router_amd import inputs

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|int|size_t)\s+(moe_\w+)\s*\(", src,
                                 re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(moe.EXPORTS)


def test_library_exports_every_symbol():
    L = moe.lib()
    for name in _declared():
        assert hasattr(L, name), name


def _cfg(**kw):
    c = moe.config(inputs.DECODE)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value", [
    ("hidden", 100), ("hidden", 0), ("hidden", 16384), ("inter", 64), ("inter", 8192),
    ("shared_inter", 100), ("shared_inter", -128), ("n_experts", 0), ("n_experts", 2048),
    ("top_k", 0), ("top_k", 17), ("flags", 1 << 20),
])
def test_workspace_refuses_bad_config(field, value):
    assert moe.workspace_bytes(_cfg(**{field: value}), 1) == 0


def test_workspace_grows_with_rows():
    c = _cfg()
    a, b = moe.workspace_bytes(c, 1), moe.workspace_bytes(c, 1024)
    assert 0 < a < b
    assert b % 256 == 0
    assert moe.workspace_bytes(c, -1) == 0 and moe.workspace_bytes(c, 65537) == 0


def _fwd(cfg, w, x, T, y, ws, nbytes):
    return moe.lib().moe_forward(ctypes.byref(cfg) if cfg is not None else None,
                                 ctypes.byref(w) if w is not None else None, x, T, y, ws,
                                 nbytes, None)


def _fake_weights(base=0x10000000):
    w = moe.Weights()
    for i, (name, _) in enumerate(moe.Weights._fields_):
        setattr(w, name, base + 0x100000 * (i + 1))
    w.router_bias = None
    return w


def test_forward_refusals_before_any_device_call():
    c = _cfg()
    w = _fake_weights()
    n = moe.workspace_bytes(c, 4)
    X, Y, WS = 0x20000000, 0x30000000, 0x40000000
    assert _fwd(None, w, X, 4, Y, WS, n) == -1
    assert _fwd(c, None, X, 4, Y, WS, n) == -1
    assert _fwd(c, w, None, 4, Y, WS, n) == -1
    assert _fwd(c, w, X, 4, Y, None, n) == -1
    assert _fwd(c, w, X, -1, Y, WS, n) == -2
    assert _fwd(c, w, X, 70000, Y, WS, n) == -2
    assert _fwd(c, w, X, 0, Y, WS, n) == 0          # T = 0 is a no-op
    assert _fwd(c, w, X + 2, 4, Y, WS, n) == -3      # misaligned x
    assert _fwd(c, w, X, 4, Y, WS + 16, n) == -3     # workspace not 256-aligned
    assert _fwd(c, w, X, 4, Y, WS, n - 1) == -4
    bad = _cfg(flags=moe.FORCE_GEMV | moe.FORCE_GROUPED)
    assert _fwd(bad, w, X, 4, Y, WS, n) == -5
    w2 = _fake_weights()
    w2.w_down = None
    assert _fwd(c, w2, X, 4, Y, WS, n) == -1
    # all arguments valid: without a gfx950 device the call is refused, not run
    assert _fwd(c, w, X, 4, Y, WS, n) == -5


def test_quant_and_route_refusals():
    L = moe.lib()
    X, Q, S = 0x20000000, 0x30000000, 0x40000000
    assert L.moe_quant_act(X, 4, 100, Q, S, None) == -2
    assert L.moe_quant_act(X, 4, 0, Q, S, None) == -2
    assert L.moe_quant_act(X, -1, 128, Q, S, None) == -2
    assert L.moe_quant_act(X, 0, 128, Q, S, None) == 0
    assert L.moe_quant_act(None, 4, 128, Q, S, None) == -1
    assert L.moe_quant_act(X + 8, 4, 128, Q, S, None) == -3
    assert L.moe_quant_act(X, 4, 128, Q, S, None) == -5
    c = _cfg()
    cb = ctypes.byref(c)
    assert L.moe_route(cb, X, 4, Q, None, S, S + 4096, None, None, 0, None) == -1
    assert L.moe_route(cb, X, 4, Q, None, S, S + 4096, S + 8192, None, 0, None) == -5
    WS = 0x50000000
    assert L.moe_route(cb, X, 4, Q, None, S, S + 4096, None, WS, 16, None) == -4


def test_renorm_refusals():
    L = moe.lib()
    Y, X = 0x20000000, 0x30000000
    assert L.moe_rms_renorm(Y, 4, 100, ctypes.c_float(1e-6), X, None) == -2
    assert L.moe_rms_renorm(Y, 4, 16384, ctypes.c_float(1e-6), X, None) == -2
    assert L.moe_rms_renorm(Y, -1, 2048, ctypes.c_float(1e-6), X, None) == -2
    assert L.moe_rms_renorm(Y, 4, 2048, ctypes.c_float(-1.0), X, None) == -2
    assert L.moe_rms_renorm(Y, 4, 2048, ctypes.c_float(float("nan")), X, None) == -2
    assert L.moe_rms_renorm(Y, 0, 2048, ctypes.c_float(1e-6), X, None) == 0
    assert L.moe_rms_renorm(None, 4, 2048, ctypes.c_float(1e-6), X, None) == -1
    assert L.moe_rms_renorm(Y + 2, 4, 2048, ctypes.c_float(1e-6), X, None) == -3
    assert L.moe_rms_renorm(Y, 4, 2048, ctypes.c_float(1e-6), Y, None) == -5  # no device


def _fake_layers(n):
    return (moe.Weights * n)(*[_fake_weights(0x10000000 + 0x4000000 * l) for l in range(n)])


def test_stack_refusals():
    """moe_forward_stack takes a host array of weight structs and checks every
    layer's pointers on the host before anything is enqueued."""
    L = moe.lib()
    c = _cfg()
    cb = ctypes.byref(c)
    n = moe.workspace_bytes(c, 1)
    TB = _fake_layers(40)
    X, Y, WS = 0x20000000, 0x30000000, 0x40000000
    f = lambda *a: L.moe_forward_stack(*a)  # noqa: E731
    eps = ctypes.c_float(1e-6)
    assert f(cb, TB, 40, X, 1, eps, Y, None, WS, n, None) == -5      # no device
    assert f(cb, TB, 0, X, 1, eps, Y, None, WS, n, None) == 0        # no layers: no-op
    assert f(cb, TB, 40, X, 0, eps, Y, None, WS, n, None) == 0       # no rows: no-op
    assert f(cb, None, 40, X, 1, eps, Y, None, WS, n, None) == -1
    assert f(cb, TB, 40, None, 1, eps, Y, None, WS, n, None) == -1
    assert f(cb, TB, -1, X, 1, eps, Y, None, WS, n, None) == -2
    assert f(cb, TB, 40, X, 1, ctypes.c_float(-1.0), Y, None, WS, n, None) == -2
    assert f(cb, TB, 40, X + 2, 1, eps, Y, None, WS, n, None) == -3
    assert f(cb, TB, 40, X, 1, eps, Y, Y + 8, WS, n, None) == -3
    assert f(cb, TB, 40, X, 1, eps, Y, None, WS, n - 1, None) == -4
    assert f(cb, TB, 40, X, 1, eps, X, None, WS, n, None) == -5      # y aliases x
    forced = _cfg(flags=moe.FORCE_GROUPED)
    assert f(ctypes.byref(forced), TB, 40, X, 1, eps, Y, None, WS, n, None) == -5
    # every layer is checked: a missing or misaligned pointer in layer 17
    bad = _fake_layers(40)
    bad[17].w_up = None
    assert f(cb, bad, 40, X, 1, eps, Y, None, WS, n, None) == -1
    bad = _fake_layers(40)
    bad[39].router_w = bad[39].router_w + 8
    assert f(cb, bad, 40, X, 1, eps, Y, None, WS, n, None) == -3
    # more rows than the one-row path takes
    n5 = moe.workspace_bytes(c, 5)
    assert f(cb, TB, 40, X, 5, eps, Y, None, WS, n5, None) == -5


def test_decode_regions_do_not_move_with_rows():
    """The one-row path's handoff regions are sized by the config alone, so
    for T = 1..4 the workspace needed differs only by the grouped regions,
    which all lie after them."""
    c = _cfg()
    g = _cfg(flags=moe.FORCE_GROUPED)
    for T in range(1, 8):
        assert moe.workspace_bytes(c, T) == moe.workspace_bytes(g, T)


def test_supported_is_false_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert moe.supported(0) is False
    assert moe.supported(-1) is False


def test_workspace_is_monotonic_in_rows():
    """A workspace sized for max_rows must serve every call with fewer rows."""
    for shape in (inputs.TINY, inputs.DECODE):
        c = moe.config(shape)
        sizes = [moe.workspace_bytes(c, T) for T in range(1, 1100)]
        assert all(b >= a for a, b in zip(sizes, sizes[1:]))


def test_add_rmsnorm_quant_refusals():
    L = moe.lib()
    H, R, O, W, X, Q, S = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, \
        0x60000000, 0x70000000
    eps = ctypes.c_float(1e-6)
    f = lambda *a: L.moe_add_rmsnorm_quant(*a)  # noqa: E731
    assert f(H, R, O, W, 4, 2048, eps, X, Q, S, None) == -5            # no device
    assert f(H, R, R, W, 4, 2048, eps, X, Q, S, None) == -5            # in place: no device
    assert f(H, R, O, W, 0, 2048, eps, X, Q, S, None) == 0             # no rows: no-op
    assert f(H, R, O, W, 4, 2000, eps, X, Q, S, None) == -2
    assert f(H, R, O, W, 4, 16384, eps, X, Q, S, None) == -2
    assert f(H, R, O, W, -1, 2048, eps, X, Q, S, None) == -2
    assert f(H, R, O, W, 4, 2048, ctypes.c_float(-1.0), X, Q, S, None) == -2
    assert f(H, R, O, W, 4, 2048, ctypes.c_float(float("nan")), X, Q, S, None) == -2
    assert f(None, R, O, W, 4, 2048, eps, X, Q, S, None) == -1
    assert f(H, R, O, None, 4, 2048, eps, X, Q, S, None) == -1
    assert f(H, R, O, W, 4, 2048, eps, X, Q, None, None) == -1
    assert f(H + 2, R, O, W, 4, 2048, eps, X, Q, S, None) == -3
    assert f(H, R, O, W, 4, 2048, eps, X, Q + 8, S, None) == -3
    assert f(H, R, O, W, 4, 2048, eps, X, Q, S + 2, None) == -3
    assert f(H, R, O, W, 4, 2048, eps, R, Q, S, None) == -5            # x aliases the residual
    assert f(H, R, H, W, 4, 2048, eps, X, Q, S, None) == -5            # residual_out aliases hidden


def test_no_act_quant_flag():
    """The control flag is known, adds exactly one bf16 [T*K, I] region to the
    workspace, and is refused with the decode path forced or in a stack."""
    c, n = _cfg(), _cfg(flags=moe.NO_ACT_QUANT)
    s = inputs.DECODE

    def extra(T):
        return (T * s.top_k * s.inter * 2 + 255) // 256 * 256

    # growth with rows is the plain layout's plus the bf16 h region; the
    # control takes the one-row path with the plain layer's handoff regions
    grow_n = moe.workspace_bytes(n, 1024) - moe.workspace_bytes(n, 1)
    grow_c = moe.workspace_bytes(c, 1024) - moe.workspace_bytes(c, 1)
    assert grow_n == grow_c + extra(1024) - extra(1)
    assert moe.workspace_bytes(n, 1) == moe.workspace_bytes(c, 1) + extra(1)
    L = moe.lib()
    TB = _fake_layers(40)
    X, Y, WS = 0x20000000, 0x30000000, 0x40000000
    eps = ctypes.c_float(1e-6)
    nb = moe.workspace_bytes(n, 1)
    assert L.moe_forward_stack(ctypes.byref(n), TB, 40, X, 1, eps, Y, None, WS, nb, None) == -5
    w = _fake_weights()
    gemv = _cfg(flags=moe.NO_ACT_QUANT | moe.FORCE_GEMV)
    assert _fwd(gemv, w, X, 1, Y, WS, moe.workspace_bytes(gemv, 1)) == -5  # no gfx950 here


def _a256(b):
    return (b + 255) // 256 * 256


def test_shared_fp8_flag():
    """The block-FP8 shared flag is known, adds its own workspace regions,
    needs the three shared scale arrays, and is refused with the control and
    in a stack."""
    c, f = _cfg(), _cfg(flags=moe.SHARED_FP8)
    s = inputs.DECODE
    # per-row regions of its own (pair list, tile list and count, h codes and
    # scales) on top of the plain layout's
    grow_f = moe.workspace_bytes(f, 1024) - moe.workspace_bytes(f, 1)
    grow_c = moe.workspace_bytes(c, 1024) - moe.workspace_bytes(c, 1)
    assert grow_f > grow_c
    # the one-row path's handoff regions, for its 4 rows in 8 copies of
    # 8-byte words: no bf16 hs, and h of K + 1 slots (the shared expert is
    # slot K) instead of K
    R, td, K, I, Is = 8, 4, s.top_k, s.inter, s.shared_inter
    own = _a256(4) + _a256(16) + _a256(4) + _a256(Is) + _a256(Is // 128 * 4)
    handoff = (_a256(R * td * (K + 1) * I * 8) - _a256(R * td * K * I * 8)
               - _a256(R * td * Is * 8))
    assert moe.workspace_bytes(f, 1) == moe.workspace_bytes(c, 1) + own + handoff
    # Is != I: the one-row kernel cannot take the block-FP8 shared expert as a
    # slot, so that config has no handoff regions at all
    odd = _cfg(shared_inter=2 * s.inter, flags=moe.SHARED_FP8)
    odd_plain = _cfg(shared_inter=2 * s.inter)
    assert moe.workspace_bytes(odd, 1) < moe.workspace_bytes(odd_plain, 1)
    assert moe.workspace_bytes(_cfg(flags=moe.SHARED_FP8 | moe.NO_ACT_QUANT), 1) == 0
    L = moe.lib()
    TB = _fake_layers(40)
    X, Y, WS = 0x20000000, 0x30000000, 0x40000000
    eps = ctypes.c_float(1e-6)
    nf = moe.workspace_bytes(f, 1)
    assert L.moe_forward_stack(ctypes.byref(f), TB, 40, X, 1, eps, Y, None, WS, nf, None) == -5
    w = _fake_weights()
    assert _fwd(f, w, X, 1, Y, WS, nf) == -5  # valid, but no gfx950 device here
    w.sh_s_down = None
    assert _fwd(f, w, X, 1, Y, WS, nf) == -1  # the scales are required
    w = _fake_weights()
    w.sh_s_up = w.sh_s_up + 2
    assert _fwd(f, w, X, 1, Y, WS, nf) == -3
    assert _fwd(c, _fake_weights(), X, 1, Y, WS, moe.workspace_bytes(c, 1)) == -5


def test_bf16_gemv_refusals():
    L = moe.lib()
    W, X, Y = 0x20000000, 0x30000000, 0x40000000
    assert L.moe_bf16_gemv(W, 16, 100, X, 1, Y, None) == -2     # K not a multiple of 128
    assert L.moe_bf16_gemv(W, 16, 16384, X, 1, Y, None) == -2   # K beyond 8192
    assert L.moe_bf16_gemv(W, 16, 2048, X, 5, Y, None) == -2    # more than 4 rows
    assert L.moe_bf16_gemv(W, -1, 2048, X, 1, Y, None) == -2
    assert L.moe_bf16_gemv(W, 0, 2048, X, 1, Y, None) == 0       # no-op
    assert L.moe_bf16_gemv(W, 16, 2048, X, 0, Y, None) == 0      # no-op
    assert L.moe_bf16_gemv(None, 16, 2048, X, 1, Y, None) == -1
    assert L.moe_bf16_gemv(W + 8, 16, 2048, X, 1, Y, None) == -3
    assert L.moe_bf16_gemv(W, 16, 2048, X, 1, Y + 1, None) == -3
    assert L.moe_bf16_gemv(W, 16, 2048, X, 1, X, None) == -5     # y aliases x
    assert L.moe_bf16_gemv(W, 16, 2048, X, 1, Y, None) == -5     # no gfx950 device here


def test_flag_values_match_the_header():
    src = open(HEADER).read()
    vals = {m.group(1): 1 << int(m.group(2))
            for m in re.finditer(r"#define\s+MOE_(\w+)\s+\(1u\s*<<\s*(\d+)\)", src)}
    assert vals == {"SHARED_FP8": moe.SHARED_FP8, "LOGITS_FP32": moe.LOGITS_FP32,
                    "NO_ACT_QUANT": moe.NO_ACT_QUANT, "FORCE_GEMV": moe.FORCE_GEMV,
                    "FORCE_GROUPED": moe.FORCE_GROUPED}
    # and the weights struct has the header's fields, in order
    body = re.search(r"typedef struct \{(.*?)\} moe_weights;", src, re.S).group(1)
    names = re.findall(r"\*\s*(\w+);", body)
    assert names == [n for n, _ in moe.Weights._fields_]


def test_noalloc_refusals_without_a_device():
    """moe_forward_noalloc refuses, before touching any device, a call whose
    workspace would not fit its 32 MiB array, and otherwise reports what
    moe_forward reports (here: no gfx950 device)."""
    L = moe.lib()
    c = _cfg()
    w = _fake_weights()
    X, Y = 0x20000000, 0x30000000
    assert moe.workspace_bytes(c, 600) <= moe.NOALLOC_WORKSPACE_BYTES
    assert moe.workspace_bytes(c, 1024) > moe.NOALLOC_WORKSPACE_BYTES
    assert L.moe_forward_noalloc(ctypes.byref(c), ctypes.byref(w), X, 1024, Y, None) == -4
    assert L.moe_forward_noalloc(ctypes.byref(c), ctypes.byref(w), X, 0, Y, None) == 0
    assert L.moe_forward_noalloc(ctypes.byref(c), ctypes.byref(w), X, -1, Y, None) == -2
    assert L.moe_forward_noalloc(ctypes.byref(c), ctypes.byref(w), None, 1, Y, None) == -1
    assert L.moe_forward_noalloc(ctypes.byref(c), ctypes.byref(w), X + 8, 1, Y, None) == -3
    assert L.moe_forward_noalloc(ctypes.byref(c), ctypes.byref(w), X, 1, Y, None) == -5
    assert L.moe_forward_noalloc(None, ctypes.byref(w), X, 1, Y, None) == -1


def test_decode_status_refusals_without_a_device():
    """moe_decode_status checks its pointers on the host; a valid call needs a
    gfx950 device."""
    L = moe.lib()
    WS, OUT = 0x40000000, 0x50000000
    assert L.moe_decode_status(None, OUT, 0, None) == -1
    assert L.moe_decode_status(WS, None, 0, None) == -1
    assert L.moe_decode_status(WS + 16, OUT, 0, None) == -3
    assert L.moe_decode_status(WS, OUT + 2, 1, None) == -3
    assert L.moe_decode_status(WS, OUT, 1, None) == -5


def test_e4m3_encode_refusals_without_a_device():
    L = moe.lib()
    X, Q = 0x20000000, 0x30000000
    assert L.moe_e4m3_encode(X, 0, Q, None) == 0
    assert L.moe_e4m3_encode(X, -1, Q, None) == -2
    assert L.moe_e4m3_encode(None, 4, Q, None) == -1
    assert L.moe_e4m3_encode(X, 4, None, None) == -1
    assert L.moe_e4m3_encode(X + 4, 4, Q, None) == -3
    assert L.moe_e4m3_encode(X, 4, Q + 1, None) == -3
    assert L.moe_e4m3_encode(X, 4, Q, None) == -5
