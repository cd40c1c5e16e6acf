"""Pins of the oracle's residual add + RMS norm + 1x128 quantisation (the
step in front of the layer), against values it does not compute itself:
torch's own bf16 rounding of the fp32 sums, a float64 evaluation of the norm,
the stack renormalisation it reduces to, exact power-of-two invariances, and
the quantiser applied to its output."""
import numpy as np
import pytest
import torch

import oracle
from tests import exact


def _rows(T, H, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(T, H, generator=g) * scale).to(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def _from_bits(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("T,H", [(3, 256), (2, 2048)])
def test_residual_is_bf16_of_the_fp32_sum(T, H):
    h, r = _rows(T, H, 1), _rows(T, H, 2, scale=3.0)
    w = _rows(1, H, 3)[0]
    ro, _, _, _ = oracle.add_rmsnorm_quant(h, r, w)
    want = (h.float() + r.float()).to(torch.bfloat16)   # torch rounds fp32 -> bf16 to nearest even
    assert np.array_equal(ro, _bits(want))


def test_unit_gain_and_zero_residual_is_the_stack_renorm():
    h = _rows(4, 2048, 5)
    zeros = torch.zeros_like(h)
    ones = torch.ones(2048, dtype=torch.bfloat16)
    for eps in (1e-6, 0.0, 0.5):
        ro, x, q, s = oracle.add_rmsnorm_quant(h, zeros, ones, eps=eps)
        assert np.array_equal(ro, _bits(h))
        assert np.array_equal(x, oracle.rms_renorm(h, eps=eps))
        q2, s2 = oracle.quant_act(_from_bits(x))
        assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_norm_against_float64():
    h, r = _rows(3, 1024, 7), _rows(3, 1024, 8)
    w = (torch.rand(1024, generator=torch.Generator().manual_seed(9)) + 0.5).to(torch.bfloat16)
    eps = 1e-3
    ro, x, _, _ = oracle.add_rmsnorm_quant(h, r, w, eps=eps)
    rv = exact.bits_to_f32(ro).astype(np.float64)
    ref = rv / np.sqrt((rv ** 2).mean(axis=1, keepdims=True) + eps) * w.double().numpy()[None, :]
    got = exact.bits_to_f32(x).astype(np.float64)
    # bf16 output rounding (2^-9 relative) plus a few fp32 roundings
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


def test_power_of_two_scalings_are_exact():
    h, r = _rows(3, 512, 11), _rows(3, 512, 12)
    w = _rows(1, 512, 13)[0]
    ro, x, q, s = oracle.add_rmsnorm_quant(h, r, w, eps=0.0)
    # inputs x2: the residual doubles, the norm's scale halves, x is unchanged
    ro2, x2, q2, s2 = oracle.add_rmsnorm_quant(h * 2, r * 2, w, eps=0.0)
    assert np.array_equal(ro2, _bits(_from_bits(ro) * 2))
    assert np.array_equal(x2, x) and np.array_equal(q2, q) and np.array_equal(s2, s)
    # gain x2: x doubles exactly, the codes stay and the scales double
    ro3, x3, q3, s3 = oracle.add_rmsnorm_quant(h, r, w * 2, eps=0.0)
    assert np.array_equal(ro3, ro)
    assert np.array_equal(x3, _bits(_from_bits(x) * 2))
    assert np.array_equal(q3, q) and np.array_equal(s3, s * 2)


def test_constant_row_closed_form():
    # a constant row c with eps 0 normalises to sign(c) * 1 (times the gain);
    # the group amax then encodes to 448 with scale 1/448 * |gain|
    H = 256
    h = torch.full((2, H), 3.0, dtype=torch.bfloat16)
    h[1] = -0.375
    r = torch.zeros_like(h)
    w = torch.full((H,), 0.5, dtype=torch.bfloat16)
    _, x, q, s = oracle.add_rmsnorm_quant(h, r, w, eps=0.0)
    xf = exact.bits_to_f32(x)
    assert np.all(xf[0] == 0.5) and np.all(xf[1] == -0.5)
    assert np.all(q[0] == 0x7E) and np.all(q[1] == 0xFE)
    assert np.all(s == np.float32(0.5) / np.float32(448.0))


def test_zero_rows_use_the_clamped_scale():
    H = 384
    z = torch.zeros(2, H, dtype=torch.bfloat16)
    w = torch.ones(H, dtype=torch.bfloat16)
    ro, x, q, s = oracle.add_rmsnorm_quant(z, z, w, eps=1e-6)
    assert not ro.any() and not (x & 0x7FFF).any()
    assert not (q & 0x7F).any()
    assert np.all(s == np.float32(1e-10) / np.float32(448.0))


def test_rows_are_independent():
    h, r = _rows(5, 768, 21), _rows(5, 768, 22)
    w = _rows(1, 768, 23)[0]
    full = oracle.add_rmsnorm_quant(h, r, w)
    for t in (0, 3):
        one = oracle.add_rmsnorm_quant(h[t:t + 1], r[t:t + 1], w)
        for a, b in zip(full, one):
            assert np.array_equal(a[t:t + 1], b)
