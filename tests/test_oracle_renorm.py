"""The stack renormalisation of the oracle against closed forms and
invariants (no re-typed formula): a single nonzero element maps to
+-sqrt(H), a constant row to +-1, scaling by a power of two changes nothing,
outputs have unit RMS, eps keeps a zero row at zero, rows are independent."""
import numpy as np
import torch

from tests import exact

H = 2048


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def _vals(bits):
    return exact.bits_to_f32(bits).astype(np.float64)


def test_single_nonzero_maps_to_sqrt_h(oracle_lib):
    for a in (1.0, -3.0, 0.375, 1024.0):
        y = np.zeros((1, H), dtype=np.float32)
        y[0, 17] = a
        x = _vals(oracle_lib.rms_renorm(_bf16(y), eps=0.0))
        want = np.sign(a) * _vals(exact.f32_to_bf16_torch(np.float32(np.sqrt(H))))
        assert x[0, 17] == want
        assert np.all(np.delete(x[0], 17) == 0)


def test_constant_row_maps_to_one(oracle_lib):
    for c in (1.0, -2.5, 3.0, 1e-3, 300.0):
        y = np.full((1, H), c, dtype=np.float32)
        x = _vals(oracle_lib.rms_renorm(_bf16(y), eps=0.0))
        assert np.all(x == np.sign(c))


def test_power_of_two_scaling_invariance(oracle_lib):
    rng = np.random.default_rng(0)
    y = _bf16(rng.standard_normal((4, H)) * 0.7)
    x0 = oracle_lib.rms_renorm(y, eps=0.0)
    for k in (-6, -1, 3, 9):
        xk = oracle_lib.rms_renorm(y.float().mul(2.0 ** k).to(torch.bfloat16), eps=0.0)
        assert np.array_equal(x0, xk)


def test_unit_rms_and_sign(oracle_lib):
    rng = np.random.default_rng(1)
    yv = rng.standard_normal((6, H)) * np.array([[0.01], [0.1], [1], [5], [40], [300]])
    y = _bf16(yv)
    x = _vals(oracle_lib.rms_renorm(y, eps=0.0))
    rms = np.sqrt((x ** 2).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) < 2 ** -8)
    yb = y.float().numpy()
    assert np.all(np.sign(x) == np.sign(yb))
    # the ratio x / y is one number per row, up to bf16 rounding of x
    nz = yb != 0
    ratio = x[nz] / yb[nz]
    per_row = np.broadcast_to(np.nanmedian(np.where(nz, x / np.where(nz, yb, 1), np.nan),
                                           axis=1)[:, None], yb.shape)[nz]
    assert np.all(np.abs(ratio / per_row - 1) <= 2 ** -8)


def test_eps_keeps_zero_row_and_damps_tiny_rows(oracle_lib):
    y = np.zeros((2, H), dtype=np.float32)
    y[1] = 2.0 ** -12            # mean square 2^-24 is well below eps = 1e-6
    x = _vals(oracle_lib.rms_renorm(_bf16(y), eps=1e-6))
    assert np.all(x[0] == 0)
    want = 2.0 ** -12 / np.sqrt(2.0 ** -24 + 1e-6)
    assert np.all(np.abs(x[1] - want) <= want * 2 ** -8)


def test_rows_independent(oracle_lib):
    rng = np.random.default_rng(2)
    y = _bf16(rng.standard_normal((5, H)))
    full = oracle_lib.rms_renorm(y)
    for t in range(5):
        assert np.array_equal(full[t], oracle_lib.rms_renorm(y[t:t + 1])[0])
