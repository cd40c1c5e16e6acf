"""Pins of the oracle's 1x128 e4m3 activation quantiser.

The pages state the rule: per row and per 128 inputs, scale amax / 448, e4m3
codes (PR #939 "drama3: Fish Audio Drama 3 text to speech on one CUDA GPU",
"How it fits the engine" > Precision; PR #925, backbone commit summary:
dynamic 1 x 128 FP8 activation quantisation). Pins: an independent
brute-force quantiser (exhaustive nearest-code search), the amax-to-448
invariant, the rounding error bound, and the row/group layout.
"""
import numpy as np
import torch

from tests import exact


def _x(rows, cols, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(rows, cols, generator=g) * scale).to(torch.bfloat16)


def test_quant_act_matches_bruteforce(oracle_lib):
    for seed, (rows, cols, scale) in enumerate([(3, 256, 1.0), (5, 2048, 1.0),
                                                (2, 384, 1e-3), (4, 128, 50.0)]):
        x = _x(rows, cols, seed, scale)
        q, s = oracle_lib.quant_act(x)
        xf = x.float().numpy()
        qb, sb = exact.quant_groups_bruteforce(xf.reshape(-1))
        assert np.array_equal(s.reshape(-1), sb)
        assert np.array_equal(q.reshape(-1), qb.reshape(-1))


def test_quant_amax_element_encodes_to_448(oracle_lib):
    x = _x(64, 1024, 7)
    q, s = oracle_lib.quant_act(x)
    xf = x.float().numpy().reshape(64, 8, 128)
    qg = q.reshape(64, 8, 128)
    idx = np.abs(xf).argmax(axis=2)
    top = np.take_along_axis(qg, idx[..., None], axis=2)[..., 0]
    sign = np.take_along_axis(xf, idx[..., None], axis=2)[..., 0] < 0
    assert np.all(top == np.where(sign, 0xFE, 0x7E))
    # the scale times 448 reproduces amax to within one fp32 ulp
    amax = np.abs(xf).max(axis=2)
    assert np.allclose(s.reshape(64, 8) * 448.0, amax, rtol=2.0 ** -22, atol=0)


def test_quant_error_bound(oracle_lib):
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(128 * 512) * np.exp(rng.standard_normal(128 * 512) * 3)).astype(
        np.float32)
    q, s = oracle_lib.quant_groups(v)
    table = exact.e4m3_table_torch()
    deq = table[q.astype(np.int64)].reshape(-1, 128) * s[:, None]
    vv = v.reshape(-1, 128).astype(np.float64)
    ss = np.broadcast_to(s[:, None].astype(np.float64), vv.shape)
    err = np.abs(vv - deq)
    normal = np.abs(vv) / ss >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(vv[normal]) * (1 + 2.0 ** -20))
    assert np.all(err[~normal] <= 2.0 ** -10 * ss[~normal] * (1 + 2.0 ** -20))


def test_quant_zero_group_and_signed_zero(oracle_lib):
    v = np.zeros(256, dtype=np.float32)
    v[128:] = -0.0
    v[200] = -1e-30  # rounds to zero, keeps its sign
    v[201] = 3.0
    q, s = oracle_lib.quant_groups(v)
    assert s[0] == np.float32(np.float32(1e-10) / np.float32(448.0))
    assert np.all(q[:128] == 0)
    assert q[200] == 0x80 and q[201] == 0x7E
    assert np.all(q[128:200] == 0x80)


def test_quant_layout_rows_and_groups(oracle_lib):
    # each (row, group) gets a distinct amax so a shifted or transposed scale
    # index cannot pass
    rows, groups = 5, 6
    v = np.zeros((rows, groups * 128), dtype=np.float32)
    for t in range(rows):
        for g in range(groups):
            v[t, g * 128 + (t + g) % 128] = float(1 + t * groups + g)
    x = torch.from_numpy(v).to(torch.bfloat16)
    q, s = oracle_lib.quant_act(x)
    for t in range(rows):
        for g in range(groups):
            assert s[t, g] == np.float32(np.float32(1 + t * groups + g) / np.float32(448.0))
            assert q[t, g * 128 + (t + g) % 128] == 0x7E
    assert np.count_nonzero(q) == rows * groups
