"""Pins of the oracle's number formats: e4m3 decode/encode and bf16 rounding.

Pinned against the published OCP E4M3 points (tests/golden), torch's own
float8_e4m3fn and bfloat16 casts (library routines), and an exhaustive
nearest-value search over the code table.
"""
import os

import numpy as np
import pytest
import torch

from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_points.txt")


def _golden_points():
    pts = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            c, v = line.split()
            pts.append((int(c, 16), v))
    return pts


def test_decode_golden_points(oracle_lib):
    for code, v in _golden_points():
        got = oracle_lib.e4m3_decode(code)
        if v == "nan":
            assert np.isnan(got), hex(code)
        elif v == "-0":
            assert got == 0.0 and np.signbit(got), hex(code)
        else:
            assert got == float(v), (hex(code), got, v)


def test_decode_all_codes_match_library_and_structure(oracle_lib):
    ours = np.array([oracle_lib.e4m3_decode(c) for c in range(256)], dtype=np.float64)
    lib = exact.e4m3_table_torch()
    both_nan = np.isnan(ours) & np.isnan(lib)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.all((ours == lib) | both_nan)
    # exactly two NaN codes, strictly increasing positive half, sign symmetry
    assert np.isnan(ours).sum() == 2
    pos = ours[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.all(ours[0x80:0xFF] == -ours[0x00:0x7F])
    # each binade above 2^-6 holds 8 evenly spaced values
    for ex in range(1, 16):
        vals = ours[ex * 8:(ex * 8 + 8)]
        vals = vals[~np.isnan(vals)]
        assert np.allclose(np.diff(vals), 2.0 ** (ex - 7 - 3))


def test_encode_all_bf16_values(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = exact.bits_to_f32(bits)
    finite = np.isfinite(vals)
    vals = vals[finite]
    got = oracle_lib.e4m3_encode(vals)
    want = exact.e4m3_nearest_bruteforce(vals)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_encode_matches_torch_cast_in_range(oracle_lib):
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 100,
        rng.standard_normal(200_000).astype(np.float32) * 0.01,
        np.float32(448.0) * (rng.random(50_000).astype(np.float32) * 2 - 1),
    ])
    # exact midpoints between neighbouring codes, and their fp32 neighbours
    table = exact.e4m3_table_torch()[:0x7F]
    mids = ((table[1:] + table[:-1]) / 2).astype(np.float32)
    mids = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1e9))])
    v = np.concatenate([v, mids, -mids]).astype(np.float32)
    v = np.clip(v, -448, 448)
    got = oracle_lib.e4m3_encode(v)
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps +0 for negative values that round to zero; compare magnitudes there
    zero = (got & 0x7F) == 0
    assert np.array_equal(got[~zero], lib[~zero])
    assert np.all((lib[zero] & 0x7F) == 0)
    assert np.all(got[zero] == np.where(np.signbit(v[zero]), 0x80, 0x00))
    want = exact.e4m3_nearest_bruteforce(v[:20000])
    assert np.array_equal(got[:20000], want)


def test_encode_saturates_and_nan(oracle_lib):
    got = oracle_lib.e4m3_encode(np.array([448.0, 449.0, 1e30, -1e30, -464.0, np.nan],
                                          dtype=np.float32))
    assert list(got[:5]) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert got[5] == 0x7F


def test_bf16_round_matches_torch(oracle_lib):
    rng = np.random.default_rng(2)
    u = rng.integers(0, 2**32, size=500_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties: low 16 bits = 0x8000
    ties = (u[:50_000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u = np.concatenate([u, ties])
    v = u.view(np.float32)
    v = v[np.isfinite(v)]
    got = oracle_lib.bf16_round(v)
    want = exact.f32_to_bf16_torch(v)
    assert np.array_equal(got, want)
