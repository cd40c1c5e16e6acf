"""Exact instances of the whole layer.

Weights and inputs are built so that every value the layer computes is
exactly representable and every sum is exact in any order. The layer output
then has one correct answer, bit for bit, whatever summation order the
block-FP8 GEMMs use. This is what lets a test compare the oracle and both GPU
paths with exact expectations instead of a tolerance.

The construction (G = H/128 activation groups):

- **x.** Column 128g+127 holds 448 in every group, so each group's scale is
  amax/448 = 1 and the codes equal the values. Column 126 holds 64. Column
  e of the routing list holds 16 when expert e is picked for that row, and 0
  otherwise. The other columns hold integers in [-4, 4].
- **Router.** Row e has a single 1 at expert e's routing column. A row's
  logits are therefore 16 on its K experts and 0 elsewhere. The K picks tie,
  so each weight is exactly 1/K and the ids come out in ascending order.
- **Gate.** Rows carry a sign sigma. The codes are sigma*16 on the 448
  columns and {-1, 0, 1} on the routing and data columns. The scales are
  powers of two, chosen so |g| >= 100. With such g, silu(g) is exactly g
  (sigma = +1) or -0 (sigma = -1, where exp overflows): the same bits for
  any exp implementation.
- **Up.** Up to 3 small codes per row on data columns, so |u| <= 24 units.
- **Marker rows.** The first row of every 128-row block has gate = the 448
  columns only, and up = 1 on the 64 column. Its h = g*u is then the group's
  unique maximum and equals 448*2^k, so the requantisation scale of h is
  the power of two 2^k. The h codes are exact divisions by that scale.
- **Down.** One code per row from {±1, ±1.5, ±2, ±3}, with power-of-two
  scales. Each e_j is then a short-mantissa value that bf16 holds exactly,
  so staging e_j in bf16 loses nothing.
- **Shared expert.**
  - Gate rows: a single ±1 on column 127, so gs = ±448.
  - Up rows: a single small value on a data column.
  - Down: small integers times 2^-12.
  - Gate vector: 1 on column 127, so gamma = sigmoid(448) = 1 exactly.

The expected output is computed here in float64. Every step asserts that its
values are exactly representable in the format the layer uses. The e4m3
codes of h come from the exhaustive nearest-code search in `tests.exact`, so
nothing here calls the oracle.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from block_fp8_mixture_router_amd import inputs
from tests import exact

GROUP = 128


def _code_lut(scale: float = 1.0) -> np.ndarray:
    """Maps int8 v (as v + 128) to the e4m3 code of the value v * scale, for
    every v whose value e4m3 holds exactly (others map to 0xFF, never used)."""
    table = exact.e4m3_table_torch()
    lut = np.full(256, 0xFF, dtype=np.uint8)
    for v in range(-128, 128):
        hits = [c for c in range(256) if table[c] == v * scale and c != 0x80]
        if hits:
            lut[v + 128] = hits[0]
    return lut


def _codes(vals: np.ndarray, scale: float = 1.0) -> np.ndarray:
    out = _code_lut(scale)[vals.astype(np.int16) + 128]
    assert not np.any(out == 0xFF)
    return out


def _bf16_exact(a: np.ndarray) -> bool:
    f = np.asarray(a, dtype=np.float32)
    b = exact.f32_to_bf16_torch(f)
    return bool(np.array_equal(exact.bits_to_f32(b), f))


def _f32_exact(a: np.ndarray) -> bool:
    a = np.asarray(a, dtype=np.float64)
    return bool(np.array_equal(a.astype(np.float32).astype(np.float64), a))


def _lowest_bit(a: np.ndarray) -> float:
    """The largest power of two dividing every nonzero value of a."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    a = np.unique(a[a > 0])
    if a.size == 0:
        return 1.0
    m, e = np.frexp(a)                      # a = m * 2^e, m in [0.5, 1)
    mi = (m * 2.0 ** 53).astype(np.int64)   # exact integer significands
    low = mi & -mi                          # lowest set bit, a power of two
    return float(np.min(np.ldexp(low.astype(np.float64), e - 53)))


def _assert_sums_exact(abs_total: np.ndarray, granule: float, what: str):
    """Every partial sum of terms that are multiples of `granule` with total
    magnitude <= abs_total fits fp32's 24-bit significand."""
    worst = float(np.max(abs_total)) / granule
    assert worst < 2.0 ** 24, f"{what}: sums need {np.log2(worst):.1f} bits"


@dataclasses.dataclass
class ExactInstance:
    shape: inputs.LayerShape
    weights: inputs.LayerWeights   # CPU tensors
    x: torch.Tensor                # bf16 [T, H]
    ids: np.ndarray                # [T, K] int32
    y_bits: np.ndarray             # [T, H] uint16, the exact answer rounded to bf16
    acc: np.ndarray                # [T, H] fp32, the exact pre-rounding sum


def _columns(H: int, E: int):
    usable = [c for c in range(H) if c % GROUP not in (GROUP - 2, GROUP - 1)]
    assert len(usable) >= E
    route = usable[:E]
    data = usable[E:]
    return route, np.array(data)


def build(shape: inputs.LayerShape, T: int, seed: int = 0, rows=None,
          act_scales: bool = False) -> ExactInstance:
    """An exact instance with T rows. The expected output is computed for
    `rows` only (all rows when None); the other rows of y_bits/acc are 0.

    With act_scales, group g's 448 column holds 448 * 2^a_g (a_g in 0..2, per
    group), so x's activation scales are 1, 2 and 4 across the groups and the
    codes are x / 2^a_g (still exact in e4m3); the gate blocks' scales carry
    2^-a_g, so the marker rows stay as above. A kernel that takes a group's
    activation scale from the wrong group then changes bits."""
    H, E, K, I, Is = shape.hidden, shape.n_experts, shape.top_k, shape.inter, shape.shared_inter
    G, NB = H // GROUP, I // GROUP
    assert G & (G - 1) == 0, "the marker construction needs a power-of-two group count"
    rng = np.random.default_rng(seed)
    route, data = _columns(H, E)
    bias_cols = np.arange(G) * GROUP + GROUP - 1
    one_col = GROUP - 2

    # ---- x and the routing it encodes
    picks = np.stack([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)])
    a_g = rng.integers(0, 3, size=G) if act_scales else np.zeros(G, dtype=np.int64)
    x = np.zeros((T, H))
    x[:, bias_cols] = 448.0 * 2.0 ** a_g
    x[:, one_col] = 64.0
    x[:, data] = rng.integers(-4, 5, size=(T, data.size))
    if act_scales:
        # data values in group g are multiples of 2^a_g, so x / 2^a_g stays an
        # integer and every sum keeps the granularity the bounds above assume
        step = 2.0 ** a_g[data // GROUP]
        x[:, data] = np.round(x[:, data] / step) * step
    for t in range(T):
        x[t, np.array(route)[picks[t]]] = 16.0
    assert _bf16_exact(x)

    wr = np.zeros((E, H))
    wr[np.arange(E), route] = 1.0

    # ---- expert weights as small integers (int8), codes and power-of-two scales
    gate_cols = np.concatenate([np.array(route), data])
    data_bound = 4 * 1 * data.size + 16 * K        # |x| * |code| over routing + data cols
    bias_min = 448 * 16 * (G / 2 if G >= 4 else G)  # marker gate value in code units
    p_hi = int(np.floor(np.log2((bias_min - data_bound) / 100)))
    other = np.setdiff1d(np.arange(H), gate_cols)
    wg = rng.integers(-1, 2, size=(E, I, H), dtype=np.int8)
    wg[:, :, other] = 0
    sigma = rng.choice(np.array([-1, 1], dtype=np.int8), size=(E, I))
    wg[:, :, bias_cols] = (16 * sigma)[:, :, None]
    wg[:, ::GROUP, :] = 0
    wg[:, ::GROUP, bias_cols] = 16
    # k-block exponents r_b per (expert, row block): sum of 2^-r_b is a power of
    # two, so the marker's gate value is 7 * 2^m
    if G >= 4:
        pattern = np.array([0] * (G // 4) + [1] * (G // 4) + [2] * (G // 2))
    else:
        pattern = np.zeros(G, dtype=np.int64)
    r = rng.permuted(np.broadcast_to(pattern, (E, NB, G)).copy(), axis=2)
    p = p_hi - rng.integers(0, 2, size=(E, NB))
    sg = 2.0 ** -(p[:, :, None] + r + a_g[None, None, :]).astype(np.float64)
    su = np.broadcast_to(2.0 ** -rng.integers(7, 9, size=(E, NB, 1)).astype(np.float64),
                         (E, NB, G)).copy()
    wu = np.zeros((E, I, H), dtype=np.int8)
    cols = data[rng.integers(0, data.size, size=(E, I, 3))]
    ei, ni = np.meshgrid(np.arange(E), np.arange(I), indexing="ij")
    for c in range(3):
        wu[ei, ni, cols[:, :, c]] = rng.choice(np.array([-2, -1, 1, 2], dtype=np.int8),
                                               size=(E, I))
    wu[:, ::GROUP, :] = 0
    wu[:, ::GROUP, one_col] = 1
    wd2 = np.zeros((E, H, I), dtype=np.int8)      # twice the down values
    ei, mi = np.meshgrid(np.arange(E), np.arange(H), indexing="ij")
    wd2[ei, mi, rng.integers(0, I, size=(E, H))] = rng.choice(
        np.array([-6, -4, -3, -2, 2, 3, 4, 6], dtype=np.int8), size=(E, H))
    sd = 2.0 ** -rng.integers(0, 4, size=(E, H // GROUP, NB)).astype(np.float64)

    # ---- shared expert (bf16)
    if Is > 0:
        shg = np.zeros((Is, H))
        shg[:, GROUP - 1] = rng.choice([-1.0, 1.0], size=Is)
        shu = np.zeros((Is, H))
        shu[np.arange(Is), rng.choice(data, Is)] = rng.choice([-2.0, -1.0, 1.0, 2.0], size=Is)
        shd = rng.integers(-2, 3, size=(H, Is)) * 2.0 ** -12
    else:
        shg = np.zeros((0, H)); shu = np.zeros((0, H)); shd = np.zeros((H, 0))
    gw = np.zeros(H)
    gw[GROUP - 1] = 1.0

    # ---- the exact forward pass (float64, every step checked)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    expand = lambda s: np.kron(s, np.ones((GROUP, GROUP)))  # noqa: E731
    dense = {}

    def expert(e):
        if e not in dense:
            wg_f = wg[e].astype(np.float64) * expand(sg[e])
            wu_f = wu[e].astype(np.float64) * expand(su[e])
            wd_f = 0.5 * wd2[e].astype(np.float64) * expand(sd[e])
            dense[e] = (wg_f, wu_f, wd_f, _lowest_bit(wg_f), _lowest_bit(wu_f))
        return dense[e]

    logits = x @ wr.T
    assert set(np.unique(logits)) <= {0.0, 16.0}
    table = exact.e4m3_table_torch()
    acc = np.zeros((T, H))
    abs_sum = np.zeros((T, H))
    granule = 1.0
    for t in rows:
        for j in range(K):
            wg_f, wu_f, wd_f, lg, lu = expert(picks[t, j])
            g, u = wg_f @ x[t], wu_f @ x[t]
            _assert_sums_exact(np.abs(wg_f) @ np.abs(x[t]), min(lg, 1.0), "gate")
            _assert_sums_exact(np.abs(wu_f) @ np.abs(x[t]), min(lu, 1.0), "up")
            assert np.all((g >= 32) | (g <= -100)), "silu would not be exact"
            h = np.where(g >= 32, g, -0.0) * u
            assert _f32_exact(h)
            hg = h.reshape(NB, GROUP)
            amax = np.abs(hg).max(axis=1)
            assert np.all(np.abs(hg[:, 0]) == amax) and np.all(
                np.abs(hg[:, 1:]) < amax[:, None]), "marker is not the unique max"
            s_h = amax / 448.0
            assert np.all(np.frexp(s_h)[0] == 0.5), "h scale is not a power of two"
            codes = exact.e4m3_nearest_bruteforce((hg / s_h[:, None]).reshape(-1))
            hq = (table[codes.astype(np.int64)].reshape(NB, GROUP) * s_h[:, None]).reshape(-1)
            ej = wd_f @ hq
            assert _bf16_exact(ej), "e_j is not exact in bf16"
            acc[t] += ej / K
            abs_sum[t] += np.abs(ej) / K
            granule = min(granule, _lowest_bit(ej / K))
    if Is > 0:
        xs = x[rows]
        gs, us = xs @ shg.T, xs @ shu.T
        hs = np.where(gs >= 32, gs, -0.0) * us
        assert _bf16_exact(hs)
        sh = hs @ shd.T
        _assert_sums_exact(np.abs(hs) @ np.abs(shd.T), min(_lowest_bit(shd), 64.0), "shared")
        assert _f32_exact(sh)
        acc[rows] += sh                     # gamma = sigmoid(448) = 1
        abs_sum[rows] += np.abs(sh)
        granule = min(granule, _lowest_bit(sh))
    _assert_sums_exact(abs_sum, granule, "combine")
    assert _f32_exact(acc)
    y_bits = exact.f32_to_bf16_torch(acc.astype(np.float32))

    # ---- pack as a layer
    to_bf16 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)  # noqa
    w = inputs.LayerWeights(
        shape=shape, router_w=to_bf16(wr), router_bias=None,
        w_gate=torch.from_numpy(_codes(wg)), s_gate=torch.from_numpy(sg.astype(np.float32)),
        w_up=torch.from_numpy(_codes(wu)), s_up=torch.from_numpy(su.astype(np.float32)),
        w_down=torch.from_numpy(_codes(wd2, 0.5)), s_down=torch.from_numpy(sd.astype(np.float32)),
        sh_gate=to_bf16(shg), sh_up=to_bf16(shu), sh_down=to_bf16(shd), sh_gate_w=to_bf16(gw))
    return ExactInstance(shape, w, to_bf16(x), picks.astype(np.int32), y_bits,
                         acc.astype(np.float32))


def zero_sign_blind(bits: np.ndarray) -> np.ndarray:
    """bf16 bits with -0 mapped to +0 (the sign of an exact zero depends on
    the order in which zeros are added)."""
    b = np.asarray(bits, dtype=np.uint16).copy()
    b[b == 0x8000] = 0
    return b
