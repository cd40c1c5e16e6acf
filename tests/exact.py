"""Exact-arithmetic and brute-force helpers for pinning the oracle.

Nothing here calls the oracle: these are independent ways to reach values
the oracle must reproduce (exact rational dot products, nearest-value
searches over the whole e4m3 table, dense numpy references).
"""
from __future__ import annotations

import numpy as np
import torch

# ------------------------------------------------------------------ bf16 bits


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_torch(v) -> np.ndarray:
    """fp32 -> bf16 bits with torch's cast (a library routine, RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return bf16_bits(t)


# ---------------------------------------------------- exact dyadic arithmetic


def bf16_int_exp(bits: np.ndarray):
    """bf16 bit patterns -> (signed integer mantissa m, exponent e), value = m*2^e."""
    b = np.asarray(bits, dtype=np.int64)
    sign = np.where(b & 0x8000, -1, 1)
    ex = (b >> 7) & 0xFF
    man = b & 0x7F
    normal = ex != 0
    m = np.where(normal, man | 0x80, man) * sign
    e = np.where(normal, ex - 127 - 7, 1 - 127 - 7)
    assert not np.any(ex == 0xFF), "inf/nan not expected"
    return m, e


def exact_dot_bf16(xb: np.ndarray, wb: np.ndarray):
    """Exact sum of x_h*w_h over bf16 bit vectors, as (integer N, exponent E0):
    value = N * 2^E0."""
    mx, ex = bf16_int_exp(xb)
    mw, ew = bf16_int_exp(wb)
    p = mx * mw                       # |p| < 2^16, exact
    e = ex + ew
    e0 = int(e.min())
    total = 0
    for ev in np.unique(e):
        s = int(p[e == ev].sum())     # <= 2^16 * n, exact in int64
        total += s << int(ev - e0)
    return total, e0


def round_dyadic_to_f32(n: int, e0: int) -> np.float32:
    """Correctly round n*2^e0 to fp32 (nearest, ties to even). Normal range only."""
    if n == 0:
        return np.float32(0.0)
    sign = -1 if n < 0 else 1
    a = abs(n)
    nb = a.bit_length()           # a in [2^(nb-1), 2^nb)
    shift = nb - 24               # keep 24 significant bits
    if shift > 0:
        q, r = divmod(a, 1 << shift)
        half = 1 << (shift - 1)
        if r > half or (r == half and (q & 1)):
            q += 1
        m, e = q, e0 + shift
    else:
        m, e = a, e0
    v = np.float32(np.ldexp(np.float64(m), e))  # exact: m has <= 25 bits
    return np.float32(sign * v)


def exact_logits_bf16(xb_row: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    """bf16(fp32(exact x . w_e)) for every router row e, as fp32 values."""
    out = np.empty(wr_bits.shape[0], dtype=np.float32)
    for e in range(wr_bits.shape[0]):
        n, e0 = exact_dot_bf16(xb_row, wr_bits[e])
        out[e] = round_dyadic_to_f32(n, e0)
    return bits_to_f32(f32_to_bf16_torch(out))


# --------------------------------------------------------------- e4m3 tables


def e4m3_table_torch() -> np.ndarray:
    """Values of all 256 e4m3 codes via torch's float8_e4m3fn (a library decode)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e4m3_nearest_bruteforce(r: np.ndarray) -> np.ndarray:
    """Nearest finite e4m3 code to each value (after saturation to +-448), by
    exhaustive search over the table; ties go to the code with an even
    mantissa; the sign of r is kept (so -tiny -> 0x80)."""
    table = e4m3_table_torch()
    pos_codes = np.array([c for c in range(0x7F)], dtype=np.int64)  # 0x00..0x7E
    pos_vals = table[pos_codes]
    r = np.asarray(r, dtype=np.float64)
    a = np.minimum(np.abs(r), 448.0)
    d = np.abs(a[:, None] - pos_vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among equally near codes prefer the even mantissa
    even = (pos_codes & 1) == 0
    pick_even = cand & even[None, :]
    has_even = pick_even.any(axis=1)
    choice = np.where(has_even, np.argmax(pick_even, axis=1), np.argmax(cand, axis=1))
    code = pos_codes[choice]
    neg = np.signbit(r)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quant_groups_bruteforce(v: np.ndarray):
    """Independent per-128 quantiser: scale = fp32(max(amax,1e-10)/448) in numpy
    float32 (IEEE division), codes by exhaustive nearest search."""
    v = np.asarray(v, dtype=np.float32).reshape(-1, 128)
    amax = np.abs(v).max(axis=1)
    s = (np.maximum(amax, np.float32(1e-10)) / np.float32(448.0)).astype(np.float32)
    r = (v / s[:, None]).astype(np.float32)
    r = np.clip(r, np.float32(-448.0), np.float32(448.0))
    q = e4m3_nearest_bruteforce(r.reshape(-1)).reshape(v.shape)
    return q, s


# ---------------------------------------------------------- dense references


def dequant_block(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[N,K] e4m3 codes and [N/128,K/128] scales -> dense fp64 matrix."""
    table = e4m3_table_torch()
    return table[codes.astype(np.int64)] * np.kron(scales.astype(np.float64),
                                                    np.ones((128, 128)))


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))
