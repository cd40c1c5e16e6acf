"""Python access to the plain CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the product path. It shares no code with
the HIP library.

``build()`` compiles ``libmoe_oracle.so`` next to this file with gcc
(-O2, no fast-math, no fp contraction, OpenMP). The wrappers take and return
numpy arrays or CPU torch tensors; bf16 arrays travel as their uint16 bit
patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
SOURCES = [os.path.join(_HERE, "moe_oracle.c")]

NO_ACT_QUANT = 1 << 0
LOGITS_FP32 = 1 << 1
SHARED_FP8 = 1 << 2  # shared expert stored block-FP8, run as the routed experts


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-std=c11",
           "-D_GNU_SOURCE", "-Wall", "-shared", "-fPIC", "-o", tmp] + SOURCES + ["-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "router_bias", "w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down",
        "sh_gate", "sh_up", "sh_down", "sh_gate_w", "sh_s_gate", "sh_s_up", "sh_s_down")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or any(
                os.path.getmtime(s) > os.path.getmtime(LIB_PATH) for s in SOURCES):
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_float
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode_n.argtypes = [vp, i64, vp]
        L.oracle_bf16_round.argtypes = [ctypes.c_float]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_round_n.argtypes = [vp, i64, vp]
        L.oracle_quant_groups.argtypes = [vp, i64, vp, vp]
        L.oracle_quant_act.argtypes = [vp, i64, i64, vp, vp]
        L.oracle_route.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp]
        L.oracle_forward.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp]
        L.oracle_rms_renorm.argtypes = [vp, i64, i64, ctypes.c_float, vp]
        L.oracle_bf16_gemv.argtypes = [vp, i64, i64, vp, i64, vp]
        L.oracle_add_rmsnorm_quant.argtypes = [vp, vp, vp, i64, i64, ctypes.c_float, vp, vp,
                                               vp, vp]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def _np(a, dtype=None):
    """numpy view of a CPU tensor or array; bf16 tensors become uint16."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.int16).numpy().view(np.uint16)
            else:
                a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if dtype is not None:
        assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def cfg_of(shape, flags: int = 0) -> _Cfg:
    return _Cfg(shape.hidden, shape.n_experts, shape.top_k, shape.inter, shape.shared_inter,
                flags)


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(code)


def e4m3_encode(values) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_n(_p(v), v.size, _p(out))
    return out


def bf16_round(values) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_bf16_round_n(_p(v), v.size, _p(out))
    return out


def quant_groups(values):
    """Quantise fp32 values in groups of 128 -> (codes uint8, scales fp32)."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    assert v.size % 128 == 0
    q = np.empty(v.shape, dtype=np.uint8)
    s = np.empty(v.size // 128, dtype=np.float32)
    lib().oracle_quant_groups(_p(v), v.size // 128, _p(q), _p(s))
    return q, s


def quant_act(x):
    """x bf16 [T, C] -> codes uint8 [T, C], scales fp32 [T, C/128]."""
    xa = _np(x, np.uint16)
    T, C = xa.shape
    q = np.empty((T, C), dtype=np.uint8)
    s = np.empty((T, C // 128), dtype=np.float32)
    lib().oracle_quant_act(_p(xa), T, C, _p(q), _p(s))
    return q, s


def rms_renorm(y, eps: float = 1e-6):
    """Stack renormalisation: y bf16 [T, H] -> x bf16 bits uint16 [T, H]."""
    ya = _np(y, np.uint16)
    T, H = ya.shape
    x = np.empty((T, H), dtype=np.uint16)
    lib().oracle_rms_renorm(_p(ya), T, H, eps, _p(x))
    return x


def add_rmsnorm_quant(hidden, residual, norm_w, eps: float = 1e-6):
    """Residual add, RMS norm and 1x128 quantisation of rows (bf16 [T, H]
    inputs, norm_w bf16 [H]) -> (new residual bf16 bits, normed x bf16 bits,
    codes uint8 [T, H], scales fp32 [T, H/128])."""
    ha = _np(hidden, np.uint16)
    ra = _np(residual, np.uint16)
    wa = _np(norm_w, np.uint16)
    T, H = ha.shape
    assert ra.shape == (T, H) and wa.shape == (H,)
    ro = np.empty((T, H), dtype=np.uint16)
    x = np.empty((T, H), dtype=np.uint16)
    q = np.empty((T, H), dtype=np.uint8)
    s = np.empty((T, H // 128), dtype=np.float32)
    lib().oracle_add_rmsnorm_quant(_p(ha), _p(ra), _p(wa), T, H, eps, _p(ro), _p(x), _p(q), _p(s))
    return ro, x, q, s


def bf16_gemv(W, x):
    """One-row bf16 projection: W bf16 [N, K], x bf16 [T, K] -> y bf16 bits
    [T, N], y = bf16(fp32(exact sum of products))."""
    wa = _np(W, np.uint16)
    xa = _np(x, np.uint16)
    N, K = wa.shape
    T = xa.shape[0]
    assert xa.shape == (T, K)
    y = np.empty((T, N), dtype=np.uint16)
    lib().oracle_bf16_gemv(_p(wa), N, K, _p(xa), T, _p(y))
    return y


def route(shape, x, router_w, router_bias=None, flags: int = 0):
    """-> ids int32 [T,K], weights fp32 [T,K], logits fp32 [T,E]."""
    xa = _np(x, np.uint16)
    T = xa.shape[0]
    rw = _np(router_w, np.uint16)
    rb = None if router_bias is None else _np(router_bias, np.float32)
    ids = np.empty((T, shape.top_k), dtype=np.int32)
    w = np.empty((T, shape.top_k), dtype=np.float32)
    lg = np.empty((T, shape.n_experts), dtype=np.float32)
    c = cfg_of(shape, flags)
    lib().oracle_route(ctypes.byref(c), _p(xa), T, _p(rw), _p(rb), _p(ids), _p(w), _p(lg))
    return ids, w, lg


def forward(shape, weights, x, flags: int = 0, shared: Optional[bool] = None):
    """Whole layer on host tensors.

    weights: an object with the tensor attributes of ``inputs.LayerWeights``.
    Returns (y bf16 bits uint16 [T,H], acc fp32 [T,H], ids [T,K], w [T,K]).
    """
    xa = _np(x, np.uint16)
    T = xa.shape[0]
    arrs = {}
    sh = np.uint8 if flags & SHARED_FP8 else np.uint16  # e4m3 codes or bf16
    dt = {"router_w": np.uint16, "router_bias": np.float32, "w_gate": np.uint8,
          "s_gate": np.float32, "w_up": np.uint8, "s_up": np.float32, "w_down": np.uint8,
          "s_down": np.float32, "sh_gate": sh, "sh_up": sh, "sh_down": sh,
          "sh_gate_w": np.uint16, "sh_s_gate": np.float32, "sh_s_up": np.float32,
          "sh_s_down": np.float32}
    for name, d in dt.items():
        a = getattr(weights, name, None)
        if shared is False and name.startswith("sh_"):
            a = None  # no shared expert: its matrices are never read
        arrs[name] = None if a is None else _np(a, d)
    W = _Weights(**{k: (None if v is None else v.ctypes.data) for k, v in arrs.items()})
    y = np.empty((T, shape.hidden), dtype=np.uint16)
    acc = np.empty((T, shape.hidden), dtype=np.float32)
    ids = np.empty((T, shape.top_k), dtype=np.int32)
    w = np.empty((T, shape.top_k), dtype=np.float32)
    c = cfg_of(shape, flags)
    if shared is False:
        c.shared_inter = 0
    lib().oracle_forward(ctypes.byref(c), ctypes.byref(W), _p(xa), T, _p(y), _p(acc),
                         _p(ids), _p(w))
    return y, acc, ids, w


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Worker threads of later oracle calls (timing only; results do not
    depend on it)."""
    lib().oracle_set_num_threads(int(n))


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)
