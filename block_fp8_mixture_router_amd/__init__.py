"""Python binding of libmoe, the gfx950 block-FP8 MoE layer (include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
Tensors are torch tensors on the current device; the stream is torch's current
stream. If the library is missing or the device is not gfx950 the calls raise
(there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_E_NULL", -2: "MOE_E_SHAPE", -3: "MOE_E_ALIGN",
          -4: "MOE_E_WORKSPACE", -5: "MOE_E_UNSUPPORTED", -6: "MOE_E_LAUNCH"}
LOGITS_FP32 = 1 << 1
SHARED_FP8 = 1 << 0  # shared expert stored block-FP8 (grouped path)
NO_ACT_QUANT = 1 << 2  # fidelity control: no activation quantisation (grouped path)
FORCE_GEMV = 1 << 8
FORCE_GROUPED = 1 << 9

EXPORTS = ("moe_supported", "moe_workspace_bytes", "moe_route", "moe_quant_act",
           "moe_forward", "moe_rms_renorm", "moe_forward_stack", "moe_add_rmsnorm_quant",
           "moe_bf16_gemv", "moe_forward_noalloc", "moe_decode_status", "moe_e4m3_encode")


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "router_bias", "w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down",
        "sh_gate", "sh_up", "sh_down", "sh_gate_w", "sh_s_gate", "sh_s_up", "sh_s_down")]


_lib = None


def lib():
    """Load libmoe.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (loads the HIP runtime torch uses)
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() or "
                "python block_fp8_mixture_router_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.moe_supported.argtypes = [ctypes.c_int]
        L.moe_supported.restype = ctypes.c_int
        L.moe_workspace_bytes.argtypes = [vp, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_route.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_route.restype = ctypes.c_int
        L.moe_quant_act.argtypes = [vp, i32, i32, vp, vp, vp]
        L.moe_quant_act.restype = ctypes.c_int
        L.moe_forward.argtypes = [vp, vp, vp, i32, vp, vp, sz, vp]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward_noalloc.argtypes = [vp, vp, vp, i32, vp, vp]
        L.moe_forward_noalloc.restype = ctypes.c_int
        L.moe_decode_status.argtypes = [vp, vp, i32, vp]
        L.moe_decode_status.restype = ctypes.c_int
        L.moe_e4m3_encode.argtypes = [vp, ctypes.c_int64, vp, vp]
        L.moe_e4m3_encode.restype = ctypes.c_int
        L.moe_rms_renorm.argtypes = [vp, i32, i32, ctypes.c_float, vp, vp]
        L.moe_rms_renorm.restype = ctypes.c_int
        L.moe_add_rmsnorm_quant.argtypes = [vp, vp, vp, vp, i32, i32, ctypes.c_float, vp, vp,
                                            vp, vp]
        L.moe_add_rmsnorm_quant.restype = ctypes.c_int
        L.moe_bf16_gemv.argtypes = [vp, i32, i32, vp, i32, vp, vp]
        L.moe_bf16_gemv.restype = ctypes.c_int
        L.moe_forward_stack.argtypes = [vp, vp, i32, vp, i32, ctypes.c_float, vp, vp, vp, sz, vp]
        L.moe_forward_stack.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status)


def config(shape, flags: int = 0, shared: bool = True) -> Config:
    return Config(shape.hidden, shape.n_experts, shape.top_k, shape.inter,
                  shape.shared_inter if shared else 0, flags)


def supported(device: int = 0) -> bool:
    return bool(lib().moe_supported(device))


def workspace_bytes(cfg: Config, max_rows: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(cfg), max_rows))


def alloc_workspace(cfg: Config, max_rows: int, device="cuda"):
    """A zero-filled workspace (the library requires zero before first use)."""
    import torch
    n = workspace_bytes(cfg, max_rows)
    if n == 0:
        raise MoeError("moe_workspace_bytes", -2)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def weights_array(layers):
    """A host array of moe_weights structs for moe_forward_stack, from
    objects with the tensor attributes of inputs.LayerWeights or from Weights
    structs (the caller keeps the layers' tensors alive)."""
    structs = [lw if isinstance(lw, Weights) else weights_struct(lw) for lw in layers]
    return (Weights * len(structs))(*structs)


def forward_stack(cfg: Config, layers, x, y=None, ys=None, eps: float = 1e-6,
                  workspace=None, stream=None):
    """The layers in sequence on the rows x (T <= 4), each layer after the
    first renormalising its predecessor's output in its own launch; equals
    forward() and rms_renorm() called in turn, bit for bit. layers: a list
    (see weights_array) or an array from weights_array(). ys, if given, gets
    every layer's output [n_layers, T, H]. Returns the last layer's output."""
    import torch
    T = x.shape[0]
    arr = layers if isinstance(layers, ctypes.Array) else weights_array(layers)
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(cfg, max(T, 1), x.device)
    _check("moe_forward_stack", lib().moe_forward_stack(
        ctypes.byref(cfg), arr, len(arr), _ptr(x), T, eps, _ptr(y), _ptr(ys),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def rms_renorm(y, x=None, eps: float = 1e-6, stream=None):
    """Row RMS normalisation between stacked layers: x = bf16(y / rms(y))."""
    import torch
    T, H = y.shape
    if x is None:
        x = torch.empty_like(y)
    _check("moe_rms_renorm", lib().moe_rms_renorm(_ptr(y), T, H, eps, _ptr(x), _stream(stream)))
    return x


def add_rmsnorm_quant(hidden, residual, norm_w, eps: float = 1e-6, residual_out=None, x=None,
                      q=None, scales=None, stream=None):
    """Residual add, RMS norm and 1x128 quantisation of the normed rows.
    Returns (residual_out, x, q, scales); residual_out may be `residual`
    (in place)."""
    import torch
    T, H = hidden.shape
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    if x is None:
        x = torch.empty_like(hidden)
    if q is None:
        q = torch.empty((T, H), dtype=torch.uint8, device=hidden.device)
    if scales is None:
        scales = torch.empty((T, H // 128), dtype=torch.float32, device=hidden.device)
    _check("moe_add_rmsnorm_quant", lib().moe_add_rmsnorm_quant(
        _ptr(hidden), _ptr(residual), _ptr(residual_out), _ptr(norm_w), T, H, eps, _ptr(x),
        _ptr(q), _ptr(scales), _stream(stream)))
    return residual_out, x, q, scales


def bf16_gemv(W, x, y=None, stream=None):
    """One-row bf16 projection: W bf16 [N, K], x bf16 [T, K] (T <= 4) ->
    y bf16 [T, N] = bf16(fp32(exact sum of products))."""
    import torch
    N, K = W.shape
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _check("moe_bf16_gemv", lib().moe_bf16_gemv(_ptr(W), N, K, _ptr(x), T, _ptr(y),
                                                _stream(stream)))
    return y


def quant_act(x, q=None, scales=None, stream=None):
    """x bf16 [T, C] -> (q uint8 [T, C] e4m3 codes, scales fp32 [T, C/128])."""
    import torch
    T, C = x.shape
    if q is None:
        q = torch.empty((T, C), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((T, C // 128), dtype=torch.float32, device=x.device)
    _check("moe_quant_act", lib().moe_quant_act(_ptr(x), T, C, _ptr(q), _ptr(scales),
                                                _stream(stream)))
    return q, scales


def route(cfg: Config, x, router_w, router_bias=None, ids=None, weights=None, logits=None,
          workspace=None, stream=None):
    """-> (ids int32 [T,K], weights fp32 [T,K], logits fp32 [T,E] or None)."""
    import torch
    T = x.shape[0]
    if ids is None:
        ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((T, cfg.top_k), dtype=torch.float32, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check("moe_route", lib().moe_route(
        ctypes.byref(cfg), _ptr(x), T, _ptr(router_w), _ptr(router_bias), _ptr(ids),
        _ptr(weights), _ptr(logits), _ptr(workspace), ws_bytes, _stream(stream)))
    return ids, weights, logits


def weights_struct(lw) -> Weights:
    """Weights struct from an object with the tensor attributes of
    inputs.LayerWeights (all on the device)."""
    return Weights(**{k: _ptr(getattr(lw, k, None)) for k, _ in Weights._fields_})


def e4m3_encode(x, q=None, stream=None):
    """The kernels' fp32 -> e4m3 conversion of fp32 tensor x (any shape):
    uint8 codes of the same shape."""
    import torch
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check("moe_e4m3_encode", lib().moe_e4m3_encode(_ptr(x), x.numel(), _ptr(q), _stream(stream)))
    return q


def decode_status(workspace, clear: bool = False, stream=None) -> int:
    """The decode path's spin-out word of `workspace` (0: every bounded wait
    was met), read on `stream` after the work enqueued there; with clear,
    also zeroes it."""
    import torch
    out = torch.zeros(1, dtype=torch.int32, device=workspace.device)
    _check("moe_decode_status", lib().moe_decode_status(_ptr(workspace), _ptr(out),
                                                         int(bool(clear)), _stream(stream)))
    if stream is not None:
        stream.synchronize()
    else:
        torch.cuda.synchronize(workspace.device)
    return int(out.item())


NOALLOC_WORKSPACE_BYTES = 32 << 20  # MOE_NOALLOC_WORKSPACE_BYTES


def forward_noalloc(cfg: Config, lw, x, y, stream=None, wstruct=None):
    """Whole layer through moe_forward_noalloc (the library's own workspace):
    y bf16 [T, H], allocated by the caller."""
    T = x.shape[0]
    ws = wstruct if wstruct is not None else weights_struct(lw)
    _check("moe_forward_noalloc", lib().moe_forward_noalloc(
        ctypes.byref(cfg), ctypes.byref(ws), _ptr(x), T, _ptr(y), _stream(stream)))
    return y


def forward(cfg: Config, lw, x, y=None, workspace=None, stream=None, wstruct=None):
    """Whole layer: y bf16 [T, H]."""
    import torch
    T = x.shape[0]
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(cfg, max(T, 1), x.device)
    ws = wstruct if wstruct is not None else weights_struct(lw)
    _check("moe_forward", lib().moe_forward(
        ctypes.byref(cfg), ctypes.byref(ws), _ptr(x), T, _ptr(y), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return y
