"""moe_forward_noalloc (the library's own 32 MiB workspace array) against
moe_forward with a caller-owned workspace: the same bytes on consecutive
calls, the second with fewer rows, across a change of config and back."""
import ctypes

import pytest
import torch

import block_fp8_mixture_router_amd as moe
from block_fp8_mixture_router_amd import inputs

pytestmark = pytest.mark.gpu


def _same(cfg, lw, ws, x):
    y = torch.empty_like(x)
    moe.forward_noalloc(cfg, lw, x, y, wstruct=ws)
    ref = moe.forward(cfg, lw, x, wstruct=ws)
    torch.cuda.synchronize()
    return torch.equal(y.view(torch.int16), ref.view(torch.int16))


def test_noalloc_matches_forward():
    torch.cuda.set_device(0)
    shape = inputs.DECODE
    cfg = moe.config(shape)
    lw = inputs.make_layer(shape, seed=3, layer=0, device="cuda")
    ws = moe.weights_struct(lw)
    print("noalloc: decode shape, 96 rows then 1, 1, 4", flush=True)
    # the expert-grouped path, then the one-row path with fewer rows (twice,
    # so the one-row path's call counters carry over between calls), then
    # the one-row path with a few rows
    for T, seed in ((96, 11), (1, 12), (1, 13), (4, 14)):
        x = inputs.make_x(shape, T, seed=seed, device="cuda")
        assert _same(cfg, lw, ws, x), T
    # another config on the same device clears the array first; then back
    print("noalloc: tiny shape, 3 rows, then decode shape, 2 rows", flush=True)
    tiny = inputs.TINY
    ct = moe.config(tiny)
    lt = inputs.make_layer(tiny, seed=4, layer=0, device="cuda")
    assert _same(ct, lt, moe.weights_struct(lt), inputs.make_x(tiny, 3, seed=5, device="cuda"))
    assert _same(cfg, lw, ws, inputs.make_x(shape, 2, seed=15, device="cuda"))


def test_noalloc_refuses_rows_beyond_its_array():
    torch.cuda.set_device(0)
    shape = inputs.DECODE
    cfg = moe.config(shape)
    lw = inputs.make_layer(shape, seed=3, layer=0, device="cuda")
    ws = moe.weights_struct(lw)
    T = 640
    assert moe.workspace_bytes(cfg, T) > moe.NOALLOC_WORKSPACE_BYTES
    x = inputs.make_x(shape, T, seed=16, device="cuda")
    y = torch.zeros_like(x)
    st = moe.lib().moe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(ws), x.data_ptr(), T,
                                       y.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == -4
    assert int(y.view(torch.int16).abs().sum()) == 0  # nothing was enqueued
