"""Shared helpers of the GPU parity tests (imported by tests only)."""
from __future__ import annotations

import dataclasses
import functools
import sys

import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
import oracle
from block_fp8_mixture_router_amd import inputs
from tests import exact

# Output tolerance: relative L2 of the bf16 layer output against the oracle's
# fp32 value before rounding. The benchmark spec's bound for this layer is 1e-2; the
# expected value is about 2e-3 (bf16 output rounding ~1.7e-3 plus summation
# order); skipping the activation quantisation would cost ~3e-2 to 4e-2.
OUT_TOL = 1e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not moe.supported(torch.cuda.current_device()):
        pytest.fail("the GPU is not gfx950 or libmoe cannot see it")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def layer(shape_name: str, seed: int = 0, skewed: bool = False):
    """A synthetic layer generated on the GPU, with a host copy for the oracle."""
    shape = getattr(inputs, shape_name)
    dev = inputs.make_layer(shape, seed=seed, device="cuda", skewed=skewed)
    torch.cuda.synchronize()
    host = dev.to("cpu")
    return shape, dev, host


def x_rows(shape, T, seed=0):
    x = inputs.make_x(shape, T, seed=seed, device="cuda")
    return x, x.cpu()


def rel_rows(y_gpu_bits, acc):
    yg = exact.bits_to_f32(y_gpu_bits).astype(np.float64)
    a = acc.astype(np.float64)
    num = np.linalg.norm(yg - a, axis=1)
    den = np.maximum(np.linalg.norm(a, axis=1), 1e-30)
    return exact.rel_l2(yg, a), float((num / den).max())


def run_forward(shape, lw_dev, x_dev, flags=0, shared=True, workspace=None, poison=False):
    cfg = moe.config(shape, flags, shared)
    T = x_dev.shape[0]
    if workspace is None:
        workspace = moe.alloc_workspace(cfg, max(T, 1))
    if poison:
        workspace.view(torch.uint8).fill_(0xFF)
    y = torch.full_like(x_dev, float("nan")) if poison else torch.empty_like(x_dev)
    moe.forward(cfg, lw_dev, x_dev, y=y, workspace=workspace)
    torch.cuda.synchronize()
    return y


def bits(t):
    return exact.bf16_bits(t)
