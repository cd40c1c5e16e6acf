"""Both GPU paths on exact instances of the layer: bit-for-bit equality.

On these instances (tests/exact_instance.py) every product and sum the layer
forms is exact, so the FP8 MFMA grouped GEMMs, the fp32 GEMV of the decode
kernel, the fp64 router, the SwiGLU requantisation, the bf16 shared expert
and the combine must all give exactly the output computed in float64 (and
reproduced by the oracle), whatever their summation order. A wrong index,
scale or operand anywhere in the path changes bits here.

Rows are independent, so one instance of T_max rows serves every T: a call
with T rows runs on the first T rows of x.
"""
import dataclasses
import functools

import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
import oracle
from block_fp8_mixture_router_amd import inputs
from tests import exact_instance as xi
from tests.gpu_common import bits, need_gpu, run_forward, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


SHAPES = {
    "tiny": (inputs.TINY, 70, None),
    "tiny_one": (dataclasses.replace(inputs.TINY, n_experts=1, top_k=1), 40, None),
    "decode": (inputs.DECODE, 1024, np.unique(np.concatenate([
        np.arange(40), np.arange(1020, 1024),
        np.random.default_rng(0).choice(np.arange(40, 1020), 40, replace=False)]))),
    "decode_noshared": (dataclasses.replace(inputs.DECODE, shared_inter=0, n_experts=64), 40,
                        None),
    # activation scales 1, 2 and 4 across the groups (non-unit powers of two)
    "decode_act": (inputs.DECODE, 300, None),
}
ACT_SCALES = {"decode_act"}


@functools.lru_cache(maxsize=1)
def _instance(name):
    shape, T, rows = SHAPES[name]
    say(f"building exact instance {name} ({T} rows)")
    inst = xi.build(shape, T, seed=5, rows=rows, act_scales=name in ACT_SCALES)
    sel = np.arange(T) if rows is None else rows
    return shape, inst, inst.weights.to("cuda"), inst.x.cuda(), sel


def _check(name, T, flags=0):
    shape, inst, dev, x_all, sel = _instance(name)
    say(f"exact instance {name} T={T} flags={flags}")
    x = x_all[:T].contiguous()
    y = run_forward(shape, dev, x, flags)
    rows = sel[sel < T]
    yb = xi.zero_sign_blind(bits(y.cpu()))[rows]
    want = xi.zero_sign_blind(inst.y_bits)[rows]
    bad = np.argwhere(yb != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first (row idx, col) {bad[:4].tolist()}"
    # routing through the C ABI: ids exact, weights exactly 1/K
    cfg = moe.config(shape, flags)
    logits = torch.empty((T, shape.n_experts), dtype=torch.float32, device="cuda")
    ids, w, _ = moe.route(cfg, x, dev.router_w, None, logits=logits)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), inst.ids[:T])
    assert torch.all(w == 1.0 / shape.top_k)


@pytest.mark.parametrize("T,flags", [(1, 0), (3, 0), (5, 0), (70, 0), (1, moe.FORCE_GROUPED),
                                     (2, moe.FORCE_GEMV), (4, moe.FORCE_GEMV)])
def test_exact_tiny(T, flags):
    _check("tiny", T, flags)


@pytest.mark.parametrize("T,flags", [(1, 0), (2, 0), (4, 0), (1, moe.FORCE_GROUPED),
                                     (3, moe.FORCE_GEMV), (37, 0), (300, 0), (1023, 0),
                                     (1024, 0)])
def test_exact_decode_shape(T, flags):
    """Up to the 1024-row chunk in the launch configuration the bench times
    (exact expectations for 84 of its rows)."""
    _check("decode", T, flags)


@pytest.mark.parametrize("T,flags", [(1, 0), (4, 0), (1, moe.FORCE_GROUPED), (300, 0)])
def test_exact_decode_shape_activation_scales(T, flags):
    """Activation scales 1, 2 and 4 across the groups: every path takes each
    group's own scale."""
    _check("decode_act", T, flags)


@pytest.mark.parametrize("T", [1, 40])
def test_exact_single_expert(T):
    _check("tiny_one", T)


@pytest.mark.parametrize("T", [1, 3, 40])
def test_exact_no_shared_expert(T):
    _check("decode_noshared", T)


def test_exact_instance_matches_oracle_too():
    """The tiny instance through the oracle as well (ties the two checkers)."""
    shape, inst, _, _, _ = _instance("tiny")
    y, _, _, _ = oracle.forward(shape, inst.weights, inst.x)
    assert np.array_equal(xi.zero_sign_blind(y), xi.zero_sign_blind(inst.y_bits))
