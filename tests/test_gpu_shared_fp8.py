"""The block-FP8 shared-expert variant (MOE_SHARED_FP8) on the GPU against
the oracle's matching mode: the shared matrices stored block-FP8 run through
the routed kernels as one expert holding every row, gamma as its weight."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
import oracle
from block_fp8_mixture_router_amd import inputs
from tests.gpu_common import OUT_TOL, bits, need_gpu, rel_rows, run_forward, say, x_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _layer(shape_name, seed=0, skewed=False):
    shape = getattr(inputs, shape_name)
    dev = inputs.make_layer(shape, seed=seed, device="cuda", skewed=skewed, shared_fp8=True)
    torch.cuda.synchronize()
    return shape, dev, dev.to("cpu")


def _rel(shape, host, xh, y, rows=None):
    xs = xh if rows is None else xh[rows]
    yb = bits(y.cpu())
    if rows is not None:
        yb = yb[rows]
    _, acc, _, _ = oracle.forward(shape, host, xs, flags=oracle.SHARED_FP8)
    return rel_rows(yb, acc)


@pytest.mark.parametrize("shape_name,T", [
    ("TINY", 1), ("TINY", 5), ("TINY", 70), ("DECODE", 1), ("DECODE", 4), ("DECODE", 37),
])
def test_shared_fp8_matches_oracle_mode(shape_name, T):
    say(f"shared-fp8 {shape_name} T={T}")
    shape, dev, host = _layer(shape_name)
    x, xh = x_rows(shape, T, seed=500 + T)
    y = run_forward(shape, dev, x, moe.SHARED_FP8)
    rel, worst = _rel(shape, host, xh, y)
    say(f"  relL2 {rel:.2e} worst row {worst:.2e}")
    assert rel <= OUT_TOL, (rel, worst)


@pytest.mark.parametrize("skewed", [False, True])
def test_shared_fp8_full_chunk_sampled_rows(skewed):
    say(f"shared-fp8 chunk T=1024 skewed={skewed}")
    shape, dev, host = _layer("DECODE", 0, skewed)
    T = 1024
    x, xh = x_rows(shape, T, seed=91 + skewed)
    y = run_forward(shape, dev, x, moe.SHARED_FP8)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(T - 4, T),
                                     np.random.default_rng(6).choice(T, 40, replace=False)]))
    rel, worst = _rel(shape, host, xh, y, rows=rows)
    say(f"  relL2 {rel:.2e} worst row {worst:.2e}")
    assert rel <= OUT_TOL, (rel, worst)


def test_shared_fp8_deterministic_and_poison_proof():
    shape, dev, _ = _layer("DECODE", 0)
    x, _ = x_rows(shape, 100, seed=12)
    a = run_forward(shape, dev, x, moe.SHARED_FP8)
    b = run_forward(shape, dev, x, moe.SHARED_FP8, poison=True)
    assert np.array_equal(bits(a.cpu()), bits(b.cpu()))


def test_shared_fp8_zero_down_equals_no_shared():
    """All-zero FP8 shared down codes: the output is the routed sum alone,
    bit for bit that of the same layer run without a shared expert."""
    shape, dev, _ = _layer("DECODE", 0)
    dev.sh_down = torch.zeros_like(dev.sh_down)
    x, _ = x_rows(shape, 40, seed=13)
    a = run_forward(shape, dev, x, moe.SHARED_FP8)
    b = run_forward(shape, dev, x, moe.FORCE_GROUPED, shared=False)
    assert np.array_equal(bits(a.cpu()), bits(b.cpu()))
