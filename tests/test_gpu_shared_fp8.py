"""The block-FP8 shared-expert variant (MOE_SHARED_FP8) on the GPU against
the oracle's matching mode: the shared matrices stored block-FP8 run through
the routed kernels as one expert holding every row, gamma as its weight. The
one-row kernel runs them as one more slot of every row, with the same bits."""
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
    assert worst <= OUT_TOL, (rel, worst)  # each row on its own


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
    assert worst <= OUT_TOL, (rel, worst)  # each row on its own


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


def _shape_layer(shape, seed=4):
    dev = inputs.make_layer(shape, seed=seed, device="cuda", shared_fp8=True)
    torch.cuda.synchronize()
    return dev, dev.to("cpu")


# the decode shape, the small one, odd block counts (three 128-blocks), more
# than eight slots (two phase-C tiles per wave), and H > 2048 (gate/up
# batches past the first, four router chunks per lane)
ONE_ROW_SHAPES = {
    "TINY": inputs.TINY,
    "DECODE": inputs.DECODE,
    "ODD": inputs.LayerShape(hidden=384, n_experts=12, top_k=3, inter=384, shared_inter=384),
    "K12": inputs.LayerShape(hidden=256, n_experts=32, top_k=12, inter=128, shared_inter=128),
    "H4096": inputs.LayerShape(hidden=4096, n_experts=16, top_k=2, inter=256, shared_inter=256),
}


@pytest.mark.parametrize("name,T", [
    ("TINY", 1), ("TINY", 3), ("DECODE", 1), ("DECODE", 2), ("DECODE", 4), ("ODD", 1),
    ("ODD", 4), ("K12", 2), ("H4096", 1), ("H4096", 3),
])
def test_shared_fp8_one_row_kernel(name, T):
    """The one-row kernel with the block-FP8 shared expert as slot K: within
    the oracle mode's tolerance, and bit for bit the expert-grouped kernels'
    output for the same rows."""
    say(f"shared-fp8 one-row kernel {name} T={T}")
    shape = ONE_ROW_SHAPES[name]
    dev, host = _shape_layer(shape)
    x, xh = x_rows(shape, T, seed=600 + T)
    yd = run_forward(shape, dev, x, moe.SHARED_FP8 | moe.FORCE_GEMV)
    yg = run_forward(shape, dev, x, moe.SHARED_FP8 | moe.FORCE_GROUPED)
    rel, worst = _rel(shape, host, xh, yd)
    say(f"  relL2 {rel:.2e} worst row {worst:.2e}")
    assert rel <= OUT_TOL, (rel, worst)
    assert worst <= OUT_TOL, (rel, worst)  # each row on its own
    assert np.array_equal(bits(yd.cpu()), bits(yg.cpu()))


def test_shared_fp8_one_row_is_the_default_and_poison_proof():
    """T = 1 without a path flag takes the one-row kernel: the same bits as the
    forced one, on a workspace filled with 0xFF and on a reused one."""
    shape, dev, _ = _layer("DECODE", 0)
    x, _ = x_rows(shape, 1, seed=14)
    a = run_forward(shape, dev, x, moe.SHARED_FP8 | moe.FORCE_GEMV)
    b = run_forward(shape, dev, x, moe.SHARED_FP8, poison=True)
    cfg = moe.config(shape, moe.SHARED_FP8)
    ws = moe.alloc_workspace(cfg, 1)
    c = run_forward(shape, dev, x, moe.SHARED_FP8, workspace=ws)
    d = run_forward(shape, dev, x, moe.SHARED_FP8, workspace=ws)
    for o in (b, c, d):
        assert np.array_equal(bits(a.cpu()), bits(o.cpu()))


def test_shared_fp8_shared_width_unlike_routed():
    """Is != I: the shared expert cannot be a slot of the one-row kernel, so
    forcing that kernel is refused, and one row runs on the grouped kernels."""
    shape = inputs.LayerShape(hidden=256, n_experts=16, top_k=4, inter=128, shared_inter=256)
    dev, host = _shape_layer(shape)
    x, xh = x_rows(shape, 1, seed=17)
    with pytest.raises(moe.MoeError):
        run_forward(shape, dev, x, moe.SHARED_FP8 | moe.FORCE_GEMV)
    y = run_forward(shape, dev, x, moe.SHARED_FP8)
    rel, worst = _rel(shape, host, xh, y)
    assert rel <= OUT_TOL, (rel, worst)
    assert worst <= OUT_TOL, (rel, worst)  # each row on its own
