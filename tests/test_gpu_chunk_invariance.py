"""Chunk invariance: a row's output bytes do not depend on
the other rows it is computed with. On the expert-grouped kernels every
per-row result is a function of that row alone, so row t of a 1024-row
chunk equals, byte for byte, the same row run alone through the grouped
path (MOE_FORCE_GROUPED at T = 1). The one-row decode path is a different
arithmetic (vector GEMV sums) and only agrees within the output tolerance."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
from block_fp8_mixture_router_amd import inputs
from tests.gpu_common import bits, layer, need_gpu, run_forward, say, x_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("skewed", [False, True])
def test_row_bytes_equal_alone_and_in_a_chunk(skewed):
    shape, dev, _ = layer("DECODE", 0, skewed)
    T = 1024
    x, _ = x_rows(shape, T, seed=41 + skewed)
    yc = bits(run_forward(shape, dev, x).cpu())
    rows = sorted(set([0, 1, 63, 64, 65, 127, 128, 511, 512, 777, 1023] +
                      list(np.random.default_rng(7).choice(T, 21, replace=False))))
    cfg = moe.config(shape, moe.FORCE_GROUPED)
    ws = moe.alloc_workspace(cfg, 1)
    bad = []
    for t in rows:
        y1 = bits(run_forward(shape, dev, x[t:t + 1].contiguous(), moe.FORCE_GROUPED,
                              workspace=ws).cpu())
        if not np.array_equal(y1[0], yc[t]):
            bad.append((t, int((y1[0] != yc[t]).sum())))
    say(f"  rows checked {len(rows)}, differing {bad}")
    assert not bad


def test_decode_path_agrees_within_tolerance():
    shape, dev, _ = layer("DECODE", 0)
    x, _ = x_rows(shape, 64, seed=43)
    yc = run_forward(shape, dev, x).float().cpu()
    worst = 0.0
    for t in (0, 17, 63):
        y1 = run_forward(shape, dev, x[t:t + 1].contiguous()).float().cpu()[0]
        rel = float((y1 - yc[t]).norm() / yc[t].norm())
        worst = max(worst, rel)
    say(f"  decode path vs chunk row, worst relL2 {worst:.2e}")
    assert worst < 1e-2
