"""Chunk invariance: a row's output bytes do not depend on the other rows
it is computed with (PR #920 "drama: Drama 3 (fishaudio/drama-3)
text-to-speech on CUDA", Receipt: backbone outputs hash-identical at chunk
sizes 1, 7 and 128; PR #925, commit summary of the single-row projection:
the same matrix instructions on the same fragments in the same K order give
the same bits). Row t of a 1024-row chunk (the expert-grouped kernels) equals
byte for byte the same row run alone on the default path (the one-row
kernel), in groups of up to four rows on that kernel, and alone on the
grouped kernels."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
from tests.gpu_common import bits, layer, need_gpu, run_forward, say, x_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _rows(T):
    return sorted(set([0, 1, 63, 64, 65, 127, 128, 511, 512, 777, T - 1] +
                      list(np.random.default_rng(7).choice(T, 21, replace=False))))


@pytest.mark.parametrize("skewed", [False, True])
def test_row_bytes_equal_alone_and_in_a_chunk(skewed):
    shape, dev, _ = layer("DECODE", 0, skewed)
    T = 1024
    x, _ = x_rows(shape, T, seed=41 + skewed)
    yc = bits(run_forward(shape, dev, x).cpu())
    rows = _rows(T)
    ws_d = moe.alloc_workspace(moe.config(shape), 4)
    cfg_g = moe.config(shape, moe.FORCE_GROUPED)
    ws_g = moe.alloc_workspace(cfg_g, 1)
    bad_d, bad_g = [], []
    for t in rows:
        xt = x[t:t + 1].contiguous()
        yd = bits(run_forward(shape, dev, xt, workspace=ws_d).cpu())      # one-row kernel
        yg = bits(run_forward(shape, dev, xt, moe.FORCE_GROUPED, workspace=ws_g).cpu())
        if not np.array_equal(yd[0], yc[t]):
            bad_d.append((t, int((yd[0] != yc[t]).sum())))
        if not np.array_equal(yg[0], yc[t]):
            bad_g.append((t, int((yg[0] != yc[t]).sum())))
    # groups of 2, 3 and 4 rows through the one-row kernel
    for n in (2, 3, 4):
        for start in (0, 126, 509):
            yd = bits(run_forward(shape, dev, x[start:start + n].contiguous(),
                                  workspace=ws_d).cpu())
            for i in range(n):
                if not np.array_equal(yd[i], yc[start + i]):
                    bad_d.append((start + i, n, int((yd[i] != yc[start + i]).sum())))
    say(f"  rows checked {len(rows)}: one-row kernel differing {bad_d}, "
        f"grouped alone differing {bad_g}")
    assert not bad_d
    assert not bad_g
    assert moe.decode_status(ws_d) == 0


@pytest.mark.parametrize("shape_name", ["TINY", "DECODE"])
def test_one_row_kernel_equals_chunk_on_every_row(shape_name):
    """Every row of a 64-row chunk, one at a time on the one-row kernel."""
    shape, dev, _ = layer(shape_name, 0, False)
    T = 64
    x, _ = x_rows(shape, T, seed=43)
    yc = bits(run_forward(shape, dev, x).cpu())
    ws = moe.alloc_workspace(moe.config(shape), 1)
    bad = []
    for t in range(T):
        y1 = bits(run_forward(shape, dev, x[t:t + 1].contiguous(), workspace=ws).cpu())
        if not np.array_equal(y1[0], yc[t]):
            bad.append((t, int((y1[0] != yc[t]).sum())))
    say(f"  {shape_name}: rows differing {bad}")
    assert not bad
