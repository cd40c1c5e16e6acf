"""The no-activation-quantisation control (MOE_NO_ACT_QUANT) on the GPU
against the oracle's matching mode, which multiplies unquantised x and h
by the decoded e4m3 weights; the control's h goes to the down product in
bf16, inside the output tolerance. The one-row kernel gives the bits of the
expert-grouped kernels."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
from block_fp8_mixture_router_amd import inputs
import oracle
from tests.gpu_common import OUT_TOL, bits, layer, need_gpu, rel_rows, run_forward, say, x_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _rel(shape, host, xh, y, flags, rows=None, shared=True):
    xs = xh if rows is None else xh[rows]
    yb = bits(y.cpu())
    if rows is not None:
        yb = yb[rows]
    _, acc, _, _ = oracle.forward(shape, host, xs, flags=flags, shared=shared)
    return rel_rows(yb, acc)


@pytest.mark.parametrize("shape_name,T,shared", [
    ("TINY", 1, True), ("TINY", 5, True), ("TINY", 70, True), ("TINY", 9, False),
    ("DECODE", 1, True), ("DECODE", 37, True), ("DECODE", 5, False),
])
def test_control_matches_oracle_mode(shape_name, T, shared):
    say(f"no-act-quant {shape_name} T={T} shared={shared}")
    shape, dev, host = layer(shape_name, 0)
    x, xh = x_rows(shape, T, seed=300 + T)
    yn = run_forward(shape, dev, x, moe.NO_ACT_QUANT, shared=shared)
    yq = run_forward(shape, dev, x, 0, shared=shared)
    rel_n, worst_n = _rel(shape, host, xh, yn, oracle.NO_ACT_QUANT, shared=shared)
    rel_q, _ = _rel(shape, host, xh, yq, oracle.NO_ACT_QUANT, shared=shared)
    say(f"  control vs its oracle {rel_n:.2e} (worst row {worst_n:.2e}); "
        f"quantised layer vs the same oracle {rel_q:.2e}")
    assert rel_n <= OUT_TOL, (rel_n, worst_n)
    assert worst_n <= OUT_TOL, (rel_n, worst_n)  # each row on its own
    # the switch takes effect: the quantised layer sits further from this mode
    assert rel_n < 0.5 * rel_q, (rel_n, rel_q)


@pytest.mark.parametrize("skewed", [False, True])
def test_control_full_chunk_sampled_rows(skewed):
    say(f"no-act-quant chunk T=1024 skewed={skewed}")
    shape, dev, host = layer("DECODE", 0, skewed)
    T = 1024
    x, xh = x_rows(shape, T, seed=77 + skewed)
    y = run_forward(shape, dev, x, moe.NO_ACT_QUANT)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(T - 4, T),
                                     np.random.default_rng(5).choice(T, 40, replace=False)]))
    rel, worst = _rel(shape, host, xh, y, oracle.NO_ACT_QUANT, rows=rows)
    say(f"  relL2 {rel:.2e} worst row {worst:.2e}")
    assert rel <= OUT_TOL, (rel, worst)
    assert worst <= OUT_TOL, (rel, worst)  # each row on its own


def test_control_is_deterministic_and_poison_proof():
    shape, dev, _ = layer("DECODE", 0)
    x, _ = x_rows(shape, 64, seed=9)
    a = run_forward(shape, dev, x, moe.NO_ACT_QUANT)
    b = run_forward(shape, dev, x, moe.NO_ACT_QUANT, poison=True)
    assert np.array_equal(bits(a.cpu()), bits(b.cpu()))


ONE_ROW_SHAPES = {
    "TINY": inputs.TINY,
    "DECODE": inputs.DECODE,
    "ODD": inputs.LayerShape(hidden=384, n_experts=12, top_k=3, inter=384, shared_inter=384),
    "K12": inputs.LayerShape(hidden=256, n_experts=32, top_k=12, inter=128, shared_inter=128),
    "H4096": inputs.LayerShape(hidden=4096, n_experts=16, top_k=2, inter=256, shared_inter=256),
}


@pytest.mark.parametrize("name,T,shared", [
    ("TINY", 1, True), ("TINY", 4, True), ("TINY", 2, False), ("DECODE", 1, True),
    ("DECODE", 3, True), ("DECODE", 1, False), ("ODD", 2, True), ("K12", 1, True),
    ("H4096", 2, True),
])
def test_control_one_row_kernel(name, T, shared):
    """The control on the one-row kernel: within its oracle mode's tolerance,
    and bit for bit the expert-grouped control kernels' output."""
    say(f"no-act-quant one-row kernel {name} T={T} shared={shared}")
    shape = ONE_ROW_SHAPES[name]
    dev = inputs.make_layer(shape, seed=5, device="cuda")
    torch.cuda.synchronize()
    host = dev.to("cpu")
    x, xh = x_rows(shape, T, seed=700 + T)
    yd = run_forward(shape, dev, x, moe.NO_ACT_QUANT | moe.FORCE_GEMV, shared=shared)
    yg = run_forward(shape, dev, x, moe.NO_ACT_QUANT | moe.FORCE_GROUPED, shared=shared)
    rel, worst = _rel(shape, host, xh, yd, oracle.NO_ACT_QUANT, shared=shared)
    say(f"  relL2 {rel:.2e} worst row {worst:.2e}")
    assert rel <= OUT_TOL, (rel, worst)
    assert worst <= OUT_TOL, (rel, worst)  # each row on its own
    assert np.array_equal(bits(yd.cpu()), bits(yg.cpu()))


def test_control_one_row_default_and_poison_proof():
    shape, dev, _ = layer("DECODE", 0)
    x, _ = x_rows(shape, 2, seed=19)
    a = run_forward(shape, dev, x, moe.NO_ACT_QUANT | moe.FORCE_GEMV)
    b = run_forward(shape, dev, x, moe.NO_ACT_QUANT, poison=True)
    assert np.array_equal(bits(a.cpu()), bits(b.cpu()))
