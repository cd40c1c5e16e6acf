"""GPU parity of moe_forward against the oracle, on both paths, plus the
layer's invariants on the GPU (determinism, poisoned scratch, row order,
identical experts, closed shared gate)."""
import dataclasses

import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
import oracle
from block_fp8_mixture_router_amd import inputs
from tests import exact
from tests.gpu_common import OUT_TOL, bits, layer, need_gpu, rel_rows, run_forward, say, x_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _check(shape, host, x_host, y_dev, rows=None, tol=OUT_TOL, flags=0, shared=True):
    xs = x_host if rows is None else x_host[rows]
    yb = bits(y_dev.cpu())
    if rows is not None:
        yb = yb[rows]
    _, acc, _, _ = oracle.forward(shape, host, xs, flags=flags, shared=shared)
    rel, worst = rel_rows(yb, acc)
    say(f"  relL2 {rel:.2e}  worst row {worst:.2e}")
    assert np.all(np.isfinite(exact.bits_to_f32(yb)))
    assert rel <= tol, (rel, worst)
    assert worst <= tol, (rel, worst)  # every row on its own, not only the whole
    return rel, worst


CASES = [
    # (shape, T, flags, skewed)
    ("TINY", 1, 0, False),
    ("TINY", 3, 0, False),
    ("TINY", 5, 0, False),
    ("TINY", 70, 0, False),
    ("TINY", 1, moe.FORCE_GROUPED, False),
    ("TINY", 4, moe.FORCE_GEMV, False),
    ("DECODE", 1, 0, False),
    ("DECODE", 2, 0, False),
    ("DECODE", 4, 0, False),
    ("DECODE", 1, moe.FORCE_GROUPED, False),
    ("DECODE", 3, moe.FORCE_GEMV, False),
    ("DECODE", 37, 0, False),
]


@pytest.mark.parametrize("shape_name,T,flags,skewed", CASES)
def test_forward_matches_oracle(shape_name, T, flags, skewed):
    say(f"forward {shape_name} T={T} flags={flags} skewed={skewed}")
    shape, dev, host = layer(shape_name, 0, skewed)
    x, xh = x_rows(shape, T, seed=100 + T)
    y = run_forward(shape, dev, x, flags)
    _check(shape, host, xh, y)


@pytest.mark.parametrize("skewed", [False, True])
@pytest.mark.parametrize("T", [1023, 1024])
def test_forward_chunk_sampled_rows(T, skewed):
    """Full chunk sizes in the launch configuration the bench times; the
    oracle checks a sample of rows (rows are independent)."""
    say(f"forward chunk T={T} skewed={skewed}")
    shape, dev, host = layer("DECODE", 0, skewed)
    x, xh = x_rows(shape, T, seed=T + skewed)
    y = run_forward(shape, dev, x)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(T - 8, T),
                                     np.random.default_rng(T).choice(T, 48, replace=False)]))
    _check(shape, host, xh, y, rows=rows)


def test_forward_deterministic_and_poison_proof():
    shape, dev, host = layer("DECODE", 0, False)
    for T, flags in ((1, 0), (300, 0), (3, moe.FORCE_GROUPED)):
        say(f"determinism T={T} flags={flags}")
        x, _ = x_rows(shape, T, seed=5)
        y1 = run_forward(shape, dev, x, flags)
        ws = moe.alloc_workspace(moe.config(shape, flags), T)
        ws.fill_(0xFF)
        moe.decode_status(ws, clear=True)  # zero the decode kernel's spin-out word
        y2 = run_forward(shape, dev, x, flags, workspace=ws)
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        y3 = run_forward(shape, dev, x, flags, workspace=ws)
        assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
        assert moe.decode_status(ws) == 0


def test_workspace_fills_and_path_mixing():
    """A workspace filled with any one repeated byte serves the decode path,
    and decode and grouped calls can alternate on one workspace."""
    shape, dev, host = layer("DECODE", 0, False)
    x1, _ = x_rows(shape, 1, seed=21)
    x3, _ = x_rows(shape, 300, seed=22)
    ref1, ref3 = run_forward(shape, dev, x1), run_forward(shape, dev, x3)
    cfg = moe.config(shape)
    for fill in (0x00, 0x01, 0x3F, 0xA5, 0xFF):
        say(f"workspace fill {fill:#04x}")
        ws = moe.alloc_workspace(cfg, 300)
        ws.fill_(fill)
        moe.decode_status(ws, clear=True)  # zero the decode kernel's spin-out word
        for xx, ref in ((x1, ref1), (x3, ref3), (x1, ref1), (x1, ref1), (x3, ref3), (x1, ref1)):
            y = run_forward(shape, dev, xx, workspace=ws)
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
        assert moe.decode_status(ws) == 0


def test_grouped_rows_independent_of_order():
    shape, dev, host = layer("DECODE", 0, False)
    x, _ = x_rows(shape, 200, seed=6)
    y = run_forward(shape, dev, x)
    p = torch.randperm(200, generator=torch.Generator().manual_seed(0)).cuda()
    yp = run_forward(shape, dev, x[p].contiguous())
    assert torch.equal(y[p].view(torch.int16), yp.view(torch.int16))
    # a row alone through the grouped path gives the same bytes as in the chunk
    y1 = run_forward(shape, dev, x[17:18].contiguous(), moe.FORCE_GROUPED)
    assert torch.equal(y[17:18].view(torch.int16), y1.view(torch.int16))


def test_all_rows_on_the_same_experts():
    """A bias that sends every row to experts 0..7: 16 full tiles per expert."""
    shape, dev, host = layer("DECODE", 0, False)
    bias = torch.zeros(shape.n_experts)
    bias[:8] = 64.0
    dev_b = dataclasses.replace(dev, router_bias=bias.cuda())
    host_b = dataclasses.replace(host, router_bias=bias)
    x, xh = x_rows(shape, 1024, seed=7)
    y = run_forward(shape, dev_b, x)
    rows = np.arange(0, 1024, 16)
    _check(shape, host_b, xh, y, rows=rows)


def test_single_expert_layer():
    shape = dataclasses.replace(inputs.TINY, n_experts=1, top_k=1)
    dev = inputs.make_layer(shape, seed=3, device="cuda")
    host = dev.to("cpu")
    for T in (1, 40):
        x, xh = x_rows(shape, T, seed=3)
        y = run_forward(shape, dev, x)
        _check(shape, host, xh, y)


def test_identical_experts_on_gpu():
    shape, _, _ = layer("TINY", 0, False)
    dev = inputs.make_layer(shape, seed=4, device="cuda")
    for name in ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down"):
        t = getattr(dev, name)
        t[:] = t[5:6].clone()
    host = dev.to("cpu")
    one = dataclasses.replace(shape, n_experts=1, top_k=1)
    dev1 = dataclasses.replace(dev, shape=one, router_w=dev.router_w[5:6].contiguous())
    for name in ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down"):
        setattr(dev1, name, getattr(dev, name)[5:6].contiguous())
    for T in (2, 50):
        x, xh = x_rows(shape, T, seed=4)
        y = run_forward(shape, dev, x)
        y1 = run_forward(one, dev1, x)
        d = exact.rel_l2(y.float().cpu().numpy(), y1.float().cpu().numpy())
        say(f"  identical experts T={T}: relL2 vs single expert {d:.2e}")
        assert d <= 1e-2
        _check(shape, host, xh, y)


def test_closed_shared_gate_removes_shared_branch():
    shape, dev, host = layer("TINY", 0, False)
    x, xh = x_rows(shape, 1, seed=9)
    gw = (-0.125 * torch.sign(x[0].float())).to(torch.bfloat16)
    dev_g = dataclasses.replace(dev, sh_gate_w=gw)
    for flags in (0, moe.FORCE_GROUPED):
        y = run_forward(shape, dev_g, x, flags)
        y0 = run_forward(shape, dev, x, flags, shared=False)
        assert torch.equal(y.float(), y0.float())


def test_no_shared_expert_matches_oracle():
    shape, dev, host = layer("DECODE", 0, False)
    for T in (1, 64):
        x, xh = x_rows(shape, T, seed=10)
        y = run_forward(shape, dev, x, shared=False)
        _check(shape, host, xh, y, shared=False)


@pytest.mark.parametrize("T", [2048, 2500])
def test_forward_sort_capacity_edges(T):
    """Chunks at and past the one-pass sort's capacity (16,384 pairs: T = 2048
    at top-8; T = 2500 takes the segmented sort): sampled rows against the
    oracle, and the first 300 rows bit-identical to the same rows run as a
    chunk of their own (rows are independent of the sort that placed them)."""
    say(f"forward sort capacity T={T}")
    shape, dev, host = layer("DECODE", 0, False)
    x, xh = x_rows(shape, T, seed=T)
    y = run_forward(shape, dev, x)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(T - 4, T),
                                     np.random.default_rng(T).choice(T, 24, replace=False)]))
    _check(shape, host, xh, y, rows=rows)
    y300 = run_forward(shape, dev, x[:300].contiguous())
    assert torch.equal(y[:300].view(torch.int16), y300.view(torch.int16))


def test_force_gemv_beyond_four_rows_is_refused():
    """The one-row path takes at most four rows; forcing it on five is
    refused before anything is enqueued."""
    shape, dev, _ = layer("DECODE", 0, False)
    x, _ = x_rows(shape, 5, seed=9)
    with pytest.raises(moe.MoeError, match="UNSUPPORTED"):
        run_forward(shape, dev, x, moe.FORCE_GEMV)


def test_workspace_regions_do_not_move_with_rows():
    """Grouped calls at few rows and one-row calls share a fresh zero-filled
    workspace: a grouped call's plain data never lands where a later one-row
    call polls for tagged words, so every output equals its lone call's."""
    shape, dev, _ = layer("DECODE", 0, False)
    cfg = moe.config(shape)
    sequences = [
        [(1, moe.FORCE_GROUPED), (4, 0)],
        [(5, 0), (4, moe.FORCE_GEMV)],
        [(2, moe.FORCE_GROUPED), (3, 0), (1, 0), (16, 0), (2, 0)],
    ]
    for seq in sequences:
        say(f"workspace sequence {seq}")
        ws = moe.alloc_workspace(cfg, max(T for T, _ in seq))
        for i, (T, flags) in enumerate(seq):
            x, _ = x_rows(shape, T, seed=60 + i)
            want = run_forward(shape, dev, x, flags)
            got = run_forward(shape, dev, x, flags, workspace=ws)
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (seq, i)
        assert moe.decode_status(ws) == 0


def test_decode_status_reads_and_clears():
    """moe_decode_status returns the spin-out word as it stands and zeroes it
    on request (the word is set here from the host, as a spin-out would)."""
    shape, dev, host = layer("DECODE", 0, False)
    cfg = moe.config(shape)
    ws = moe.alloc_workspace(cfg, 1)
    ws.zero_()
    x, _ = x_rows(shape, 1, seed=31)
    run_forward(shape, dev, x, workspace=ws)
    assert moe.decode_status(ws) == 0
    ws[128:132].view(torch.int32).fill_(7)
    assert moe.decode_status(ws) == 7
    assert moe.decode_status(ws, clear=True) == 7
    assert moe.decode_status(ws) == 0
    y = run_forward(shape, dev, x, workspace=ws)
    assert torch.equal(y.view(torch.int16), run_forward(shape, dev, x).view(torch.int16))
    assert moe.decode_status(ws) == 0
