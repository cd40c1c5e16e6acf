"""moe_forward on several streams at once (each with its own workspace) and
inside captured graphs: every result equals the same call made alone."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
from block_fp8_mixture_router_amd import inputs
from tests.gpu_common import bits, layer, need_gpu, say, x_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _alone(shape, lw, x, cfg):
    ws = moe.alloc_workspace(cfg, x.shape[0])
    y = moe.forward(cfg, lw, x, workspace=ws)
    torch.cuda.synchronize()
    return bits(y.cpu())


def test_two_streams_two_workspaces():
    shape, dev0, _ = layer("DECODE", 0)
    dev1 = inputs.make_layer(shape, seed=0, layer=1, device="cuda")
    cfg = moe.config(shape)
    xd, _ = x_rows(shape, 6, seed=21)    # six decode rows, one call each
    xc, _ = x_rows(shape, 300, seed=22)  # one grouped call
    want_d = [_alone(shape, dev0, xd[i:i + 1].contiguous(), cfg) for i in range(6)]
    want_c = _alone(shape, dev1, xc, cfg)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    wa, wb = moe.alloc_workspace(cfg, 1), moe.alloc_workspace(cfg, 300)
    ya = [torch.empty(1, shape.hidden, dtype=torch.bfloat16, device="cuda") for _ in range(6)]
    yb = torch.empty_like(xc)
    torch.cuda.synchronize()
    for rep in range(3):
        for i in range(6):
            moe.forward(cfg, dev0, xd[i:i + 1], y=ya[i], workspace=wa, stream=sa)
            if i == 2:
                moe.forward(cfg, dev1, xc, y=yb, workspace=wb, stream=sb)
        torch.cuda.synchronize()
        for i in range(6):
            assert np.array_equal(bits(ya[i].cpu()), want_d[i]), (rep, i)
        assert np.array_equal(bits(yb.cpu()), want_c), rep
    say("  two streams: every call equals its lone run")


@pytest.mark.parametrize("T", [1, 300])
def test_forward_graph_replays(T):
    shape, dev, _ = layer("DECODE", 0)
    cfg = moe.config(shape)
    xs = [x_rows(shape, T, seed=30 + k)[0] for k in range(3)]
    want = [_alone(shape, dev, x, cfg) for x in xs]
    ws = moe.alloc_workspace(cfg, T)
    ys = [torch.empty_like(x) for x in xs]
    wsr = moe.weights_struct(dev)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        for x, y in zip(xs, ys):
            moe.forward(cfg, dev, x, y=y, workspace=ws, wstruct=wsr, stream=st)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=st):
        for x, y in zip(xs, ys):
            moe.forward(cfg, dev, x, y=y, workspace=ws, wstruct=wsr, stream=st)
    for rep in range(3):
        for y in ys:
            y.fill_(0)
        # eager work between replays, on the same workspace
        moe.forward(cfg, dev, xs[rep], y=torch.empty_like(xs[rep]), workspace=ws)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for k, y in enumerate(ys):
            assert np.array_equal(bits(y.cpu()), want[k]), (rep, k)
    say(f"  T={T}: three replays equal the eager calls")
