"""The 40-layer decode stack on the GPU: the row renormalisation between
layers (bit-exact against the oracle); a chain of decode layers,
teacher-forced against the oracle layer by layer (each oracle layer gets the
GPU's input to that layer), eager and as a captured graph; and
moe_forward_stack, one launch per layer with the renormalisation folded into
each later layer's prologue, which must equal that chain bit for bit."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
import oracle
from block_fp8_mixture_router_amd import inputs
from tests import exact
from tests.gpu_common import OUT_TOL, bits, need_gpu, rel_rows, say

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _special_rows(H):
    rows = np.zeros((5, H), dtype=np.float32)
    rows[1, 7] = -3.0                       # one nonzero element
    rows[2] = 2.5                           # constant
    rows[3] = 2.0 ** -12                    # below eps
    rows[4] = np.linspace(-300, 300, H)     # wide range
    return torch.from_numpy(rows).to(torch.bfloat16)


@pytest.mark.parametrize("T,H", [(1, 2048), (5, 256), (64, 2048), (3, 8192), (1024, 2048),
                                 (2, 384), (3, 6144)])
def test_renorm_bit_exact(T, H):
    say(f"renorm T={T} H={H}")
    g = torch.Generator().manual_seed(T * H)
    y = (torch.randn(T, H, generator=g) * torch.rand(T, 1, generator=g) * 10).to(torch.bfloat16)
    y = torch.cat([y, _special_rows(H)])
    yd = y.cuda()
    x = moe.rms_renorm(yd, eps=EPS)
    torch.cuda.synchronize()
    want = oracle.rms_renorm(y, eps=EPS)
    assert np.array_equal(bits(x.cpu()), want)
    # in place
    moe.rms_renorm(yd, x=yd, eps=EPS)
    torch.cuda.synchronize()
    assert np.array_equal(bits(yd.cpu()), want)


def _chain(cfg, layers, wstructs, xs, ys, ws, stream):
    for l in range(len(layers)):
        moe.forward(cfg, layers[l], xs[l], y=ys[l], workspace=ws, wstruct=wstructs[l],
                    stream=stream)
        moe.rms_renorm(ys[l], x=xs[l + 1], eps=EPS, stream=stream)


def test_stack_teacher_forced_and_graph():
    L = 6
    shape = inputs.DECODE
    say(f"stack of {L} decode layers")
    layers = [inputs.make_layer(shape, seed=0, layer=100 + l, device="cuda") for l in range(L)]
    wstructs = [moe.weights_struct(lw) for lw in layers]
    cfg = moe.config(shape)
    ws = moe.alloc_workspace(cfg, 1)
    xs = [torch.empty(1, shape.hidden, dtype=torch.bfloat16, device="cuda") for _ in range(L + 1)]
    ys = [torch.empty_like(xs[0]) for _ in range(L)]
    x0 = inputs.make_x(shape, 1, seed=42, device="cuda")
    xs[0].copy_(x0)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()  # the copy ran on the default stream
    with torch.cuda.stream(stream):
        _chain(cfg, layers, wstructs, xs, ys, ws, stream)
    torch.cuda.synchronize()
    eager_x = [bits(t.cpu()) for t in xs]
    eager_y = [bits(t.cpu()) for t in ys]

    # teacher-forced: oracle layer l on the GPU's x_l
    for l in range(L):
        host = layers[l].to("cpu")
        xl = xs[l].cpu()
        yo, acc, ids, _ = oracle.forward(shape, host, xl)
        rel, worst = rel_rows(eager_y[l], acc)
        gids, _, _ = moe.route(cfg, xs[l], layers[l].router_w, None,
                               logits=torch.empty(1, shape.n_experts, device="cuda"))
        torch.cuda.synchronize()
        say(f"  layer {l}: relL2 {rel:.2e}")
        assert np.array_equal(gids.cpu().numpy(), ids)
        assert rel <= OUT_TOL
        assert worst <= OUT_TOL, (rel, worst)  # each row on its own
        assert np.array_equal(oracle.rms_renorm(ys[l].cpu(), eps=EPS), eager_x[l + 1])
        assert abs(np.sqrt(np.mean(exact.bits_to_f32(eager_x[l + 1]).astype(np.float64) ** 2))
                   - 1.0) < 1e-2

    # the same chain captured as one graph, replayed with eager work between
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        _chain(cfg, layers, wstructs, xs, ys, ws, stream)  # warm the capture stream
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        _chain(cfg, layers, wstructs, xs, ys, ws, stream)
    for rep in range(3):
        for t in xs[1:] + ys:
            t.fill_(float("nan"))
        xs[0].copy_(x0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert np.array_equal(bits(ys[l].cpu()), eager_y[l]), (rep, l)
            assert np.array_equal(bits(xs[l + 1].cpu()), eager_x[l + 1]), (rep, l)


def _chain_outputs(shape, layers, wstructs, x0, eps=EPS):
    cfg = moe.config(shape)
    ws = moe.alloc_workspace(cfg, x0.shape[0])
    x = x0
    ys = []
    for l in range(len(layers)):
        y = torch.empty_like(x0)
        moe.forward(cfg, layers[l], x, y=y, workspace=ws, wstruct=wstructs[l])
        ys.append(y)
        x = moe.rms_renorm(y, eps=eps)
    torch.cuda.synchronize()
    return [bits(y.cpu()) for y in ys]


@pytest.mark.parametrize("shape_name,T,L", [("DECODE", 1, 6), ("DECODE", 2, 3), ("TINY", 1, 5),
                                            ("TINY", 4, 4), ("DECODE", 1, 1), ("DECODE", 4, 2)])
def test_forward_stack_equals_chain(shape_name, T, L):
    shape = getattr(inputs, shape_name)
    say(f"stack {shape_name} T={T} L={L}")
    layers = [inputs.make_layer(shape, seed=1, layer=200 + l, device="cuda") for l in range(L)]
    wstructs = [moe.weights_struct(lw) for lw in layers]
    x0 = inputs.make_x(shape, T, seed=43, device="cuda")
    want = _chain_outputs(shape, layers, wstructs, x0)
    cfg = moe.config(shape)
    arr = moe.weights_array(layers)
    ws = moe.alloc_workspace(cfg, T)
    ys = torch.empty(L, T, shape.hidden, dtype=torch.bfloat16, device="cuda")
    for rep in range(3):  # repeated calls on one workspace (epochs advance)
        ys.fill_(float("nan"))
        y = moe.forward_stack(cfg, arr, x0, ys=ys, eps=EPS, workspace=ws)
        torch.cuda.synchronize()
        for l in range(L):
            assert np.array_equal(bits(ys[l].cpu()), want[l]), (rep, l)
        assert np.array_equal(bits(y.cpu()), want[-1])
    assert moe.decode_status(ws) == 0
    # the last output alone, no per-layer outputs (the workspace's buffers)
    y2 = moe.forward_stack(cfg, arr, x0, eps=EPS, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y2.cpu()), want[-1])


def test_forward_stack_graph_replays():
    shape, L = inputs.DECODE, 4
    layers = [inputs.make_layer(shape, seed=2, layer=300 + l, device="cuda") for l in range(L)]
    wstructs = [moe.weights_struct(lw) for lw in layers]
    x0 = inputs.make_x(shape, 1, seed=44, device="cuda")
    want = _chain_outputs(shape, layers, wstructs, x0)
    cfg = moe.config(shape)
    arr = moe.weights_array(layers)
    ws = moe.alloc_workspace(cfg, 1)
    y = torch.empty_like(x0)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        moe.forward_stack(cfg, arr, x0, y=y, eps=EPS, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        moe.forward_stack(cfg, arr, x0, y=y, eps=EPS, workspace=ws, stream=stream)
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(y.cpu()), want[-1]), rep
        # eager work on the same workspace between replays
        moe.forward(cfg, layers[0], x0, workspace=ws, wstruct=wstructs[0])
        torch.cuda.synchronize()


def test_forward_stack_refuses_more_than_four_rows():
    shape = inputs.TINY
    layers = [inputs.make_layer(shape, seed=3, layer=l, device="cuda") for l in range(2)]
    cfg = moe.config(shape)
    x0 = inputs.make_x(shape, 5, seed=45, device="cuda")
    ws = moe.alloc_workspace(cfg, 5)
    with pytest.raises(moe.MoeError, match="UNSUPPORTED"):
        moe.forward_stack(cfg, layers, x0, eps=EPS, workspace=ws)
    torch.cuda.synchronize()
