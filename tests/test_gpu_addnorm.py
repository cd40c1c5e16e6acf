"""GPU parity of moe_add_rmsnorm_quant (residual add, RMS norm and 1x128
quantisation in front of the layer): every output bit-exact against the
oracle, in place and out of place, and its FP8 groups equal to moe_quant_act
applied to its normed rows."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
import oracle
from tests.gpu_common import bits, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _inputs(T, H, seed):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(T, H, generator=g).to(torch.bfloat16)
    r = (torch.randn(T, H, generator=g) * 4).to(torch.bfloat16)
    w = (torch.rand(H, generator=g) + 0.25).to(torch.bfloat16)
    if T >= 4:
        h[0] = 0.0                                  # zero row: the clamped group scale
        r[0] = 0.0
        h[1] = 3.0                                  # constant row
        r[1] = 0.0
        h[2] = torch.linspace(-300, 300, H)         # wide range
        r[3] = -h[3]                                # cancels to zero
    return h, r, w


@pytest.mark.parametrize("T,H", [(1, 2048), (5, 256), (64, 2048), (3, 8192), (1024, 2048),
                                 (2, 384), (3, 6144)])
@pytest.mark.parametrize("in_place", [False, True])
def test_add_rmsnorm_quant_bit_exact(T, H, in_place):
    say(f"add_rmsnorm_quant T={T} H={H} in_place={in_place}")
    h, r, w = _inputs(T, H, seed=T * 7 + H)
    eps = 1e-6
    want = oracle.add_rmsnorm_quant(h, r, w, eps=eps)
    hd, rd, wd = h.cuda(), r.cuda(), w.cuda()
    ro, x, q, s = moe.add_rmsnorm_quant(hd, rd, wd, eps=eps,
                                        residual_out=rd if in_place else None)
    torch.cuda.synchronize()
    assert np.array_equal(bits(ro.cpu()), want[0])
    assert np.array_equal(bits(x.cpu()), want[1])
    assert np.array_equal(q.cpu().numpy(), want[2])
    assert np.array_equal(s.cpu().numpy().view(np.uint32), want[3].view(np.uint32))
    # the FP8 groups are those of the separate quantisation of x
    q2, s2 = moe.quant_act(x)
    torch.cuda.synchronize()
    assert torch.equal(q2, q) and torch.equal(s2.view(torch.int32), s.view(torch.int32))


def test_add_rmsnorm_quant_in_a_graph():
    """Captured in a graph and replayed (with eager work between replays),
    every replay gives the eager bytes."""
    T, H = 64, 2048
    h, r, w = _inputs(T, H, seed=77)
    hd, rd, wd = h.cuda(), r.cuda(), w.cuda()
    ro, x, q, s = moe.add_rmsnorm_quant(hd, rd, wd)
    torch.cuda.synchronize()
    want = [t.clone() for t in (ro, x, q, s)]
    stream = torch.cuda.Stream()
    outs = [torch.empty_like(t) for t in want]
    with torch.cuda.stream(stream):
        moe.add_rmsnorm_quant(hd, rd, wd, residual_out=outs[0], x=outs[1], q=outs[2],
                              scales=outs[3], stream=stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        moe.add_rmsnorm_quant(hd, rd, wd, residual_out=outs[0], x=outs[1], q=outs[2],
                              scales=outs[3], stream=stream)
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep


def test_add_norm_then_layer_matches_the_oracle_chain():
    """The step in front of the layer feeding the layer: the layer's output on
    the GPU's normed rows is within tolerance of the oracle layer on the
    oracle's normed rows (which are bit-identical to the GPU's)."""
    from tests.gpu_common import OUT_TOL, layer, rel_rows
    shape, dev, host = layer("DECODE", 0, False)
    for T in (1, 300):
        say(f"add-norm then layer T={T}")
        h, r, w = _inputs(T, shape.hidden, seed=90 + T)
        _, x_o, _, _ = oracle.add_rmsnorm_quant(h, r, w)
        _, x_d, _, _ = moe.add_rmsnorm_quant(h.cuda(), r.cuda(), w.cuda())
        assert np.array_equal(bits(x_d.cpu()), x_o)
        cfg = moe.config(shape)
        y = moe.forward(cfg, dev, x_d)
        torch.cuda.synchronize()
        xt = torch.from_numpy(x_o.view(np.int16)).view(torch.bfloat16)
        _, acc, _, _ = oracle.forward(shape, host, xt)
        rel, worst = rel_rows(bits(y.cpu()), acc)
        say(f"  relL2 {rel:.2e} worst row {worst:.2e}")
        assert rel <= OUT_TOL
