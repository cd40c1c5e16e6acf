"""The one-row bf16 projection on the GPU against the oracle, bit for bit
(the same exact-products-in-fp64 rule, rounded once to fp32, then bf16)."""
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


@pytest.mark.parametrize("N,K,T", [
    (1, 128, 1), (8, 128, 4), (37, 384, 3), (1000, 1152, 1), (2048, 2048, 1),
    (4096, 2048, 4), (2048, 4096, 2), (513, 8192, 1), (6144, 2048, 1),
])
def test_gemv_matches_oracle(N, K, T):
    say(f"bf16 gemv N={N} K={K} T={T}")
    g = torch.Generator(device="cuda").manual_seed(N + K + T)
    W = (torch.randn(N, K, device="cuda", generator=g) * 0.02).bfloat16()
    x = torch.randn(T, K, device="cuda", generator=g).bfloat16()
    y = moe.bf16_gemv(W, x)
    torch.cuda.synchronize()
    want = oracle.bf16_gemv(W.cpu(), x.cpu())
    got = bits(y.cpu())
    bad = int((got != want).sum())
    say(f"  mismatches {bad} of {got.size}")
    assert bad == 0


def test_gemv_cancellation_and_specials():
    # fp32 accumulation would lose the 1 in 2^30 + 1 - 2^30
    K = 256
    x = torch.zeros(2, K)
    x[0, :3] = torch.tensor([2.0 ** 30, 1.0, -(2.0 ** 30)])
    x[1, 5] = 3.0
    W = torch.ones(16, K)
    W[3, 1] = -0.5
    y = moe.bf16_gemv(W.bfloat16().cuda(), x.bfloat16().cuda())
    torch.cuda.synchronize()
    assert np.array_equal(bits(y.cpu()), oracle.bf16_gemv(W.bfloat16(), x.bfloat16()))
    yc = y.float().cpu()
    assert yc[0, 0] == 1.0 and yc[0, 3] == -0.5 and torch.all(yc[1] == 3.0)


def test_gemv_graph_replay_and_rotation():
    """Captured in a graph over rotated weights (the bench's launch), every
    replay equal to the eager result."""
    N, K = 4096, 2048
    g = torch.Generator(device="cuda").manual_seed(3)
    Ws = [(torch.randn(N, K, device="cuda", generator=g) * 0.02).bfloat16() for _ in range(3)]
    x = torch.randn(1, K, device="cuda", generator=g).bfloat16()
    ys = [torch.empty(1, N, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    eager = [moe.bf16_gemv(W, x).clone() for W in Ws]
    st = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        for W, y in zip(Ws, ys):
            moe.bf16_gemv(W, x, y=y, stream=st)
        torch.cuda.synchronize()
        with torch.cuda.graph(gr, stream=st):
            for W, y in zip(Ws, ys):
                moe.bf16_gemv(W, x, y=y, stream=st)
    for rep in range(3):
        for y in ys:
            y.fill_(0)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y.view(torch.int16), e.view(torch.int16))
