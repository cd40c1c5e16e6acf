"""Pins of the oracle's one-row bf16 projection y = bf16(fp32(sum_k x W[n])):
exact sums (math.fsum) with torch's own float32 -> bfloat16 cast, identity
and all-ones closed forms, a cancellation that fp32 accumulation would lose,
and row order."""
import math

import numpy as np
import torch

import oracle


def _bf16(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def _exact_ref(W, x):
    Wf = W.float().double().numpy()
    xf = x.float().double().numpy()
    out = np.empty((xf.shape[0], Wf.shape[0]), dtype=np.float32)
    for t in range(xf.shape[0]):
        for n in range(Wf.shape[0]):
            out[t, n] = np.float32(math.fsum(xf[t] * Wf[n]))  # products exact in fp64
    return _bits(torch.from_numpy(out).to(torch.bfloat16))


def test_brute_force_exact_sums():
    g = torch.Generator().manual_seed(0)
    for (N, K, T) in ((5, 256, 3), (7, 384, 1), (3, 1024, 4)):
        W = (torch.randn(N, K, generator=g) * 0.02).bfloat16()
        x = torch.randn(T, K, generator=g).bfloat16()
        assert np.array_equal(oracle.bf16_gemv(W, x), _exact_ref(W, x))


def test_identity_and_ones():
    x = torch.randn(3, 128, generator=torch.Generator().manual_seed(1)).bfloat16()
    eye = torch.eye(128).bfloat16()
    assert np.array_equal(oracle.bf16_gemv(eye, x), _bits(x))
    xi = _bf16(np.arange(-64, 64, dtype=np.float32)[None, :] * np.array([[1.0], [3.0]]))
    ones = torch.ones(4, 128).bfloat16()
    want = np.float32(np.arange(-64, 64).sum()) * np.array([1.0, 3.0], dtype=np.float32)
    got = oracle.bf16_gemv(ones, xi)
    assert np.array_equal(got, np.repeat(_bits(_bf16(want))[:, None], 4, axis=1))


def test_cancellation_needs_more_than_fp32():
    # 2^30 + 1 - 2^30 = 1: an fp32 running sum loses the 1, fp64 keeps it
    K = 128
    x = np.zeros((1, K), dtype=np.float32)
    x[0, :3] = [2.0 ** 30, 1.0, -(2.0 ** 30)]
    W = np.ones((2, K), dtype=np.float32)
    W[1, 1] = 0.5
    y = oracle.bf16_gemv(_bf16(W), _bf16(x))
    assert np.array_equal(y, _bits(_bf16([[1.0, 0.5]])))


def test_rows_permute_with_weights():
    g = torch.Generator().manual_seed(2)
    W = (torch.randn(16, 256, generator=g) * 0.05).bfloat16()
    x = torch.randn(2, 256, generator=g).bfloat16()
    p = torch.randperm(16, generator=g)
    assert np.array_equal(oracle.bf16_gemv(W[p], x), oracle.bf16_gemv(W, x)[:, p.numpy()])
