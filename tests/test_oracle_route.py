"""Pins of the oracle's router: logits, top-K selection and weights.

The router scores 256 experts and keeps 8 (PR #925 "drama: load the
checkpoint with direct I/O in file order and build the codec on its own
thread", commit summary of the backbone); it decides on bf16 logits and its
softmax is fp32 (PR #939 "drama3: Fish Audio Drama 3 text to speech on one
CUDA GPU", "Fidelity against the PyTorch oracle" and "How it fits the
engine" > Precision). Pins: exact rational logits, brute force over all
K-subsets, closed-form softmax, and equivariance under relabelling experts.
"""
import itertools

import numpy as np
import torch

from block_fp8_mixture_router_amd import inputs
from tests import exact


def _case(shape, rows, seed):
    x = inputs.make_x(shape, rows, seed=seed)
    rw = inputs.make_router(shape, seed=seed)
    return x, rw


def test_logits_are_exactly_rounded_sums(oracle_lib):
    for shape, rows, sample in ((inputs.TINY, 8, None), (inputs.DECODE, 4, 64)):
        x, rw = _case(shape, rows, seed=11)
        ids, w, lg = oracle_lib.route(shape, x, rw)
        xb, wb = exact.bf16_bits(x), exact.bf16_bits(rw)
        experts = range(shape.n_experts) if sample is None else \
            np.random.default_rng(0).choice(shape.n_experts, sample, replace=False)
        for t in range(rows):
            for e in experts:
                want = exact.exact_logits_bf16(xb[t], wb[e:e + 1])[0]
                assert lg[t, e] == want, (t, e, lg[t, e], want)


def test_logits_fp32_variant_is_exact_fp32(oracle_lib):
    shape = inputs.TINY
    x, rw = _case(shape, 4, seed=5)
    _, _, lg = oracle_lib.route(shape, x, rw, flags=oracle_lib.LOGITS_FP32)
    xb, wb = exact.bf16_bits(x), exact.bf16_bits(rw)
    for t in range(4):
        for e in range(shape.n_experts):
            n, e0 = exact.exact_dot_bf16(xb[t], wb[e])
            assert lg[t, e] == exact.round_dyadic_to_f32(n, e0)


def test_selection_bruteforce_all_subsets(oracle_lib):
    shape = inputs.TINY
    x, rw = _case(shape, 32, seed=3)
    # make exact ties: expert 9 copies expert 2's router row, 14 copies 5's
    rw = rw.clone()
    rw[9] = rw[2]
    rw[14] = rw[5]
    ids, w, lg = oracle_lib.route(shape, x, rw)
    K, E = shape.top_k, shape.n_experts

    def key(t, e):  # larger is better: higher logit, then lower index
        return (lg[t, e], -e)

    for t in range(32):
        best = max(itertools.combinations(range(E), K),
                   key=lambda S: sorted((key(t, e) for e in S), reverse=True))
        want = sorted(best, key=lambda e: key(t, e), reverse=True)
        assert list(ids[t]) == want
        assert lg[t, 9] == lg[t, 2] and lg[t, 14] == lg[t, 5]


def test_weights_softmax_of_selected(oracle_lib):
    shape = inputs.DECODE
    x, rw = _case(shape, 16, seed=4)
    ids, w, lg = oracle_lib.route(shape, x, rw)
    sel = np.take_along_axis(lg, ids, axis=1).astype(np.float64)
    ref = np.exp(sel - sel.max(axis=1, keepdims=True))
    ref /= ref.sum(axis=1, keepdims=True)
    assert np.max(np.abs(w - ref)) <= 1e-6
    assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 1e-6
    assert np.all(np.diff(w, axis=1) <= 0)
    assert np.all(np.diff(sel, axis=1) <= 0)


def test_bias_added_before_selection(oracle_lib):
    shape = inputs.DECODE
    x, rw = _case(shape, 64, seed=9)
    bias = inputs.skew_bias(shape.n_experts)
    ids0, _, lg0 = oracle_lib.route(shape, x, rw)
    ids, w, lg = oracle_lib.route(shape, x, rw, router_bias=bias)
    assert np.array_equal(lg, (lg0 + bias.numpy()).astype(np.float32))
    cold = bias.numpy() < 0
    assert not np.any(cold[ids])
    hot = bias.numpy() > 0
    assert hot[ids].mean() > 0.5


def test_relabelling_experts_permutes_ids(oracle_lib):
    shape = inputs.TINY
    x, rw = _case(shape, 16, seed=21)
    perm = np.random.default_rng(1).permutation(shape.n_experts)  # new e' = perm[e]
    rw_p = torch.empty_like(rw)
    rw_p[torch.from_numpy(perm)] = rw
    ids, w, lg = oracle_lib.route(shape, x, rw)
    ids_p, w_p, lg_p = oracle_lib.route(shape, x, rw_p)
    assert np.array_equal(lg_p[:, perm], lg)
    for t in range(16):
        vals = np.sort(lg[t])[::-1]
        if vals[shape.top_k - 1] == vals[shape.top_k]:
            continue  # a tie at the boundary may resolve differently after relabelling
        assert sorted(perm[ids[t]]) == sorted(ids_p[t])
        assert np.allclose(np.sort(w[t]), np.sort(w_p[t]), atol=0, rtol=0)
