"""Pins of the oracle's whole layer.

Special cases that reduce to a library routine (one expert = a dense SwiGLU
MLP by numpy matmul on dequantised weights), invariants the method fixes
(identical experts, a shared gate of exactly 0 or 1/2, relabelling experts,
row independence), an independent fp64 brute force of the tiny layer, and the
size of the effect of the activation quantisation, which the pages put near
1e-2 relative (PR #939 "drama3: Fish Audio Drama 3 text to speech on one CUDA
GPU", "How it fits the engine" > Precision).
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_fp8_mixture_router_amd import inputs
from tests import exact


def _layer(shape, seed=0, skewed=False):
    return inputs.make_layer(shape, seed=seed, skewed=skewed)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _dense_routed(shape, lw, e, x_row_bits, quant):
    """Routed expert e on one row by numpy matmul on dequantised weights."""
    xf = exact.bits_to_f32(x_row_bits).astype(np.float64)
    if quant:
        q, s = exact.quant_groups_bruteforce(xf.astype(np.float32))
        xd = exact.e4m3_table_torch()[q.reshape(-1).astype(np.int64)] * np.repeat(s, 128)
    else:
        xd = xf
    Wg = exact.dequant_block(lw.w_gate[e].numpy(), lw.s_gate[e].numpy())
    Wu = exact.dequant_block(lw.w_up[e].numpy(), lw.s_up[e].numpy())
    Wd = exact.dequant_block(lw.w_down[e].numpy(), lw.s_down[e].numpy())
    h = _silu(Wg @ xd) * (Wu @ xd)
    if quant:
        q, s = exact.quant_groups_bruteforce(h.astype(np.float32))
        h = exact.e4m3_table_torch()[q.reshape(-1).astype(np.int64)] * np.repeat(s, 128)
    return Wd @ h


def _dense_shared(lw, x_row_bits):
    xf = exact.bits_to_f32(x_row_bits).astype(np.float64)
    Wsg = lw.sh_gate.double().numpy()
    Wsu = lw.sh_up.double().numpy()
    Wsd = lw.sh_down.double().numpy()
    hs = _silu(Wsg @ xf) * (Wsu @ xf)
    hs = exact.bits_to_f32(exact.f32_to_bf16_torch(hs.astype(np.float32))).astype(np.float64)
    z = float(lw.sh_gate_w.double().numpy() @ xf)
    return Wsd @ hs, 1.0 / (1.0 + np.exp(-z))


def test_single_expert_is_dense_mlp(oracle_lib):
    shape = dataclasses.replace(inputs.TINY, n_experts=1, top_k=1)
    lw = _layer(shape, seed=1)
    x = inputs.make_x(shape, 3, seed=1)
    xb = exact.bf16_bits(x)
    # without activation quantisation the block GEMM structure is pinned tightly
    _, acc, ids, w = oracle_lib.forward(shape, lw, x, flags=oracle_lib.NO_ACT_QUANT,
                                        shared=False)
    assert np.all(ids == 0) and np.all(w == 1.0)
    for t in range(3):
        ref = _dense_routed(shape, lw, 0, xb[t], quant=False)
        assert exact.rel_l2(acc[t], ref) < 1e-6
    # with quantisation the same, up to rare one-code flips of the intermediate
    _, acc, _, _ = oracle_lib.forward(shape, lw, x, shared=False)
    for t in range(3):
        ref = _dense_routed(shape, lw, 0, xb[t], quant=True)
        assert exact.rel_l2(acc[t], ref) < 2e-3


def test_identical_experts_reduce_to_one(oracle_lib):
    shape = inputs.TINY
    lw = _layer(shape, seed=2)
    for name in ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down"):
        t = getattr(lw, name)
        t[:] = t[3:4].clone()
    one = dataclasses.replace(shape, n_experts=1, top_k=1)
    lw1 = dataclasses.replace(lw, shape=one, router_w=lw.router_w[3:4].clone())
    for name in ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down"):
        setattr(lw1, name, getattr(lw, name)[3:4].clone())
    x = inputs.make_x(shape, 6, seed=2)
    _, acc, _, w = oracle_lib.forward(shape, lw, x)
    _, acc1, _, _ = oracle_lib.forward(one, lw1, x)
    assert np.max(np.abs(w.sum(axis=1) - 1)) < 1e-6
    assert exact.rel_l2(acc, acc1) < 1e-6


def test_zero_gate_removes_shared_branch(oracle_lib):
    shape = inputs.TINY
    lw = _layer(shape, seed=3)
    x = inputs.make_x(shape, 5, seed=3)
    # a single gate vector must close the gate for every row: one row here
    for t in range(5):
        xt = x[t:t + 1]
        lw.sh_gate_w = (-0.125 * torch.sign(xt[0].float())).to(torch.bfloat16)
        y, acc, _, _ = oracle_lib.forward(shape, lw, xt)
        y0, acc0, _, _ = oracle_lib.forward(shape, lw, xt, shared=False)
        assert np.array_equal(exact.bits_to_f32(y), exact.bits_to_f32(y0))
        assert np.array_equal(acc, acc0)


def test_half_gate_and_shared_mlp(oracle_lib):
    shape = inputs.TINY
    lw = _layer(shape, seed=4)
    # routed experts output exactly zero: all-zero codes
    lw.w_down.zero_()
    lw.sh_gate_w = torch.zeros_like(lw.sh_gate_w)
    x = inputs.make_x(shape, 4, seed=4)
    _, acc, _, _ = oracle_lib.forward(shape, lw, x)
    xb = exact.bf16_bits(x)
    for t in range(4):
        s, gamma = _dense_shared(lw, xb[t])
        assert gamma == 0.5
        assert exact.rel_l2(acc[t], 0.5 * s) < 1e-5


def test_whole_tiny_layer_bruteforce(oracle_lib):
    shape = inputs.TINY
    lw = _layer(shape, seed=0)
    x = inputs.make_x(shape, 4, seed=0)
    xb = exact.bf16_bits(x)
    wb = exact.bf16_bits(lw.router_w)
    y, acc, ids, w = oracle_lib.forward(shape, lw, x)
    for t in range(4):
        lg = exact.exact_logits_bf16(xb[t], wb)
        order = sorted(range(shape.n_experts), key=lambda e: (-lg[e], e))[:shape.top_k]
        assert list(ids[t]) == order
        sel = lg[order].astype(np.float64)
        ww = np.exp(sel - sel.max())
        ww /= ww.sum()
        ref = sum(ww[j] * _dense_routed(shape, lw, order[j], xb[t], quant=True)
                  for j in range(shape.top_k))
        s, gamma = _dense_shared(lw, xb[t])
        ref = ref + gamma * s
        assert exact.rel_l2(acc[t], ref) < 2e-3
    assert np.array_equal(y, exact.f32_to_bf16_torch(acc))


def test_activation_quantisation_effect_size(oracle_lib):
    shape = inputs.TINY
    lw = _layer(shape, seed=5)
    x = inputs.make_x(shape, 16, seed=5)
    _, acc, _, _ = oracle_lib.forward(shape, lw, x, shared=False)
    _, acc_nq, _, _ = oracle_lib.forward(shape, lw, x, flags=oracle_lib.NO_ACT_QUANT,
                                         shared=False)
    d = exact.rel_l2(acc_nq, acc)
    assert 3e-3 < d < 1e-1, d


def test_relabelling_experts_leaves_output(oracle_lib):
    shape = inputs.TINY
    lw = _layer(shape, seed=6)
    x = inputs.make_x(shape, 8, seed=6)
    perm = torch.from_numpy(np.random.default_rng(2).permutation(shape.n_experts))
    lwp = dataclasses.replace(lw)
    for name in ("router_w", "w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down"):
        t = getattr(lw, name)
        tp = torch.empty_like(t)
        tp[perm] = t
        setattr(lwp, name, tp)
    y, acc, ids, _ = oracle_lib.forward(shape, lw, x)
    yp, accp, idsp, _ = oracle_lib.forward(shape, lwp, x)
    assert np.array_equal(perm.numpy()[ids], idsp)
    assert np.array_equal(acc, accp)


def test_rows_are_independent(oracle_lib):
    shape = inputs.TINY
    lw = _layer(shape, seed=7)
    x = inputs.make_x(shape, 9, seed=7)
    y, acc, _, _ = oracle_lib.forward(shape, lw, x)
    for t in (0, 4, 8):
        y1, acc1, _, _ = oracle_lib.forward(shape, lw, x[t:t + 1])
        assert np.array_equal(y[t], y1[0]) and np.array_equal(acc[t], acc1[0])


def test_empty_input(oracle_lib):
    shape = inputs.TINY
    lw = _layer(shape, seed=8)
    x = inputs.make_x(shape, 0, seed=8)
    y, acc, ids, w = oracle_lib.forward(shape, lw, x)
    assert y.shape == (0, shape.hidden)
