"""GPU parity of moe_quant_act and moe_route against the oracle: codes,
scales, expert ids and logits bit-exact; routing weights within 1e-6."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
import oracle
from block_fp8_mixture_router_amd import inputs
from tests import exact
from tests.gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("T,C,scale", [(1, 256, 1.0), (1, 2048, 1.0), (3, 384, 1e-3),
                                       (1024, 2048, 1.0), (17, 2048, 300.0), (5, 128, 1e-30)])
def test_quant_act_bit_exact(T, C, scale):
    say(f"quant_act T={T} C={C} scale={scale}")
    g = torch.Generator(device="cuda").manual_seed(T * 7 + C)
    x = (torch.randn(T, C, generator=g, device="cuda") * scale).to(torch.bfloat16)
    q, s = moe.quant_act(x)
    torch.cuda.synchronize()
    qo, so = oracle.quant_act(x.cpu())
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qo)


def test_quant_act_every_bf16_value():
    """Every finite bf16 value up to 448 * 2^k, in groups whose amax is
    448 * 2^k: the scale is then the power of two 2^k and x / s is exact, so
    the e4m3 conversion itself is checked against the oracle for every bf16
    input, at several k."""
    vals = exact.bits_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    vals = vals[np.isfinite(vals)]
    for k in (0, -3, 5):
        anchor = np.float32(448.0 * 2.0 ** k)
        v = vals[np.abs(vals) <= anchor]
        pad = (-len(v)) % 127
        v = np.concatenate([v, np.zeros(pad, np.float32)]).reshape(-1, 127)
        rows = np.concatenate([np.full((v.shape[0], 1), anchor, np.float32), v], axis=1)
        x = torch.from_numpy(rows.reshape(1, -1)).to(torch.bfloat16)
        assert np.array_equal(x.float().numpy().reshape(rows.shape), rows)
        say(f"quant sweep k={k} groups={rows.shape[0]}")
        q, s = moe.quant_act(x.cuda())
        torch.cuda.synchronize()
        qo, so = oracle.quant_act(x)
        assert np.all(so == np.float32(2.0 ** k))
        assert np.array_equal(s.cpu().numpy(), so)
        bad = np.nonzero(q.cpu().numpy() != qo)[1]
        assert bad.size == 0, [(float(x[0, i]), int(q[0, i]), int(qo[0, i])) for i in bad[:8]]


@pytest.mark.parametrize("amax_bits", [0x3F80, 0x4049, 0x3BE0, 0x447A, 0x37C9, 0x5082, 0x3F7F])
def test_quant_act_every_bf16_value_inexact_scales(amax_bits):
    """Every finite bf16 value a with |a| <= amax, in groups whose amax is not
    448 times a power of two: the quotients a / s are inexact, so the
    kernel's correctly rounded division and the e4m3 rounding of its result
    are checked against the oracle for every bf16 numerator at each scale."""
    vals = exact.bits_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    vals = vals[np.isfinite(vals)]
    anchor = exact.bits_to_f32(np.array([amax_bits], np.uint16))[0]
    v = vals[np.abs(vals) <= anchor]
    pad = (-len(v)) % 127
    v = np.concatenate([v, np.zeros(pad, np.float32)]).reshape(-1, 127)
    rows = np.concatenate([np.full((v.shape[0], 1), anchor, np.float32), v], axis=1)
    x = torch.from_numpy(rows.reshape(1, -1)).to(torch.bfloat16)
    say(f"quant sweep amax={anchor} groups={rows.shape[0]}")
    q, s = moe.quant_act(x.cuda())
    torch.cuda.synchronize()
    qo, so = oracle.quant_act(x)
    assert np.array_equal(s.cpu().numpy(), so)
    bad = np.nonzero(q.cpu().numpy() != qo)[1]
    assert bad.size == 0, [(float(x[0, i]), int(q[0, i]), int(qo[0, i])) for i in bad[:8]]


def test_quant_act_special_groups():
    x = torch.zeros(1, 512)
    x[0, 128:256] = -0.0
    x[0, 200] = -1e-38
    x[0, 300] = 3.0e38
    x[0, 301] = -2.0
    x[0, 384:] = torch.linspace(-1, 1, 128)
    xb = x.to(torch.bfloat16)
    q, s = moe.quant_act(xb.cuda())
    torch.cuda.synchronize()
    qo, so = oracle.quant_act(xb)
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(q.cpu().numpy(), qo)


def _route_case(shape, T, seed, bias=None, dup=False, flags=0):
    x = inputs.make_x(shape, T, seed=seed, device="cuda")
    rw = inputs.make_router(shape, seed=seed, device="cuda")
    if dup:
        rw[9] = rw[2]
        rw[shape.n_experts - 1] = rw[0]
    b = None if bias is None else bias.cuda()
    cfg = moe.config(shape, flags)
    logits = torch.empty(T, shape.n_experts, dtype=torch.float32, device="cuda")
    ids, w, _ = moe.route(cfg, x, rw, b, logits=logits)
    torch.cuda.synchronize()
    ido, wo, lo = oracle.route(shape, x.cpu(), rw.cpu(), None if bias is None else bias,
                               flags=(oracle.LOGITS_FP32 if flags & moe.LOGITS_FP32 else 0))
    return ids.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy(), ido, wo, lo


@pytest.mark.parametrize("shape_name,T,skewed,dup,flags", [
    ("TINY", 1, False, False, 0), ("TINY", 7, False, True, 0), ("TINY", 40, False, True, 0),
    ("DECODE", 1, False, False, 0), ("DECODE", 4, False, False, 0),
    ("DECODE", 16, False, True, 0), ("DECODE", 17, False, True, 0),
    ("DECODE", 1024, False, False, 0), ("DECODE", 1024, True, False, 0),
    ("DECODE", 333, False, True, 0), ("DECODE", 64, False, False, moe.LOGITS_FP32),
    ("DECODE", 3, False, False, moe.LOGITS_FP32),
])
def test_route_bit_exact(shape_name, T, skewed, dup, flags):
    shape = getattr(inputs, shape_name)
    say(f"route {shape_name} T={T} skewed={skewed} dup={dup} flags={flags}")
    bias = inputs.skew_bias(shape.n_experts) if skewed else None
    ids, w, lg, ido, wo, lo = _route_case(shape, T, seed=T, bias=bias, dup=dup, flags=flags)
    bad = np.nonzero(lg.view(np.uint32) != lo.view(np.uint32))
    assert bad[0].size == 0, list(zip(bad[0][:5], bad[1][:5]))
    assert np.array_equal(ids, ido)
    assert np.max(np.abs(w - wo)) <= 1e-6
    if skewed:
        cold = bias.numpy() < 0
        assert not np.any(cold[ids])
        share = (bias.numpy()[ids] > 0).mean()
        say(f"  hot share {share:.3f}, empty experts {256 - len(np.unique(ids))}")


@pytest.mark.parametrize("shape_name,T,case,flags", [
    ("TINY", 40, "dup", 0), ("DECODE", 17, "dup", 0), ("DECODE", 300, "plain", 0),
    ("DECODE", 1024, "plain", 0), ("DECODE", 1024, "skewed", 0), ("DECODE", 1024, "dup", 0),
    ("DECODE", 513, "plain", moe.LOGITS_FP32), ("DECODE", 200, "concentrated", 0),
    ("DECODE", 64, "zero_router", 0), ("DECODE", 64, "tied_block", 0),
])
def test_route_bounded_scores_bit_exact(shape_name, T, case, flags):
    """Without a logits buffer and above 16 rows, moe_route ranks bf16 MFMA
    scores with an error bound and computes exact logits only for the
    experts the bound leaves undecided. ids must equal the oracle's, and the
    weights must equal, bit for bit, those of the path that computes every
    logit exactly."""
    shape = getattr(inputs, shape_name)
    say(f"bounded route {shape_name} T={T} case={case} flags={flags}")
    x = inputs.make_x(shape, T, seed=T + 7, device="cuda")
    rw = inputs.make_router(shape, seed=T + 7, device="cuda")
    bias = None
    if case == "dup":
        rw[9] = rw[2]
        rw[shape.n_experts - 1] = rw[0]
    elif case == "skewed":
        bias = inputs.skew_bias(shape.n_experts)
    elif case == "concentrated":
        bias = inputs.concentrated_bias(shape.n_experts)
    elif case == "zero_router":
        rw.zero_()
    elif case == "tied_block":
        rw[16:48] = rw[16]  # 32 identical experts: exact ties decided by index
    b = None if bias is None else bias.cuda()
    cfg = moe.config(shape, flags)
    ws = moe.alloc_workspace(cfg, T)
    ids, w, _ = moe.route(cfg, x, rw, b, workspace=ws)
    logits = torch.empty(T, shape.n_experts, dtype=torch.float32, device="cuda")
    ids_x, w_x, _ = moe.route(cfg, x, rw, b, logits=logits)
    torch.cuda.synchronize()
    ido, wo, _ = oracle.route(shape, x.cpu(), rw.cpu(), bias,
                              flags=(oracle.LOGITS_FP32 if flags & moe.LOGITS_FP32 else 0))
    assert np.array_equal(ids.cpu().numpy(), ido)
    assert np.array_equal(ids.cpu().numpy(), ids_x.cpu().numpy())
    assert np.array_equal(w.cpu().numpy().view(np.uint32), w_x.cpu().numpy().view(np.uint32))
    assert np.max(np.abs(w.cpu().numpy() - wo)) <= 1e-6


def test_route_logits_in_workspace():
    shape = inputs.DECODE
    x = inputs.make_x(shape, 20, seed=1, device="cuda")
    rw = inputs.make_router(shape, seed=1, device="cuda")
    cfg = moe.config(shape)
    ws = moe.alloc_workspace(cfg, 20)
    ids, w, _ = moe.route(cfg, x, rw, workspace=ws)
    torch.cuda.synchronize()
    ido, wo, _ = oracle.route(shape, x.cpu(), rw.cpu())
    assert np.array_equal(ids.cpu().numpy(), ido)
