"""The oracle on exact instances of the whole layer.

The instances in tests/exact_instance.py make every product and sum of the
layer exact, so the layer has a single correct output, computed there in
float64 without the oracle. The oracle must reproduce it bit for bit: ids,
weights (exactly 1/K), the fp32 pre-rounding sum and the bf16 output. This
checks the oracle's block scales, gate/up/down indexing, requantisation of h,
shared expert and combine all at once, free of any summation-order question.
"""
import dataclasses

import numpy as np
import pytest

from block_fp8_mixture_router_amd import inputs
from tests import exact_instance as xi

SHAPES = {
    "tiny": inputs.TINY,
    "decode_E32": dataclasses.replace(inputs.DECODE, n_experts=32),
    "tiny_single_expert": dataclasses.replace(inputs.TINY, n_experts=1, top_k=1),
    "tiny_no_shared": dataclasses.replace(inputs.TINY, shared_inter=0),
    "tiny_I256_K2": dataclasses.replace(inputs.TINY, inter=256, top_k=2),
}


@pytest.mark.parametrize("name,T", [("tiny", 7), ("decode_E32", 3), ("tiny_single_expert", 4),
                                    ("tiny_no_shared", 5), ("tiny_I256_K2", 6)])
def test_oracle_reproduces_exact_instance(oracle_lib, name, T):
    shape = SHAPES[name]
    inst = xi.build(shape, T, seed=11)
    y, acc, ids, w = oracle_lib.forward(shape, inst.weights, inst.x)
    assert np.array_equal(ids, inst.ids)
    assert np.all(w == np.float32(1.0 / shape.top_k))
    assert np.array_equal(acc, inst.acc)
    assert np.array_equal(xi.zero_sign_blind(y), xi.zero_sign_blind(inst.y_bits))
    # the instance is not degenerate: almost every output is nonzero and the
    # routed experts move the output (it differs from the shared part alone)
    assert np.mean(inst.acc != 0) > 0.9
    if shape.shared_inter:
        _, acc_sh, _, _ = oracle_lib.forward(shape, inst.weights, inst.x, shared=True)
        no_routed = dataclasses.replace(inst.weights, w_down=inst.weights.w_down * 0)
        _, acc_only_shared, _, _ = oracle_lib.forward(shape, no_routed, inst.x)
        assert np.mean(acc_only_shared != acc_sh) > 0.3


@pytest.mark.parametrize("name,T", [("tiny", 7), ("decode_E32", 3), ("tiny_I256_K2", 5)])
def test_oracle_reproduces_exact_instance_with_activation_scales(oracle_lib, name, T):
    """The same with activation scales of 1, 2 and 4 across the groups, so
    each group's scale enters its own block products."""
    shape = SHAPES[name]
    inst = xi.build(shape, T, seed=13, act_scales=True)
    g = shape.hidden // 128
    amax = inst.x.float().numpy()[:, 127::128]
    assert len(np.unique(amax)) > 1 or g == 1
    y, acc, ids, w = oracle_lib.forward(shape, inst.weights, inst.x)
    assert np.array_equal(ids, inst.ids)
    assert np.array_equal(acc, inst.acc)
    assert np.array_equal(xi.zero_sign_blind(y), xi.zero_sign_blind(inst.y_bits))
