"""Every fp32 value through the kernels' fp32 -> e4m3 conversion
(moe_e4m3_encode: saturate to +-448, round to nearest even) against the
oracle's encoder, which works from the definition (exact grid spacing per
binade, nearest with ties to even). All 2^32 bit patterns are swept in
chunks; NaN inputs are outside the contract and skipped."""
import numpy as np
import pytest
import torch

import block_fp8_mixture_router_amd as moe
import oracle
from tests.gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26


def test_e4m3_encode_every_fp32_value():
    need_gpu()
    torch.cuda.set_device(0)
    base = torch.arange(CHUNK, dtype=torch.int64, device="cuda")
    q = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    mismatches, first = 0, None
    for c in range((1 << 32) // CHUNK):
        start = c * CHUNK
        v = base + start
        v = torch.where(v >= (1 << 31), v - (1 << 32), v).to(torch.int32)  # the same 32 bits
        moe.e4m3_encode(v.view(torch.float32), q)
        got = q.cpu().numpy()
        xa = np.arange(start, start + CHUNK, dtype=np.uint32).view(np.float32)
        want = oracle.e4m3_encode(xa)
        ok = (got == want) | np.isnan(xa)
        if not ok.all():
            bad = np.flatnonzero(~ok)
            mismatches += bad.size
            if first is None:
                i = bad[0]
                first = (hex(start + int(i)), float(xa[i]), int(got[i]), int(want[i]))
        if c % 16 == 15:
            say(f"  e4m3 sweep: {(c + 1) * CHUNK:#x} patterns, mismatches {mismatches}")
    assert mismatches == 0, (mismatches, first)
