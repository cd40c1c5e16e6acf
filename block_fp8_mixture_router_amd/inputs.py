"""Seeded synthetic inputs for the block-FP8 MoE layer.

This module only draws random tensors. It holds none of the layer's
arithmetic (routing, activation quantisation, expert GEMMs, SwiGLU, gate,
combine). Both the HIP path and the CPU oracle consume what it produces, so
neither side's maths can leak into the other through it.

The layer is the backbone MoE of the pages' "Drama 3" text-to-speech model:
256 experts, top-8, block-FP8 (e4m3) expert weights with one fp32 scale per
128x128 block, bf16 router and bf16 gated shared expert (page 1, PR #925,
commit summary of the backbone; page 4, PR #939, "What it adds" and
"How it fits the engine" > Precision).

The synthetic checkpoint is built the way such a checkpoint is made: fp32
normals N(0, 0.02) per 128x128 block, scale = block amax / 448, codes = the
block divided by its scale and cast with torch's own float8_e4m3fn cast (a
library routine). The hot path never re-quantises weights; it reads these
codes and scales as stored.

Streams: every tensor has its own torch.Generator seeded from
(seed, layer, tensor id), so any tensor can be regenerated alone. Values
depend on the device the generator runs on (CPU and GPU generators differ);
a comparison always generates once and copies the same tensors to both
sides.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

GROUP = 128  # block edge of the weight scales and width of an activation group


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int

    def expert_bytes(self) -> int:
        """FP8 code bytes plus fp32 scale bytes of one routed expert."""
        h, i = self.hidden, self.inter
        codes = 3 * h * i
        scales = 3 * (h // GROUP) * (i // GROUP) * 4
        return codes + scales


# The workloads. Names describe what they are; sizes follow the pages' layer.
TINY = LayerShape(hidden=256, n_experts=16, top_k=4, inter=128, shared_inter=128)
DECODE = LayerShape(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    rows: int
    skewed: bool = False
    layers: int = 1
    renorm_between_layers: bool = False
    description: str = ""


WORKLOADS: Dict[str, Workload] = {
    "tiny_1row": Workload(
        "tiny_1row", TINY, 1,
        description="H256 E16 top4 I=Is=128, one bf16 row"),
    "decode_1row": Workload(
        "decode_1row", DECODE, 1,
        description="H2048 E256 top8 I=Is=512, one bf16 row"),
    "chunk1024_uniform": Workload(
        "chunk1024_uniform", DECODE, 1024,
        description="decode layer on a 1024-row chunk, router N(0,0.02)"),
    "chunk1024_skewed": Workload(
        "chunk1024_skewed", DECODE, 1024, skewed=True,
        description="1024-row chunk, router bias puts ~80% of picks on 16 experts"),
    "stack40_decode": Workload(
        "stack40_decode", DECODE, 1, layers=40, renorm_between_layers=True,
        description="40 independent decode layers chained on one row"),
}

# Tensor ids of the per-tensor streams.
_T_ROUTER, _T_GATE, _T_UP, _T_DOWN, _T_SH_GATE, _T_SH_UP, _T_SH_DOWN, _T_SH_GW, _T_X = range(9)


def _gen(seed: int, layer: int, tensor: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + layer * 1_009 + tensor * 7_919) & 0x7FFF_FFFF_FFFF)
    return g


def _normal(shape, std, gen, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def skew_bias(n_experts: int) -> torch.Tensor:
    """Router bias of the skewed chunk: +1.9375 on experts 16j (16 hot ones),
    -64 on experts 16j+r for j < 15 and r in 1..4 (60 that receive no row),
    0 elsewhere. All values are exact in bf16 and fp32."""
    b = torch.zeros(n_experts, dtype=torch.float32)
    for j in range(n_experts // 16):
        b[16 * j] = 1.9375
        if j < 15:
            for r in range(1, 5):
                b[16 * j + r] = -64.0
    return b


def concentrated_bias(n_experts: int) -> torch.Tensor:
    """Router bias that sends every row to the 16 experts 16j: -64 on every
    other expert, so each of the 16 receives about T/2 rows of a chunk and the
    expert GEMMs have enough rows per weight tile to be bound by the matrix
    cores rather than by HBM."""
    b = torch.full((n_experts,), -64.0, dtype=torch.float32)
    b[::16] = 0.0
    return b


def fp8_block_weights(n_experts, rows, cols, std, gen, device, chunk_experts=8):
    """Synthetic block-FP8 matrices [E, rows, cols] (e4m3 codes as uint8) and
    their fp32 scales [E, rows/128, cols/128] (dequantised w = code * scale)."""
    assert rows % GROUP == 0 and cols % GROUP == 0
    codes = torch.empty((n_experts, rows, cols), dtype=torch.uint8, device=device)
    scales = torch.empty((n_experts, rows // GROUP, cols // GROUP), dtype=torch.float32,
                         device=device)
    for e0 in range(0, n_experts, chunk_experts):
        e1 = min(n_experts, e0 + chunk_experts)
        w = _normal((e1 - e0, rows, cols), std, gen, device)
        blk = w.view(e1 - e0, rows // GROUP, GROUP, cols // GROUP, GROUP)
        amax = blk.abs().amax(dim=(2, 4))
        s = amax / 448.0
        s = torch.where(s > 0, s, torch.ones_like(s))
        r = (blk / s[:, :, None, :, None]).clamp(-448.0, 448.0)
        codes[e0:e1] = r.to(torch.float8_e4m3fn).view(torch.uint8).view(e1 - e0, rows, cols)
        scales[e0:e1] = s
    return codes, scales


@dataclass
class LayerWeights:
    shape: LayerShape
    router_w: torch.Tensor            # bf16 [E, H]
    router_bias: Optional[torch.Tensor]  # fp32 [E] or None
    w_gate: torch.Tensor              # uint8 e4m3 [E, I, H]
    s_gate: torch.Tensor              # fp32 [E, I/128, H/128]
    w_up: torch.Tensor
    s_up: torch.Tensor
    w_down: torch.Tensor              # uint8 e4m3 [E, H, I]
    s_down: torch.Tensor              # fp32 [E, H/128, I/128]
    sh_gate: torch.Tensor             # bf16 [Is, H]
    sh_up: torch.Tensor               # bf16 [Is, H]
    sh_down: torch.Tensor             # bf16 [H, Is]
    sh_gate_w: torch.Tensor           # bf16 [H]
    # block-FP8 shared expert (make_layer(shared_fp8=True)): sh_gate, sh_up
    # and sh_down then hold e4m3 codes [Is, H], [Is, H], [H, Is] and these
    # their fp32 scales [Is/128, H/128], [Is/128, H/128], [H/128, Is/128]
    sh_s_gate: Optional[torch.Tensor] = None
    sh_s_up: Optional[torch.Tensor] = None
    sh_s_down: Optional[torch.Tensor] = None
    extra: Dict[str, torch.Tensor] = field(default_factory=dict)

    def tensors(self) -> Dict[str, Optional[torch.Tensor]]:
        return {k: getattr(self, k) for k in (
            "router_w", "router_bias", "w_gate", "s_gate", "w_up", "s_up", "w_down",
            "s_down", "sh_gate", "sh_up", "sh_down", "sh_gate_w", "sh_s_gate", "sh_s_up",
            "sh_s_down")}

    def to(self, device) -> "LayerWeights":
        kw = {k: (None if v is None else v.to(device)) for k, v in self.tensors().items()}
        return LayerWeights(shape=self.shape, **kw)


def make_router(shape: LayerShape, seed: int = 0, layer: int = 0, device="cpu",
                std: float = 0.02) -> torch.Tensor:
    """Router weight bf16 [E, H] ~ N(0, std^2) (the same stream make_layer uses)."""
    dev = torch.device(device)
    return _normal((shape.n_experts, shape.hidden), std, _gen(seed, layer, _T_ROUTER, dev),
                   dev).to(torch.bfloat16)


def make_layer(shape: LayerShape, seed: int = 0, layer: int = 0, device="cpu",
               skewed: bool = False, std: float = 0.02,
               shared_fp8: bool = False) -> LayerWeights:
    E, H, I, Is = shape.n_experts, shape.hidden, shape.inter, shape.shared_inter
    dev = torch.device(device)
    g = lambda t: _gen(seed, layer, t, dev)  # noqa: E731
    router_w = make_router(shape, seed, layer, dev, std)
    w_gate, s_gate = fp8_block_weights(E, I, H, std, g(_T_GATE), dev)
    w_up, s_up = fp8_block_weights(E, I, H, std, g(_T_UP), dev)
    w_down, s_down = fp8_block_weights(E, H, I, std, g(_T_DOWN), dev)
    sh_gate = _normal((Is, H), std, g(_T_SH_GATE), dev).to(torch.bfloat16)
    sh_up = _normal((Is, H), std, g(_T_SH_UP), dev).to(torch.bfloat16)
    sh_down = _normal((H, Is), std, g(_T_SH_DOWN), dev).to(torch.bfloat16)
    sh_gate_w = _normal((H,), std, g(_T_SH_GW), dev).to(torch.bfloat16)
    bias = skew_bias(E).to(dev) if skewed else None
    if shared_fp8:
        # the same recipe as the routed experts, one expert, from the shared
        # matrices' own streams
        (sg, ssg), (su, ssu), (sd, ssd) = (
            fp8_block_weights(1, r, c, std, g(t), dev)
            for r, c, t in ((Is, H, _T_SH_GATE), (Is, H, _T_SH_UP), (H, Is, _T_SH_DOWN)))
        return LayerWeights(shape, router_w, bias, w_gate, s_gate, w_up, s_up, w_down, s_down,
                            sg[0], su[0], sd[0], sh_gate_w, ssg[0], ssu[0], ssd[0])
    return LayerWeights(shape, router_w, bias, w_gate, s_gate, w_up, s_up, w_down, s_down,
                        sh_gate, sh_up, sh_down, sh_gate_w)


def make_x(shape: LayerShape, rows: int, seed: int = 0, layer: int = 0, device="cpu",
           std: float = 1.0) -> torch.Tensor:
    """Activation rows x ~ N(0, std^2), rounded to bf16: [rows, H]."""
    dev = torch.device(device)
    return _normal((rows, shape.hidden), std, _gen(seed, layer, _T_X, dev), dev).to(
        torch.bfloat16)
