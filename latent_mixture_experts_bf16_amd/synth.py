"""Seeded synthetic workloads for the latent mixture-of-experts decode layer.

This module only draws numbers and lays them out. It holds none of the layer's
arithmetic: no dot product, no routing, no rounding point of the method. Both the
HIP path (through the binding) and the CPU oracle consume what it produces, and
it is the only module the two share.

Workload shapes come from the layer the pages describe (TensorFold pull request
1038, «What's in it»: hidden 4096, a 1024-wide latent, expert counts 240 to 496
per Puzzle layer, top-k 9) and from the non-latent family router of TensorFold
pull request 1295 («What this changes», family kernels bullet: fp16 activations,
fp32 router, sigmoid top-8). Value distributions:

* activations N(0, 1); gate, latent projections and shared expert N(0, 0.02);
  correction bias fp32 N(0, 0.01);
* routed experts are 4-bit affine with groups of 64 along the input dimension:
  codes uniform in 0..15, bf16 scale U(0.005, 0.02), bias = -8 * scale; the other widths
  of the affine family (2, 3, 5, 6, 8 bits; groups of 32 or 128) take codes uniform in
  0 .. 2^b - 1, scale U(0.005, 0.02) * 8 / 2^(b-1) and bias = -2^(b-1) * scale.

Draw order inside one layer (tensor-major, one generator per layer):
x, Wg, c, W1, W2, up codes, up scales, down codes, down scales, Su, Sd.
Normals are drawn in float64, cast to float32, then to bf16 (round to nearest
even) or fp16. Codes are uniform uint32 words holding 8 uniform nibbles, the
lowest nibble being the lowest input index.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

# dtype tags shared by the C-ABI header and the oracle (plain integers, no logic)
BF16, F16, F32 = 1, 2, 3


@dataclasses.dataclass(frozen=True)
class LayerDims:
    """Sizes and switches of one MoE layer (all integers / flags, no arithmetic)."""
    hidden: int
    latent: int            # 0 = non-latent: experts act on the hidden vector
    n_experts: int
    n_group: int
    topk_group: int
    top_k: int
    expert_inter: int
    shared_inter: int      # 0 = no shared expert
    group_size: int = 64
    act_dtype: int = BF16  # BF16 or F16
    router_dtype: int = BF16  # BF16 (bf16 gemv, bf16 logits) or F32
    has_bias: bool = True
    norm_topk: bool = True
    routed_scaling: float = 2.5
    quant_bits: int = 4    # routed expert code width: 2, 3, 4, 5, 6 or 8

    @property
    def expert_dim(self) -> int:
        """Input width of the routed experts (latent, or hidden when non-latent)."""
        return self.latent if self.latent else self.hidden


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    rows: int
    layers: List[LayerDims]
    weight_seeds: List[int]
    input_seeds: List[Optional[int]]  # None: x is the first draw of the weight stream


def _bolt(E: int) -> LayerDims:
    return LayerDims(hidden=4096, latent=1024, n_experts=E, n_group=8, topk_group=4,
                     top_k=9, expert_inter=2048, shared_inter=4096)


WORKLOADS: Dict[int, Workload] = {
    0: Workload("tiny-latent-E16-rows1", 1,
                [LayerDims(hidden=512, latent=128, n_experts=16, n_group=4, topk_group=2,
                           top_k=2, expert_inter=256, shared_inter=512)],
                [1000], [None]),
    1: Workload("bolt-latent-E240-rows1", 1, [_bolt(240)], [1001], [None]),
    2: Workload("bolt-latent-E496-rows16", 16, [_bolt(496)], [1002], [None]),
    3: Workload("nonlatent-fp16-E256-rows4", 4,
                [LayerDims(hidden=5120, latent=0, n_experts=256, n_group=1, topk_group=1,
                           top_k=8, expert_inter=1536, shared_inter=0, act_dtype=F16,
                           router_dtype=F32, has_bias=False, routed_scaling=1.0)],
                [1003], [None]),
    4: Workload("bolt-latent-stack8-rows64", 64,
                [_bolt(E) for E in (240, 304, 368, 432, 496, 240, 304, 368)],
                [1040 + l for l in range(8)], [1050 + l for l in range(8)]),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    v = rng.standard_normal(size=shape) * std          # float64
    return f32_to_bf16_bits(v.astype(np.float32))


def _normal_act(rng: np.random.Generator, shape, act_dtype: int) -> np.ndarray:
    v = rng.standard_normal(size=shape).astype(np.float32)
    if act_dtype == F16:
        return v.astype(np.float16).view(np.uint16)
    return f32_to_bf16_bits(v)


def make_layer(dims: LayerDims, rows: int, weight_seed: int,
               input_seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw one layer's weights and a [rows][hidden] input.

    Returns host arrays: 16-bit values as uint16 bit patterns, codes as uint32
    words, fp32 arrays as float32. Shapes:
      x [rows][H]; gate_w [E][H] (bf16, or fp32 when router_dtype == F32);
      corr_bias [E] fp32 (absent when has_bias is False);
      fc1_w [L][H], fc2_w [H][L] bf16 (absent when non-latent);
      up_q [E][I][D b/32] u32, up_scales/up_biases [E][I][D/gs] bf16;
      down_q [E][D][I b/32] u32, down_scales/down_biases [E][D][I/gs] bf16
      (b = quant_bits, gs = group_size);
      shared_up [SI][H], shared_down [H][SI] bf16 (absent when SI == 0).
    """
    H, L, E, I, SI = dims.hidden, dims.latent, dims.n_experts, dims.expert_inter, dims.shared_inter
    D = dims.expert_dim
    gs = dims.group_size
    rng = np.random.default_rng(weight_seed)
    out: Dict[str, np.ndarray] = {}
    if input_seed is None:
        out["x"] = _normal_act(rng, (rows, H), dims.act_dtype)
    else:
        out["x"] = _normal_act(np.random.default_rng(input_seed), (rows, H), dims.act_dtype)
    if dims.router_dtype == F32:
        out["gate_w"] = (rng.standard_normal(size=(E, H)) * 0.02).astype(np.float32)
    else:
        out["gate_w"] = _normal_bf16(rng, (E, H), 0.02)
    if dims.has_bias:
        out["corr_bias"] = (rng.standard_normal(size=E) * 0.01).astype(np.float32)
    if L:
        out["fc1_w"] = _normal_bf16(rng, (L, H), 0.02)
        out["fc2_w"] = _normal_bf16(rng, (H, L), 0.02)
    # b-bit codes as a uniform bit string (every code uniform in 0 .. 2^b - 1); scales drawn
    # as U(0.005, 0.02) * 8 / 2^(b-1), so that every width spans the weights of the 4-bit layer
    nb = dims.quant_bits
    half = 2 ** (nb - 1)
    out["up_q"] = rng.integers(0, 2**32, size=(E, I, D * nb // 32), dtype=np.uint32)
    s = f32_to_bf16_bits((rng.uniform(0.005, 0.02, size=(E, I, D // gs)) * (8.0 / half)).astype(np.float32))
    out["up_scales"] = s
    out["down_q"] = rng.integers(0, 2**32, size=(E, D, I * nb // 32), dtype=np.uint32)
    s2 = f32_to_bf16_bits((rng.uniform(0.005, 0.02, size=(E, D, I // gs)) * (8.0 / half)).astype(np.float32))
    out["down_scales"] = s2
    # bias = -2^(b-1) * scale: exact in bf16 (a power-of-two multiple, then a sign flip)
    out["up_biases"] = f32_to_bf16_bits(-float(half) * bf16_bits_to_f32(s))
    out["down_biases"] = f32_to_bf16_bits(-float(half) * bf16_bits_to_f32(s2))
    if SI:
        out["shared_up"] = _normal_bf16(rng, (SI, H), 0.02)
        out["shared_down"] = _normal_bf16(rng, (H, SI), 0.02)
    return out


def workload_layers(cfg_id: int, instance: int = 0, rows: Optional[int] = None,
                    layers: Optional[List[int]] = None):
    """Yield (dims, arrays) for each layer of workload `cfg_id`.

    `instance` > 0 draws an independent copy (weight seed + 100 * instance) used to
    rotate distinct weights through HBM when timing; instance 0 is the parity copy.
    """
    wl = WORKLOADS[cfg_id]
    r = wl.rows if rows is None else rows
    for l, dims in enumerate(wl.layers):
        if layers is not None and l not in layers:
            continue
        ws = wl.weight_seeds[l] + 100 * instance
        xs = wl.input_seeds[l]
        if xs is not None:
            xs = xs + 100 * instance
        yield dims, make_layer(dims, r, ws, xs)


def make_lm_head(K: int, N: int, rows: int, seed: int) -> Dict[str, np.ndarray]:
    """A bf16 lm_head and its input rows: W [N][K] N(0, 0.02), x [rows][K] N(0, 1), drawn as
    float32 normals (in blocks of rows, so that the 1 GiB matrix of K = 4096, N = 131072
    needs no float64 copy) and rounded to bf16 (nearest even). x is drawn first."""
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal(size=(rows, K), dtype=np.float32))
    W = np.empty((N, K), np.uint16)
    step = 4096
    for n in range(0, N, step):
        m = min(step, N - n)
        W[n:n + m] = f32_to_bf16_bits(rng.standard_normal(size=(m, K), dtype=np.float32) * np.float32(0.02))
    return {"x": x, "w": W}
