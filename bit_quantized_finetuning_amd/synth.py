"""Seeded synthetic inputs for the QLoRA linear layer.

This module draws random numbers and rounds them to the storage dtype; it holds
none of the method's arithmetic. Both the tests (for the HIP path and for the
CPU oracle) and the benchmark take their inputs from here, so the two sides see
identical bytes.

Recipe (shapes from the LLaMA/Qwen-style projections the workloads name):
  * RNG: numpy.random.default_rng([seed, config, projection, tensor]) with
    tensor ids W=0, A=1, B=2, x=3, dY=4;
  * W  ~ N(0, 0.02^2) float32 (bf16-rounded where the workload loads bf16 weights);
  * A, B ~ N(0, 0.02^2) rounded to bf16;
  * x, dY ~ N(0, 1) rounded to bf16.
Rounding to bf16 uses torch's own float32 -> bfloat16 conversion.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

T_W, T_A, T_B, T_X, T_DY = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Projection:
    name: str
    d_out: int
    d_in: int
    r: int           # LoRA rank, 0 = frozen projection without adapter
    alpha: float
    # Stacked projections (one call for several projections of one input): the row range of each adapted
    # projection; adapter k then owns B's rows in b_rows[k] and columns k r/len(b_rows) .. (k+1) r/len(b_rows),
    # and B is zero elsewhere. Empty: one projection, B dense.
    b_rows: tuple = ()


@dataclass(frozen=True)
class Workload:
    key: str
    description: str
    projections: tuple
    tokens: tuple     # token counts T exercised
    backward: bool
    weight_dtype: str  # "f32" or "bf16"
    layers: int = 1


WORKLOADS = {
    "linear1024": Workload("linear1024", "single linear 1024x1024, LoRA r=8 alpha=16, 16 tokens, fwd+bwd",
                   (Projection("linear", 1024, 1024, 8, 16.0),), (16,), True, "f32"),
    "llama7b_skinny": Workload("llama7b_skinny", "LLaMA-7B projections 4096x4096 and 11008x4096, LoRA r=64 alpha=16, "
                   "1/4/16 tokens, forward",
                   (Projection("q_proj", 4096, 4096, 64, 16.0),
                    Projection("up_proj", 11008, 4096, 64, 16.0)), (1, 4, 16), False, "f32"),
    "13b_4096tok": Workload("13b_4096tok", "13B projections 5120x5120 and 13824x5120, LoRA r=64 alpha=16, "
                   "4096 tokens (8x512), fwd+bwd",
                   (Projection("q_proj", 5120, 5120, 64, 16.0),
                    Projection("up_proj", 13824, 5120, 64, 16.0)), (4096,), True, "f32"),
    "65b_layer": Workload("65b_layer", "65B decoder layer, hidden 8192, MLP 22016, LoRA r=64 alpha=16 on all "
                   "projections, 4096 tokens, fwd+bwd",
                   (Projection("q_proj", 8192, 8192, 64, 16.0),
                    Projection("k_proj", 8192, 8192, 64, 16.0),
                    Projection("v_proj", 8192, 8192, 64, 16.0),
                    Projection("o_proj", 8192, 8192, 64, 16.0),
                    Projection("gate_proj", 22016, 8192, 64, 16.0),
                    Projection("up_proj", 22016, 8192, 64, 16.0),
                    Projection("down_proj", 8192, 22016, 64, 16.0)), (4096,), True, "f32"),
    # The same 65B layer as the layer driver runs it: the projections of one input stacked into one call each,
    # q/k/v (24576 x 8192, three rank-64 adapters as a block-diagonal rank-192 pair, alpha tripled so the scale
    # stays 16/64) and gate/up (44032 x 8192, two rank-64 adapters). The quantized storage of a stacked weight
    # is that of its parts laid end to end (every part holds a whole number of 256-block groups).
    "65b_layer_fused": Workload("65b_layer_fused", "65B decoder layer, hidden 8192, MLP 22016, LoRA r=64 alpha=16 "
                   "on all projections, 4096 tokens, fwd+bwd, q/k/v and gate/up each as one stacked call",
                   (Projection("qkv_proj", 24576, 8192, 192, 48.0, b_rows=((0, 8192), (8192, 16384), (16384, 24576))),
                    Projection("o_proj", 8192, 8192, 64, 16.0),
                    Projection("gate_up_proj", 44032, 8192, 128, 32.0, b_rows=((0, 22016), (22016, 44032))),
                    Projection("down_proj", 8192, 22016, 64, 16.0)), (4096,), True, "f32"),
    # The weight-streaming regime on the 65B layer's larger weights (34-93 MB per call instead of 9-23 MB):
    # how close the T <= 16 kernel gets to HBM once the stream is long against its fixed latency.
    "65b_skinny": Workload("65b_skinny", "65B decoder-layer projections 8192x8192, 22016x8192 and 8192x22016, "
                   "LoRA r=64 alpha=16, 1/16 tokens, forward",
                   (Projection("q_proj", 8192, 8192, 64, 16.0),
                    Projection("gate_proj", 22016, 8192, 64, 16.0),
                    Projection("down_proj", 8192, 22016, 64, 16.0)), (1, 16), False, "f32"),
    # The same layer with the projections of one input stacked into one call each: q/k/v (7168 x 5120, the
    # q and v adapters as a rank-16 block-diagonal pair, alpha doubled so the scale stays 16/8) and gate/up.
    "14b_stack_fused": Workload("14b_stack_fused", "14B-style stack, hidden 5120, MLP 17408, 40 layers, LoRA r=8 "
                   "alpha=16 on q/v, 2048 tokens, fwd+bwd, q/k/v and gate/up each as one stacked call",
                   (Projection("qkv_proj", 7168, 5120, 16, 32.0, b_rows=((0, 5120), (6144, 7168))),
                    Projection("o_proj", 5120, 5120, 0, 16.0),
                    Projection("gate_up_proj", 34816, 5120, 0, 16.0),
                    Projection("down_proj", 5120, 17408, 0, 16.0)), (2048,), True, "bf16", layers=40),
    # 14B-style stack: k/v are 1024x5120 (8 KV heads x 128); LoRA r=8 on q and v only.
    "14b_stack": Workload("14b_stack", "14B-style stack, hidden 5120, MLP 17408, 40 layers, LoRA r=8 alpha=16 "
                   "on q/v, 2048 tokens, fwd+bwd",
                   (Projection("q_proj", 5120, 5120, 8, 16.0),
                    Projection("k_proj", 1024, 5120, 0, 16.0),
                    Projection("v_proj", 1024, 5120, 8, 16.0),
                    Projection("o_proj", 5120, 5120, 0, 16.0),
                    Projection("gate_proj", 17408, 5120, 0, 16.0),
                    Projection("up_proj", 17408, 5120, 0, 16.0),
                    Projection("down_proj", 5120, 17408, 0, 16.0)), (2048,), True, "bf16", layers=40),
}
# second component of every RNG seed list, one per workload
WORKLOAD_SEED = {"linear1024": 1, "llama7b_skinny": 2, "13b_4096tok": 3, "65b_layer": 4, "14b_stack": 5,
                 "14b_stack_fused": 6, "65b_skinny": 7, "65b_layer_fused": 8}


def rng(config: int, projection: int, tensor: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, config, projection, tensor])


def to_bf16(a: np.ndarray):
    """Round float32 -> bf16 with torch; returns (values as float32, uint16 bit patterns)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.float().numpy(), bits


def normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def weight(config: int, projection: int, d_out: int, d_in: int, dtype: str = "f32", seed: int = 0):
    """W ~ N(0, 0.02^2), float32; bf16-rounded (still returned as float32 values) when dtype == 'bf16'."""
    w = normal(rng(config, projection, T_W, seed), (d_out, d_in), 0.02)
    if dtype == "bf16":
        w, _ = to_bf16(w)
    return w


def adapters(config: int, projection: int, d_out: int, d_in: int, r: int, seed: int = 0):
    """A [r, d_in], B [d_out, r] ~ N(0, 0.02^2) in bf16: ((A_val, A_bits), (B_val, B_bits))."""
    A = to_bf16(normal(rng(config, projection, T_A, seed), (r, d_in), 0.02))
    B = to_bf16(normal(rng(config, projection, T_B, seed), (d_out, r), 0.02))
    return A, B


def tokens(config: int, projection: int, T: int, d_in: int, seed: int = 0):
    """x [T, d_in] ~ N(0, 1) in bf16: (values, bits)."""
    return to_bf16(normal(rng(config, projection, T_X, seed), (T, d_in), 1.0))


def upstream_grad(config: int, projection: int, T: int, d_out: int, seed: int = 0):
    """dY [T, d_out] ~ N(0, 1) in bf16: (values, bits)."""
    return to_bf16(normal(rng(config, projection, T_DY, seed), (T, d_out), 1.0))


# The 14B-style stack as chained layers: 13.2 G weights are too many to draw on the host, so they are drawn on the
# device with torch's seeded generator, one seed per layer (the same call on any MI355X gives the same bytes).
STACK_SEED = 8
STACK_SHAPES = {"q": (5120, 5120), "k": (1024, 5120), "v": (1024, 5120), "o": (5120, 5120), "gate": (17408, 5120),
                "up": (17408, 5120), "down": (5120, 17408)}


def stack_layer_weights(layer: int, device, shapes=None, seed: int = 0) -> dict:
    """One layer's bf16 weights {name: [d_out, d_in]} ~ N(0, 0.02^2), drawn on `device` in the order q, k, v, o,
    gate, up, down from torch.Generator(seed = 1_000_000 * (seed + 1) + 1000 * STACK_SEED + layer)."""
    shapes = STACK_SHAPES if shapes is None else shapes
    gen = torch.Generator(device=device)
    gen.manual_seed(1_000_000 * (seed + 1) + 1000 * STACK_SEED + layer)
    out = {}
    for name, (d_out, d_in) in shapes.items():
        w = torch.empty(d_out, d_in, dtype=torch.float32, device=device)
        w.normal_(0.0, 0.02, generator=gen)
        out[name] = w.to(torch.bfloat16)
        del w
    return out


def stack_adapter_init(layer: int, device, seed: int = 0) -> torch.Generator:
    """The generator a stack layer draws its adapters' A from (and, for checks, B)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(1_000_000 * (seed + 1) + 1000 * STACK_SEED + 500 + layer)
    return gen
