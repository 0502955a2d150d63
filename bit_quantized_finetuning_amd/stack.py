"""A stack of decoder layers built from the QLoRA projections: the chained-layer setting of the pages' 14B runs.

"8GB, 12GB, 16GB, 24GB GPU에서 몇 B 모델까지 LoRA 학습이 될까", section "무엇을 돌렸나": a 14B model (hidden
5120, MLP 17408, 40 layers) with 4-bit NF4 + double-quant base weights, LoRA r = 8, alpha = 16 on q_proj and
v_proj only, bf16 compute, gradient checkpointing, one sequence of 2048 tokens.

Each layer holds its seven projections as the library's frozen NF4 weights: q/k/v stacked into one call that
reads the normalized input once (q and v adapted), o, gate/up stacked into one call, and down. k and v are
1024 x 5120 (8 KV heads of 128 for 40 query heads). Everything between the projections is plain torch glue and
stands in for parts of the model that are not on this path:
  * RMS normalization (no weight) before q/k/v and before gate/up;
  * attention is replaced by a gate that mixes q with k and v expanded to the query heads,
    a = q * sigmoid(k) + v, so that every projection's output reaches the loss;
  * the MLP activation is SiLU(gate) * up; residual adds around both halves.
With checkpoint=True each layer keeps only its input and runs its forward again in the backward
(torch.utils.checkpoint, non-reentrant).

Weights come from the seeded device generator of the synthetic-input module, one seed per layer, so that a
layer's weights can be drawn again to check it.
"""

from __future__ import annotations

import torch
import torch.nn.functional as F
from torch.utils.checkpoint import checkpoint

from . import synth
from .layer import QLoRAFusedLinear, QLoRALinear

HEAD = 128


def rms_norm(x: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    """x / sqrt(mean(x^2) + eps) over the last dimension, bf16 in and out (torch's fused norm)."""
    return F.rms_norm(x, (x.shape[-1],), eps=eps)


class DecoderProjections(torch.nn.Module):
    """One decoder layer of projections (see the module docstring); `weights` maps q, k, v, o, gate, up, down to
    bf16 [d_out, d_in] tensors."""

    def __init__(self, weights: dict, r: int = 8, alpha: float = 16.0, generator: torch.Generator | None = None,
                 head: int = HEAD):
        super().__init__()
        self.hidden, self.kv, self.head = weights["q"].shape[0], weights["k"].shape[0], head
        if self.hidden % head or self.kv % head or self.hidden % self.kv:
            raise ValueError("q and k/v widths must be multiples of the head width, q's of k's")
        self.qkv = QLoRAFusedLinear([weights["q"], weights["k"], weights["v"]], r=r, alpha=alpha,
                                    adapted=[True, False, True], generator=generator)
        self.o = QLoRALinear(weights["o"], r=0)
        self.gate_up = QLoRAFusedLinear([weights["gate"], weights["up"]], r=0)
        self.down = QLoRALinear(weights["down"], r=0)

    def _heads(self, t: torch.Tensor, rep: int) -> torch.Tensor:
        """[T, n * head] -> [T, kv heads, rep, head] (a view; k and v broadcast over the query heads they serve)."""
        return t.view(t.shape[0], self.kv // self.head, rep, self.head)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        q, k, v = self.qkv(rms_norm(x))
        rep = self.hidden // self.kv  # query heads per KV head
        # a = q * sigmoid(k) + v with k and v broadcast to the query heads (one bf16 rounding, float32 inside)
        a = torch.addcmul(self._heads(v, 1), self._heads(q, rep), torch.sigmoid(self._heads(k, 1)))
        x1 = x + self.o(a.reshape(x.shape[0], self.hidden))
        g, u = self.gate_up(rms_norm(x1))
        return x1 + self.down(F.silu(g) * u)


class DecoderStack(torch.nn.Module):
    """`layers` decoder layers of projections; layer i's weights are synth.stack_layer_weights(i) (shapes default
    to the 14B-style layer) and its adapters' A are drawn from synth.stack_adapter_init(i) (B starts at zero)."""

    def __init__(self, layers: int = 40, shapes: dict | None = None, r: int = 8, alpha: float = 16.0,
                 seed: int = 0, device="cuda", checkpoint: bool = True, head: int = HEAD):
        super().__init__()
        self.shapes = dict(synth.STACK_SHAPES if shapes is None else shapes)
        self.seed = seed
        self.use_checkpoint = checkpoint
        self.layers = torch.nn.ModuleList()
        for i in range(layers):
            ws = synth.stack_layer_weights(i, device, self.shapes, seed)
            gen = synth.stack_adapter_init(i, device, seed)
            self.layers.append(DecoderProjections(ws, r=r, alpha=alpha, generator=gen, head=head))
            del ws

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        for layer in self.layers:
            if self.use_checkpoint and torch.is_grad_enabled():
                x = checkpoint(layer, x, use_reentrant=False)
            else:
                x = layer(x)
        return x
