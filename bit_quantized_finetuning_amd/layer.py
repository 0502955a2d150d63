"""torch.autograd wrapper and module for the frozen-NF4 linear layer with a LoRA adapter.

    h = dequant(W_NF4, c_block) x + (alpha/r) B A x

("QLoRA는 어떻게 65B 모델을 GPU 한 장에 올렸나", section "QLoRA의 수식".) The base
weight is frozen: it has no gradient ("명제 1" on the same page; "48GB GPU
Fine-Tuning a 65B Model", section "QLoRA Puts the Two Methods in Different
Places": gradients pass through the restored W to A and B). Every step runs in
the HIP library through the C-ABI binding; this file only marshals tensors.

The forward saves u = x A^T (T x r float32) for the backward's dB, so u is not
recomputed. With a frozen A (LoRA-FA: "8GB, 12GB, 16GB, 24GB GPU에서 몇 B
모델까지 LoRA 학습이 될까", section "LoRA 변형을 바꿔도 답이 같은 이유" -- the
layer input is not kept) the input x is not saved either: dX needs only dY,
and dB only u.
"""

from __future__ import annotations

import torch

from . import qlora as q


class QLoRALinearFunction(torch.autograd.Function):
    """x [T, d_in] bf16, A [r, d_in] bf16, B [d_out, r] bf16 -> h [T, d_out] bf16."""

    @staticmethod
    def forward(ctx, x, A, B, w: q.NF4Weight, alpha: float):
        r = 0 if A is None else A.shape[0]
        h, u = q.qlora_forward(w, x, A, B, alpha, save_u=r > 0)
        keep_x = A is not None and A.requires_grad
        ctx.w, ctx.alpha, ctx.r = w, alpha, r
        ctx.save_for_backward(x if keep_x else None, A, B, u)
        return h

    @staticmethod
    def backward(ctx, dh):
        x, A, B, u = ctx.saved_tensors
        need_dx = ctx.needs_input_grad[0]
        need_dA = ctx.r > 0 and ctx.needs_input_grad[1]
        need_dB = ctx.r > 0 and ctx.needs_input_grad[2]
        dX, dA, dB = q.qlora_backward(ctx.w, x, dh.contiguous(), A, B, ctx.alpha, u_saved=u, need_dx=need_dx,
                                      need_dA=need_dA, need_dB=need_dB)
        # dA, dB come back in float32 (the library's gradient precision); autograd wants the parameters' dtype
        return (dX, None if dA is None else dA.to(A.dtype), None if dB is None else dB.to(B.dtype), None, None)


class QLoRALinear(torch.nn.Module):
    """A frozen NF4 + double-quant weight with a trainable LoRA adapter (bf16 A, B).

    A is initialised like the pages' adapters (small random values) and B to zero, so that the adapted
    layer starts as the quantized base layer ("48GB GPU Fine-Tuning a 65B Model", section "LoRA
    Freezes the Original Weights...": B = 0 at the start leaves the model unchanged).
    """

    def __init__(self, weight: torch.Tensor, r: int = 8, alpha: float = 16.0, freeze_A: bool = False,
                 generator: torch.Generator | None = None, double_quant: bool = True):
        super().__init__()
        if weight.dim() != 2:
            raise ValueError("weight must be [d_out, d_in]")
        d_out, d_in = weight.shape
        # double_quant=False keeps the float32 absmax of every block (4.5 bits per weight)
        self.w = q.qlora_quantize(weight.contiguous(), double_quant=double_quant)
        # the quantized buffers are frozen state, not parameters
        self.register_buffer("codes", self.w.codes, persistent=True)
        self.register_buffer("qscale", self.w.qscale, persistent=True)
        self.register_buffer("smax", self.w.smax, persistent=True)
        self.d_out, self.d_in, self.r, self.alpha = d_out, d_in, r, float(alpha)
        if r > 0:
            A = torch.randn(r, d_in, device=weight.device, generator=generator) * 0.02
            self.A = torch.nn.Parameter(A.to(torch.bfloat16), requires_grad=not freeze_A)
            self.B = torch.nn.Parameter(torch.zeros(d_out, r, dtype=torch.bfloat16, device=weight.device))
        else:
            self.A = self.B = None

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.d_in).to(torch.bfloat16).contiguous()
        h = QLoRALinearFunction.apply(x2, self.A, self.B, self.w, self.alpha)
        return h.reshape(*lead, self.d_out)

    @torch.no_grad()
    def merged_weight(self) -> torch.Tensor:
        """bf16 [d_out, d_in] = bf16(W_hat + (alpha/r) B A), for export."""
        return q.qlora_merge(self.w, self.A, self.B, self.alpha)
