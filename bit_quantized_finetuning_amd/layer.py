"""torch.autograd wrapper and module for the frozen-NF4 linear layer with a LoRA adapter.

    h = dequant(W_NF4, c_block) x + (alpha/r) B A x

("QLoRA는 어떻게 65B 모델을 GPU 한 장에 올렸나", section "QLoRA의 수식".) The base
weight is frozen: it has no gradient ("명제 1" on the same page; "48GB GPU
Fine-Tuning a 65B Model", section "QLoRA Puts the Two Methods in Different
Places": gradients pass through the restored W to A and B). Every step runs in
the HIP library through the C-ABI binding; this file only marshals tensors.

The forward saves u = x A^T (T x r float32) for the backward's dB, so u is not
recomputed; with recompute_u the layer keeps only x and the backward forms u
again (T x r float32 less memory per layer, one more pass over x).

The library returns dA and dB in float32. Autograd hands the parameters their
gradients in the parameters' dtype (bf16), so the layers also keep the float32
gradients on each adapter parameter, as `param.grad_fp32` (summed over
backward passes while `param.grad` accumulates, started afresh when
`param.grad` is None); PagedAdamW steps on those.

The modules compute in bf16 only: a dtype cast of a module (`.to(dtype)`,
`.half()`, `.float()`) leaves its quantized buffers and adapter parameters as
they are, and only a device move applies to them. With a frozen A (LoRA-FA: "8GB, 12GB, 16GB, 24GB GPU에서 몇 B
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
    def forward(ctx, x, A, B, w: q.NF4Weight, alpha: float, recompute_u: bool = False, grad_sink=None):
        r = 0 if A is None else A.shape[0]
        keep_u = r > 0 and not recompute_u
        h, u = q.qlora_forward(w, x, A, B, alpha, save_u=keep_u)
        keep_x = A is not None and (A.requires_grad or not keep_u)
        ctx.w, ctx.alpha, ctx.r, ctx.grad_sink = w, alpha, r, grad_sink
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
        if ctx.grad_sink is not None:
            ctx.grad_sink(dA, dB)  # the float32 gradients, for the optimizer
        # dA, dB come back in float32 (the library's gradient precision); autograd wants the parameters' dtype
        return (dX, None if dA is None else dA.to(A.dtype), None if dB is None else dB.to(B.dtype), None, None, None,
                None)


def _deposit_fp32(p: torch.nn.Parameter, g: torch.Tensor):
    """Keep the float32 gradient beside p.grad: summed while p.grad accumulates, restarted when it is None."""
    prev = getattr(p, "grad_fp32", None)
    if p.grad is None or prev is None:
        p.grad_fp32 = g.detach().clone()
    else:
        prev.add_(g)


class _Bf16Module(torch.nn.Module):
    """Dtype casts leave the quantized storage and the bf16 adapters as they are; device moves apply."""

    def _apply(self, fn, recurse=True):
        def keep_dtype(t):
            moved = fn(t)
            return moved if moved.dtype == t.dtype else t.to(moved.device)

        return super()._apply(keep_dtype, recurse)

    @property
    def w(self) -> q.NF4Weight:
        """The quantized weight as the library takes it, built from the registered buffers (so it follows
        device moves and load_state_dict)."""
        return q.NF4Weight(self.d_w_out, self.d_in, self.codes, self.qscale, self.smax)


class QLoRALinear(_Bf16Module):
    """A frozen NF4 + double-quant weight with a trainable LoRA adapter (bf16 A, B).

    A is initialised like the pages' adapters (small random values) and B to zero, so that the adapted
    layer starts as the quantized base layer ("48GB GPU Fine-Tuning a 65B Model", section "LoRA
    Freezes the Original Weights...": B = 0 at the start leaves the model unchanged).
    """

    def __init__(self, weight: torch.Tensor, r: int = 8, alpha: float = 16.0, freeze_A: bool = False,
                 generator: torch.Generator | None = None, double_quant: bool = True, recompute_u: bool = False):
        super().__init__()
        if weight.dim() != 2:
            raise ValueError("weight must be [d_out, d_in]")
        d_out, d_in = weight.shape
        # double_quant=False keeps the float32 absmax of every block (4.5 bits per weight)
        w = q.qlora_quantize(weight.contiguous(), double_quant=double_quant)
        # the quantized buffers are frozen state, not parameters
        self.register_buffer("codes", w.codes, persistent=True)
        self.register_buffer("qscale", w.qscale, persistent=True)
        self.register_buffer("smax", w.smax, persistent=True)
        self.d_out, self.d_in, self.r, self.alpha = d_out, d_in, r, float(alpha)
        self.d_w_out = d_out
        self.recompute_u = recompute_u
        if r > 0:
            A = torch.randn(r, d_in, device=weight.device, generator=generator) * 0.02
            self.A = torch.nn.Parameter(A.to(torch.bfloat16), requires_grad=not freeze_A)
            self.B = torch.nn.Parameter(torch.zeros(d_out, r, dtype=torch.bfloat16, device=weight.device))
        else:
            self.A = self.B = None

    def _sink(self, dA, dB):
        if dA is not None:
            _deposit_fp32(self.A, dA)
        if dB is not None:
            _deposit_fp32(self.B, dB)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.d_in).to(torch.bfloat16).contiguous()
        h = QLoRALinearFunction.apply(x2, self.A, self.B, self.w, self.alpha, self.recompute_u,
                                      self._sink if self.r > 0 else None)
        return h.reshape(*lead, self.d_out)

    @torch.no_grad()
    def merged_weight(self) -> torch.Tensor:
        """bf16 [d_out, d_in] = bf16(W_hat + (alpha/r) B A), for export."""
        return q.qlora_merge(self.w, self.A, self.B, self.alpha)


class QLoRAFusedLinear(_Bf16Module):
    """Several projections of one input (q/k/v, or gate/up) as one quantized weight and one call.

    The weights are stacked along d_out and quantized as one matrix, so every forward reads x once and streams all
    of them in one launch, and the backward's dX is the sum over the projections in one contraction. With the
    pages' placement of adapters on some projections only ("무엇을 돌렸나" on the GPU-fit page: LoRA on q and v),
    each adapted projection i has its own A_i [r, d_in] and B_i [d_out_i, r]. The call uses their stack
    A = [A_1; A_2; ...] and the block-diagonal B that puts B_i on projection i's rows and adapter i's columns,
    with alpha scaled by the number of adapters so that the scale stays alpha / r: every output row then gets
    exactly its own projection's term (the zero entries add exact zeros), and autograd returns dA_i, dB_i from
    the stacked gradients.

    The stacked quantization equals quantizing each projection alone whenever each projection's block count is a
    multiple of the 256-block group (true for the usual shapes: d_out_i * d_in / 64 % 256 == 0), and always with
    absmax-only storage.
    """

    def __init__(self, weights, r: int = 8, alpha: float = 16.0, adapted=None, double_quant: bool = True,
                 generator: torch.Generator | None = None):
        super().__init__()
        weights = [w.contiguous() for w in weights]
        d_in = weights[0].shape[1]
        if any(w.dim() != 2 or w.shape[1] != d_in for w in weights):
            raise ValueError("all weights must be [d_out_i, d_in] with one d_in")
        self.d_outs = [int(w.shape[0]) for w in weights]
        self.d_in, self.r, self.alpha = d_in, r, float(alpha)
        self.adapted = list(adapted) if adapted is not None else [True] * len(weights)
        if len(self.adapted) != len(weights):
            raise ValueError("one adapted flag per weight")
        n_ad = sum(self.adapted) if r > 0 else 0
        if n_ad * r > q.MAX_RANK:
            raise ValueError(f"{n_ad} adapters of rank {r} exceed the library's rank limit {q.MAX_RANK}")
        w = q.qlora_quantize(torch.cat(weights, 0), double_quant=double_quant)
        self.register_buffer("codes", w.codes, persistent=True)
        self.register_buffer("qscale", w.qscale, persistent=True)
        self.register_buffer("smax", w.smax, persistent=True)
        self.d_w_out = sum(self.d_outs)
        self.A = torch.nn.ParameterList()
        self.B = torch.nn.ParameterList()
        dev = weights[0].device
        for d_out, ad in zip(self.d_outs, self.adapted):
            if ad and r > 0:
                A = torch.randn(r, d_in, device=dev, generator=generator) * 0.02
                self.A.append(torch.nn.Parameter(A.to(torch.bfloat16)))
                self.B.append(torch.nn.Parameter(torch.zeros(d_out, r, dtype=torch.bfloat16, device=dev)))

    def stacked_adapter(self):
        """(A [n r, d_in], block-diagonal B [sum d_out_i, n r]) built from the parameters (differentiable)."""
        if len(self.A) == 0:
            return None, None
        A = torch.cat(list(self.A), 0)
        cols = len(self.A) * self.r
        parts, k = [], 0
        for d_out, ad in zip(self.d_outs, self.adapted):
            if ad and self.r > 0:
                B = self.B[k]
                parts.append(torch.nn.functional.pad(B, (k * self.r, cols - (k + 1) * self.r)))
                k += 1
            else:
                parts.append(torch.zeros(d_out, cols, dtype=torch.bfloat16, device=A.device))
        return A, torch.cat(parts, 0)

    def _sink(self, dA, dB):
        """Split the stacked float32 gradients into the adapters' own (rows of A; B's block on its projection's
        rows and its adapter's columns)."""
        row0, k = 0, 0
        for d_out, ad in zip(self.d_outs, self.adapted):
            if ad and self.r > 0:
                cols = slice(k * self.r, (k + 1) * self.r)
                if dA is not None:
                    _deposit_fp32(self.A[k], dA[cols])
                if dB is not None:
                    _deposit_fp32(self.B[k], dB[row0:row0 + d_out, cols])
                k += 1
            row0 += d_out

    def forward(self, x: torch.Tensor):
        """Returns one output per projection, [..., d_out_i] each (views of the single call's output)."""
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.d_in).to(torch.bfloat16).contiguous()
        A, B = self.stacked_adapter()
        n_ad = len(self.A)
        alpha = self.alpha * n_ad if n_ad else self.alpha  # scale alpha / (n_ad r) = self.alpha / r
        h = QLoRALinearFunction.apply(x2, A, B, self.w, alpha, False, self._sink if n_ad else None)
        return tuple(t.reshape(*lead, t.shape[-1]) for t in torch.split(h, self.d_outs, dim=1))
