"""Paged AdamW for the adapter parameters (A, B) of the QLoRA layers.

The first page ("QLoRA는 어떻게 65B 모델을 GPU 한 장에 올렸나", section "메모리 회계", paged-optimizer entry)
moves the adapters' Adam state out to pinned CPU memory and lets the update run beside the backward on another
stream. Here each bf16 parameter keeps a float32 master copy in device memory, and its moments m, v are float32
in pinned host memory (or in device memory with paged=False). One `qlora_adamw_step` per parameter updates them
in place and rewrites the bf16 parameter; the kernel reads and writes the host-side state over the host link.
Argument marshalling only: the arithmetic is the library's.

The page has the CPU run the update; here a GPU kernel runs it on a side stream, reading and writing the state in
pinned host memory in place (the same memory placement, with the arithmetic where the gradients already are, so
no gradient or state page has to be copied for the CPU to see it).

Gradients: the QLoRA layers keep the library's float32 dA and dB on each adapter parameter as `grad_fp32`
(autograd's own `.grad` is bf16, the parameters' dtype); the step uses those when present and `.grad` otherwise.
Zero gradients with `zero_grad()` here (or torch's default set_to_none): the float32 copy restarts whenever
`.grad` is None.
"""

from __future__ import annotations

import torch

from . import qlora as q


class PagedAdamW:
    """AdamW (decoupled weight decay) over bf16 parameters, with the state paged to pinned host memory.

    step() enqueues the updates on `stream` (a side stream, default priority) after the gradients are ready on the
    caller's current stream; wait() makes the current stream wait for them, and must come before the parameters
    are read again (the next forward).
    """

    def __init__(self, params, lr: float = 1e-4, betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.0,
                 paged: bool = True, stream: torch.cuda.Stream | None = None):
        self.params = [p for p in params if p.requires_grad]
        if not self.params:
            raise ValueError("no trainable parameters")
        self.lr, self.betas, self.eps, self.weight_decay = float(lr), tuple(betas), float(eps), float(weight_decay)
        self.paged = paged
        dev = self.params[0].device
        self.stream = stream if stream is not None else torch.cuda.Stream(dev)
        self.state = []
        for p in self.params:
            if p.dtype != torch.bfloat16 or not p.is_contiguous():
                raise TypeError("parameters must be contiguous bfloat16 tensors")
            master = p.detach().float().reshape(-1).clone()
            if paged:
                m = torch.zeros(p.numel(), dtype=torch.float32).pin_memory()
                v = torch.zeros(p.numel(), dtype=torch.float32).pin_memory()
            else:
                m = torch.zeros(p.numel(), dtype=torch.float32, device=p.device)
                v = torch.zeros(p.numel(), dtype=torch.float32, device=p.device)
            self.state.append((master, m, v))
        self.step_count = 0
        self._done = None

    def zero_grad(self):
        for p in self.params:
            p.grad = None
            p.grad_fp32 = None

    @torch.no_grad()
    def step(self):
        self.step_count += 1
        cur = torch.cuda.current_stream(self.params[0].device)
        grads = []
        for p in self.params:
            if p.grad is None:
                grads.append(None)
                continue
            g32 = getattr(p, "grad_fp32", None)
            # the layers' float32 gradient when they left one, else autograd's (bf16) one widened
            g = g32 if g32 is not None else p.grad.detach().float()
            grads.append(g.reshape(-1).contiguous())
        ready = torch.cuda.Event()
        ready.record(cur)
        self.stream.wait_event(ready)
        for p, g, (master, m, v) in zip(self.params, grads, self.state):
            if g is None:
                continue
            g.record_stream(self.stream)
            q.qlora_adamw_step(self.step_count, g, master, m, v, p.data.view(-1), lr=self.lr, beta1=self.betas[0],
                               beta2=self.betas[1], eps=self.eps, weight_decay=self.weight_decay, stream=self.stream)
        self._done = torch.cuda.Event()
        self._done.record(self.stream)

    def wait(self):
        """The current stream waits for the last step's updates."""
        if self._done is not None:
            torch.cuda.current_stream(self.params[0].device).wait_event(self._done)
