"""Paged AdamW for the adapter parameters (A, B) of the QLoRA layers.

The first page ("QLoRA는 어떻게 65B 모델을 GPU 한 장에 올렸나", section "메모리 회계", paged-optimizer entry)
moves the adapters' Adam state out to pinned CPU memory and lets the update run beside the backward. Here each
bf16 parameter's moments m, v are float32 in pinned host memory (or in device memory with paged=False), with a
float32 master copy of the parameter. Argument marshalling only: the arithmetic is the library's.

Two placements of the update:
  * update="device" (default): one `qlora_adamw_step` per parameter, a GPU kernel on a side stream that reads and
    writes m, v in pinned host memory in place over the host link (the master copy in device memory) and
    rewrites the bf16 parameter (the page's memory placement, with the arithmetic where the gradients already
    are; graph-capturable);
  * update="host": the page's own placement. The float32 gradients are copied to pinned host buffers (DMA), the
    library's host AdamW (qlora_adamw_step_host, native worker threads) updates the float32 master copy, m and v,
    all in pinned host memory, and the bf16 parameters are copied back (DMA). A Python worker thread runs the
    host steps, so the caller's thread goes on launching GPU work meanwhile; the compute units never run the
    update. Not graph-capturable (host work between the copies).

Gradients: the QLoRA layers keep the library's float32 dA and dB on each adapter parameter as `grad_fp32`
(autograd's own `.grad` is bf16, the parameters' dtype); the step uses those when present and `.grad` otherwise.
Zero gradients with `zero_grad()` here (or torch's default set_to_none): the float32 copy restarts whenever
`.grad` is None.
"""

from __future__ import annotations

import queue
import threading

import torch

from . import qlora as q


class HostAdamWWorker:
    """Runs host AdamW steps in a background thread, between a device-to-host copy of the gradient and a
    host-to-device copy of the bf16 parameter, both on `stream` (DMA copies). submit() returns at once; wait()
    makes the caller's current stream wait until every submitted parameter is back on the device."""

    def __init__(self, device, stream: torch.cuda.Stream | None = None):
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.Stream(self.device)  # default priority
        self._jobs = queue.Queue()
        self._pending = []
        self._error = None
        self._thread = threading.Thread(target=self._loop, daemon=True)
        self._thread.start()

    def submit(self, step, grad, grad_host, master, m, v, param, param_host, ready, **hp):
        """grad (device f32) -> grad_host (pinned) after `ready` (an event on the producing stream); host AdamW
        on master, m, v (pinned f32) writing param_host (pinned bf16); param_host -> param (device bf16)."""
        self.stream.wait_event(ready)
        with torch.cuda.stream(self.stream):
            grad_host.copy_(grad, non_blocking=True)
        grad.record_stream(self.stream)
        copied = torch.cuda.Event()
        copied.record(self.stream)
        job = dict(step=step, copied=copied, grad_host=grad_host, master=master, m=m, v=v, param=param,
                   param_host=param_host, hp=hp, enqueued=threading.Event(), done=None)
        self._pending.append(job)
        self._jobs.put(job)
        return job

    submit_job = submit

    def wait_jobs(self, jobs):
        """The current stream waits for these submitted jobs' parameters."""
        cur = torch.cuda.current_stream(self.device)
        for job in jobs:
            job["enqueued"].wait()
            if job["done"] is not None:
                cur.wait_event(job["done"])
        done = set(map(id, jobs))
        self._pending = [j for j in self._pending if id(j) not in done]
        if self._error is not None:
            e, self._error = self._error, None
            raise e

    def _loop(self):
        while True:
            job = self._jobs.get()
            if job is None:
                return
            try:
                job["copied"].synchronize()
                q.qlora_adamw_step_host(job["step"], job["grad_host"], job["master"], job["m"], job["v"],
                                        job["param_host"], **job["hp"])
                with torch.cuda.stream(self.stream):
                    job["param"].copy_(job["param_host"], non_blocking=True)
                done = torch.cuda.Event()
                done.record(self.stream)
                job["done"] = done
            except Exception as e:  # pragma: no cover - reported by wait()
                self._error = e
            finally:
                job["enqueued"].set()

    def wait(self):
        self.wait_jobs(list(self._pending))

    def close(self):
        self._jobs.put(None)
        self._thread.join()


class PagedAdamW:
    """AdamW (decoupled weight decay) over bf16 parameters, with the state paged to pinned host memory.

    step() enqueues the updates on `stream` (a side stream, default priority) after the gradients are ready on the
    caller's current stream; wait() makes the current stream wait for them, and must come before the parameters
    are read again (the next forward).
    """

    def __init__(self, params, lr: float = 1e-4, betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.0,
                 paged: bool = True, stream: torch.cuda.Stream | None = None, update: str = "device"):
        self.params = [p for p in params if p.requires_grad]
        if not self.params:
            raise ValueError("no trainable parameters")
        if update not in ("device", "host"):
            raise ValueError("update must be 'device' or 'host'")
        if update == "host" and not paged:
            raise ValueError("update='host' keeps the state in pinned host memory (paged=True)")
        self.lr, self.betas, self.eps, self.weight_decay = float(lr), tuple(betas), float(eps), float(weight_decay)
        self.paged, self.update = paged, update
        dev = self.params[0].device
        self.stream = stream if stream is not None else torch.cuda.Stream(dev)
        self.worker = HostAdamWWorker(dev, self.stream) if update == "host" else None
        self.state = []
        self.staging = []
        for p in self.params:
            if p.dtype != torch.bfloat16 or not p.is_contiguous():
                raise TypeError("parameters must be contiguous bfloat16 tensors")
            if update == "host":  # the master copy lives with m and v, in pinned host memory
                master = p.detach().float().reshape(-1).cpu().pin_memory()
                self.staging.append((torch.empty(p.numel(), dtype=torch.float32).pin_memory(),
                                     torch.empty(p.numel(), dtype=torch.bfloat16).pin_memory()))
            else:
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
        if self.update == "host":
            for p, g, (master, m, v), (g_host, p_host) in zip(self.params, grads, self.state, self.staging):
                if g is not None:
                    self.worker.submit(self.step_count, g, g_host, master, m, v, p.data.view(-1), p_host, ready,
                                       lr=self.lr, beta1=self.betas[0], beta2=self.betas[1], eps=self.eps,
                                       weight_decay=self.weight_decay)
            return
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
        if self.worker is not None:
            self.worker.wait()
            return
        if self._done is not None:
            torch.cuda.current_stream(self.params[0].device).wait_event(self._done)
