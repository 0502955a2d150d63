#!/usr/bin/env python3
"""Benchmark of the QLoRA frozen-NF4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 65b_layer]

Default workload (the largest configuration that fits one GPU): one decoder layer of a 65B model, hidden 8192,
MLP 22016 -- q, k, v, o 8192x8192, gate and up 22016x8192, down 8192x22016 -- every projection an NF4 +
double-quant weight (W ~ N(0, 0.02^2)) with a LoRA adapter r=64 alpha=16 (A, B ~ N(0, 0.02^2) bf16), at
batch 8 x seq 512 = 4096 tokens (x, dY ~ N(0, 1) bf16). One step = for every projection the forward
h = dequant(W) x + (alpha/r) B A x (u saved) and the backward dX, dA, dB. Quantization happens once before
timing, as at model load.

Timing. W warm-up steps, then exactly K steps between HIP events on the launch stream, the region bracketed by
torch.cuda.synchronize(). Launches are eager (every kernel runs hundreds of microseconds, so the host stays
ahead), with HIP events on the same stream around every forward and backward call.

Printed: one JSON line.
  value       TFLOP/s of the whole step (forward + backward flops of every projection / step time).
  roofline    the fused dequant-GEMM + LoRA forward call (qlora_forward: k_lora_tall forms u = x A^T, then
              k_gemm_fwd the tiled contraction with the adapter term as extra K columns): its algorithmic flops
              over its mean duration, from the events around every forward call in the timed region, against
              the 2.5 PFLOP/s bf16 dense MFMA peak.
  cpu_baseline the CPU oracle (float64) on a bounded sample -- row slices of one projection of each distinct
              shape at a reduced token count -- scaled linearly to the step (flagged "scaled").
  skinny      the weight-streaming regime on the LLaMA-7B projections (4096x4096 and 11008x4096, r=64, T = 1, 4
              and 16, forward): weight GB/s and the k_gemv_fwd roofline against 8 TB/s (graph-replayed, each
              call on its own weight copy so that HBM serves the stream).
  hbm_ceiling a streaming read and a device copy of 2 GiB measured in the same run (torch kernels).
  per_call    every forward and backward call's mean duration and TFLOP/s.

Other workloads (--workload) are records, not the headline line:
  llama7b_skinny / 65b_skinny  the weight-streaming forward alone (T <= 16; graph-replayed);
  13b_4096tok / linear1024 / 14b_stack  forward + backward of the 13B projections, the single-linear parity
      config, one of the 40 identical layers of the 14B-style stack (bf16 source weights, 2048 tokens, LoRA
      r=8 on q and v);
  14b_stack_fused  the same layer with q/k/v and gate/up each stacked into one call that reads its input once
      (q and v adapters as one block-diagonal rank-16 pair);
  65b_layer_fused  the 65B layer with q/k/v (three rank-64 adapters as one block-diagonal rank-192 pair) and
      gate/up stacked, TFLOP/s counted with the unstacked projections' algorithmic flops;
  14b_quantize  one pass quantizing all 280 bf16 weights of the 14B-style stack (13.2 G parameters, generated
      on the device from a seeded generator) with qlora_quantize_many (32 weights per launch), and beside it the
      same pass as one qlora_quantize call per weight;
  merge_llama7b  merge for export, bf16(W_hat + (alpha/r) B A), of the two LLaMA-7B projections with r = 64;
  13b_paged_adamw  the 13b_4096tok step, timed without and with an AdamW update of every A and B whose moments
      m, v sit in pinned host memory (float32 master on the device); the update of a projection runs on a side
      stream beside the next projection's forward and backward.
  --storage absmax  any forward/backward workload on absmax-only weights (one float32 scale per 64-weight
      block, 4.5 bits) instead of double quant.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused NF4-dequant GEMM+LoRA TFLOP/s and weight GB/s, % of roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
WORKLOAD_CHOICES = ["llama7b_skinny", "65b_skinny", "linear1024", "13b_4096tok", "65b_layer", "14b_stack", "14b_stack_fused", "65b_layer_fused",
                    "14b_chain", "14b_quantize",
                    "merge_llama7b", "13b_paged_adamw"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed steps (default: 20, or 200 for T <= 16 workloads)")
    p.add_argument("--warmup", type=int, default=None, help="warm-up steps (default: 3, or 20 for T <= 16)")
    p.add_argument("--workload", default="65b_layer", choices=WORKLOAD_CHOICES)
    p.add_argument("--chunk", type=int, default=20, help="steps per captured graph")
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying graphs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-per-call", action="store_true", help="skip the per-call-shape timings (profiling runs)")
    p.add_argument("--no-extras", action="store_true",
                   help="default workload: skip the skinny and HBM-ceiling measurements (profiling runs)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--storage", default="dq", choices=["dq", "absmax"],
                   help="weight storage: NF4 with double-quantized scales (4.13 bits) or float32 block absmax (4.5)")
    p.add_argument("--paging", default="zerocopy", choices=["zerocopy", "dma", "host"],
                   help="13b_paged_adamw: update m, v in host memory in place (GPU kernel), copy each page to the "
                        "device and back, or run the update on the host CPU (the page's placement; eager only)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy (reference for HBM counter scaling)")
    a = p.parse_args()
    if a.paging == "host":
        a.no_graph = True  # host work between the copies cannot be captured
    skinny = a.workload in ("llama7b_skinny", "65b_skinny", "merge_llama7b")
    if a.steps is None:
        a.steps = 200 if skinny else 20
    if a.warmup is None:
        a.warmup = 20 if skinny else 3
    return a


ABSMAX_STORAGE = [False]  # set from --storage


def weight_bytes(d_out, d_in):
    n = d_out * d_in
    nb = n // 64
    if ABSMAX_STORAGE[0]:
        return n // 2 + 4 * nb               # codes + one float32 scale per block (4.5 bits)
    return n // 2 + nb + 4 * ((nb + 255) // 256)


def fwd_bytes(d_out, d_in, r, T):
    """Algorithmic HBM bytes of one forward: NF4 weight + adapters + x in + h out."""
    return weight_bytes(d_out, d_in) + 2 * r * (d_in + d_out) + 2 * T * (d_in + d_out)


def bwd_bytes(d_out, d_in, r, T):
    """Backward: NF4 weight + adapters + dY, x, u in; dX, dA, dB (f32) out."""
    return (weight_bytes(d_out, d_in) + 2 * r * (d_in + d_out) + 2 * T * (d_in + d_out) + 2 * T * d_in
            + 4 * T * r + 4 * r * (d_in + d_out))


def fwd_flops(d_out, d_in, r, T):
    return 2 * T * d_in * d_out + 2 * T * r * (d_in + d_out)


def bwd_flops(d_out, d_in, r, T):
    return 2 * T * d_in * d_out + 4 * T * r * (d_in + d_out)


def proj_flops(p, T, backward):
    """Algorithmic flops of one call. A stacked call counts each adapter on its own projection's rows, not the
    zeros of its block-diagonal B: the same count as the projections called one by one."""
    f = bwd_flops if backward else fwd_flops
    if not p.b_rows:
        return f(p.d_out, p.d_in, p.r, T)
    rk = p.r // len(p.b_rows)
    return f(p.d_out, p.d_in, 0, T) + sum(f(r1 - r0, p.d_in, rk, T) - f(r1 - r0, p.d_in, 0, T) for r0, r1 in p.b_rows)


TRAIN_WORKLOADS = ("65b_layer", "65b_layer_fused", "13b_4096tok", "14b_stack", "14b_stack_fused", "linear1024")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported. The layer shards "
              "as data parallel (tokens split across GPUs, dA/dB summed); that path is not built.", flush=True)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.chunk < 1:
        sys.exit("--steps >= 1, --warmup >= 0, --chunk >= 1")

    import torch

    from bit_quantized_finetuning_amd import qlora as q
    from bit_quantized_finetuning_amd import synth

    dev = torch.device("cuda:0")
    ABSMAX_STORAGE[0] = args.storage == "absmax"
    if ABSMAX_STORAGE[0] and args.workload in ("merge_llama7b", "14b_quantize", "13b_paged_adamw"):
        sys.exit(f"--storage absmax is measured on the forward/backward workloads, not {args.workload}")
    if args.workload == "merge_llama7b":
        return bench_merge(args, torch, q, synth, dev)
    if args.workload == "14b_quantize":
        return bench_quantize_stack(args, torch, q, synth, dev)
    if args.workload == "14b_chain":
        return bench_chain(args, torch, q, synth, dev)
    if args.workload == "13b_paged_adamw":
        return bench_graph(args, torch, q, synth, dev, "13b_4096tok", paged=True)
    if args.workload in TRAIN_WORKLOADS:
        return bench_train(args, torch, q, synth, dev, args.workload)
    return bench_graph(args, torch, q, synth, dev, args.workload)


def bench_train(args, torch, q, synth, dev, wname, emit=True):
    """Forward + backward of every projection of a workload, eager launches, HIP events around every call."""
    wl = synth.WORKLOADS[wname]
    cfg = synth.WORKLOAD_SEED[wname]
    (T,) = wl.tokens

    def dev16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    projs = []
    for pi, p in enumerate(wl.projections):
        W = torch.from_numpy(synth.weight(cfg, pi, p.d_out, p.d_in, wl.weight_dtype)).to(dev)
        w = q.qlora_quantize(W, double_quant=not ABSMAX_STORAGE[0])
        del W
        A = B = None
        if p.r > 0:
            (_, A_bits), (_, B_bits) = synth.adapters(cfg, pi, p.d_out, p.d_in, p.r)
            A, B = dev16(A_bits), dev16(B_bits)
            if p.b_rows:  # stacked projections: block-diagonal B (adapter k on its projection's rows only)
                mask = torch.zeros_like(B, dtype=torch.bool)
                rk = p.r // len(p.b_rows)
                for k, (r0, r1) in enumerate(p.b_rows):
                    mask[r0:r1, k * rk:(k + 1) * rk] = True
                B = torch.where(mask, B, torch.zeros_like(B))
        x = dev16(synth.tokens(cfg, pi, T, p.d_in)[1])
        dy = dev16(synth.upstream_grad(cfg, pi, T, p.d_out)[1])
        h = torch.empty(T, p.d_out, dtype=torch.bfloat16, device=dev)
        u = torch.empty(T, p.r, dtype=torch.float32, device=dev) if p.r > 0 else None
        dX = torch.empty(T, p.d_in, dtype=torch.bfloat16, device=dev)
        dA = torch.empty(p.r, p.d_in, dtype=torch.float32, device=dev) if p.r > 0 else None
        dB = torch.empty(p.d_out, p.r, dtype=torch.float32, device=dev) if p.r > 0 else None
        projs.append((p, w, A, B, x, dy, h, u, dX, dA, dB))
    ws = q.workspace(dev, max(q.qlora_workspace_bytes(p.d_out, p.d_in, T, p.r) for p in wl.projections))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    n = len(projs)

    def step(ev=None):
        for i, (p, w, A, B, x, dy, h, u, dX, dA, dB) in enumerate(projs):
            if ev is not None:
                ev[2 * i].record(stream)
            q.qlora_forward(w, x, A, B, p.alpha, h=h, u=u, ws=ws)
            if ev is not None:
                ev[2 * i + 1].record(stream)
        for i, (p, w, A, B, x, dy, h, u, dX, dA, dB) in enumerate(reversed(projs)):
            j = n - 1 - i
            if ev is not None:
                ev[2 * n + 2 * j].record(stream)
            q.qlora_backward(w, x, dy, A, B, p.alpha, u_saved=u, dX=dX, dA=dA, dB=dB, ws=ws)
            if ev is not None:
                ev[2 * n + 2 * j + 1].record(stream)

    print(f"[bench] {wname}: inputs ready, {args.warmup} warm-up + {args.steps} timed steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4 * n)] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for k in range(args.steps):
        step(evs[k])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    fwd_ms = [np.mean([e[2 * i].elapsed_time(e[2 * i + 1]) for e in evs]) for i in range(n)]
    bwd_ms = [np.mean([e[2 * n + 2 * i].elapsed_time(e[2 * n + 2 * i + 1]) for e in evs]) for i in range(n)]

    ff = sum(proj_flops(p, T, False) for p, *_ in projs)
    bf = sum(proj_flops(p, T, True) for p, *_ in projs)
    tflops = (ff + bf) / (ms_step * 1e-3) / 1e12
    # the fused dequant-GEMM + LoRA forward: algorithmic flops of all forward calls over their summed duration
    fwd_tf = ff / (sum(fwd_ms) * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(fwd_tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(fwd_tf / BF16_PEAK_TFLOPS, 4),
            # the recorded counters are those of this call on the 65B layer with double-quant storage
            "traffic": recorded_traffic(FWD_TRAFFIC_RECORD) if wname == "65b_layer" and not ABSMAX_STORAGE[0] else None,
            "kernel": "qlora_forward at T = %d: k_lora_tall (u = x A^T) then k_gemm_fwd (dequant GEMM with the "
                      "adapter term as extra K columns)" % T if T >= 65 else "qlora_forward",
            "flops_per_launch": round(ff / n), "us_per_launch": round(1e3 * sum(fwd_ms) / n, 2),
            "launches": args.steps * n, "timing": "HIP events around every forward call in the timed region"}
    label_traffic(roof, FWD_TRAFFIC_RECORD)
    per_call = []
    for i, (p, *_r) in enumerate(projs):
        for kind, ms, fl in (("fwd", fwd_ms[i], proj_flops(p, T, False)),
                             ("bwd", bwd_ms[i], proj_flops(p, T, True))):
            per_call.append({"proj": f"{p.name} {p.d_out}x{p.d_in}", "call": kind, "r": p.r,
                             "us": round(ms * 1e3, 1), "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 1)})
    wbytes = 2 * sum(weight_bytes(p.d_out, p.d_in) for p, *_ in projs)
    line = {
        "metric": METRIC,
        "value": round(tflops, 1),
        "unit": "TFLOP/s (forward + backward of every projection)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02^2) weights and adapters, N(0,1) tokens and upstream gradients)",
        "config": {"workload": wl.description, "projections": [f"{p.name} {p.d_out}x{p.d_in}" for p in wl.projections],
                   "tokens": T, "lora_r": [p.r for p in wl.projections], "lora_alpha": wl.projections[0].alpha,
                   "backward": True, "launch": "eager",
                   "weight_storage": ("NF4 + float32 absmax per 64-weight block (4.5 bits)" if ABSMAX_STORAGE[0]
                                      else "NF4 + double-quantized block scales (4.127 bits)"),
                   **({"layers_in_stack": wl.layers, "layers_per_step": 1} if wl.layers > 1 else {})},
        "weight_GBs": round(wbytes / (ms_step * 1e-3) / 1e9, 1),
        "roofline": roof,
        "per_call": per_call,
        "workspace_fallbacks": q.qlora_workspace_fallbacks(ws),
        "cpu_baseline": None,
    }
    print(f"[bench] {wname}: {ms_step:.3f} ms/step, {tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)
    if args.copy_calibration:
        copy_calibration(torch, dev)
    if not emit:
        return line
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_train(args, wl, cfg, ms_step, ff + bf)
        print("[bench] cpu baseline done", file=sys.stderr, flush=True)
    if wname == "65b_layer" and not args.no_extras:
        import copy

        del projs
        torch.cuda.empty_cache()
        sargs = copy.copy(args)
        sargs.steps, sargs.warmup, sargs.no_cpu_baseline = 200, 20, True
        sk = bench_graph(sargs, torch, q, synth, dev, "llama7b_skinny", emit=False)
        line["skinny"] = {"workload": sk["config"]["workload"], "value": sk["value"], "unit": sk["unit"],
                          "ms_per_step": sk["ms_per_step"], "steps": sargs.steps, "roofline": sk["roofline"],
                          "per_call": sk["per_call"], "grouped": sk.get("grouped")}
        print("[bench] skinny record done", file=sys.stderr, flush=True)
        line["hbm_ceiling"] = hbm_ceiling(torch, dev)
    print(json.dumps(line), flush=True)


def bench_chain(args, torch, q, synth, dev):
    """All 40 layers of the 14B-style stack chained (bit_quantized_finetuning_amd.stack): one step = forward of the
    stack under gradient checkpointing and the backward (each layer's forward again, then its backward), at 2048
    tokens, from a bf16 input that requires grad and a seeded upstream gradient. Eager launches."""
    from bit_quantized_finetuning_amd.stack import DecoderStack

    wl = synth.WORKLOADS["14b_stack"]
    (T,) = wl.tokens
    layers = wl.layers
    st = DecoderStack(layers=layers, device=dev, checkpoint=True)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    with torch.no_grad():  # B starts at zero; give it values so that the adapter terms are real work
        for layer in st.layers:
            for B in layer.qkv.B:
                B.copy_((torch.randn(B.shape, device=dev, generator=gen) * 0.02).to(torch.bfloat16))
    params = [p for p in st.parameters() if p.requires_grad]
    x0 = torch.randn(T, 5120, device=dev, generator=gen).to(torch.bfloat16).requires_grad_(True)
    dy = torch.randn(T, 5120, device=dev, generator=gen).to(torch.bfloat16)
    stream = torch.cuda.current_stream(dev)

    def step():
        for p in params + [x0]:
            p.grad = None
            if hasattr(p, "grad_fp32"):
                p.grad_fp32 = None
        st(x0).backward(dy)

    torch.cuda.synchronize()
    print(f"[bench] 14b_chain: {layers} layers built, {args.warmup} warm-up + {args.steps} timed steps",
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    ff = layers * sum(fwd_flops(p.d_out, p.d_in, p.r, T) for p in wl.projections)
    bf = layers * sum(bwd_flops(p.d_out, p.d_in, p.r, T) for p in wl.projections)
    tflops = (ff + bf) / (ms_step * 1e-3) / 1e12
    executed = (2 * ff + bf) / (ms_step * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
            "kernel": "whole step: the projections' forward + backward flops over the step time (the recomputed "
                      "forward and the torch glue between the calls count as time only)"}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_train(args, wl, synth.WORKLOAD_SEED["14b_stack"], ms_step, ff + bf, layers=layers)
    extra = {"data": "synthetic (seeded N(0,0.02^2) bf16 weights drawn on the device, LoRA A N(0,0.02^2), "
                     "B N(0,0.02^2), N(0,1) input and upstream gradient)",
             "config": {"workload": f"14B-style stack, all {layers} layers chained, hidden 5120, MLP 17408, k/v "
                                    f"1024, LoRA r=8 alpha=16 on q/v, {T} tokens, gradient checkpointing, q/k/v "
                                    "and gate/up as stacked calls, fwd+bwd",
                        "layers": layers, "tokens": T, "launch": "eager"},
             "executed_TFLOPs_incl_recompute": round(executed, 1),
             "ms_per_layer": round(ms_step / layers, 3)}
    _line(args, round(tflops, 1), "TFLOP/s (forward + backward of every projection of the 40 layers)", ms_step,
          args.steps, extra["config"]["workload"], roof, cpu, extra)


def copy_calibration(torch, dev):
    """A plain device copy of known size (256 MiB read + 256 MiB written per launch, three launches): the
    reference that scales the HBM byte counters of a profiled run."""
    a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def hbm_ceiling(torch, dev, nbytes=2 << 30, reps=10):
    """Measured HBM ceilings: a streaming read (a sum over nbytes of float32) and a device copy."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        a.sum()
        b.copy_(a)
    torch.cuda.synchronize()
    out = {}
    for name, fn, moved in (("read_GBs", lambda: a.sum(), nbytes),
                            ("copy_GBs", lambda: b.copy_(a), 2 * nbytes)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(moved * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    out["bytes"] = nbytes
    out["kernels"] = "torch sum (read) and copy_ (read + write) over 2 GiB of float32"
    return out


class HostJobs:
    """The host-update jobs of one projection's adapters: wait() makes the current stream wait for all of them."""

    def __init__(self, worker):
        self.worker, self.jobs = worker, []

    def add(self, job):
        self.jobs.append(job)

    def wait(self):
        self.worker.wait_jobs(self.jobs)


def bench_graph(args, torch, q, synth, dev, wname, paged=False, emit=True):
    """Steps captured into HIP graphs and replayed (the weight-streaming workloads, whose 8-80 us kernels would
    otherwise wait on the host, and the paged-AdamW record). Returns the JSON line (printed when emit)."""
    wl = synth.WORKLOADS[wname]
    seed_cfg = synth.WORKLOAD_SEED[wname]
    bw = bool(wl.backward)
    chunk = min(args.chunk, args.steps)
    nT = len(wl.tokens)

    def dev16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs: quantize once, then replicate the quantized weight so each call of a chunk has its own
    projs = []
    for pi, p in enumerate(wl.projections):
        W = torch.from_numpy(synth.weight(seed_cfg, pi, p.d_out, p.d_in, wl.weight_dtype)).to(dev)
        w0 = q.qlora_quantize(W, double_quant=not ABSMAX_STORAGE[0])
        del W
        A0 = B0 = None
        if p.r > 0:
            (_, A_bits), (_, B_bits) = synth.adapters(seed_cfg, pi, p.d_out, p.d_in, p.r)
            A0, B0 = dev16(A_bits), dev16(B_bits)
            if p.b_rows:  # stacked projections: block-diagonal B (adapter k on its projection's rows only)
                mask = torch.zeros_like(B0, dtype=torch.bool)
                rk = p.r // len(p.b_rows)
                for k, (r0, r1) in enumerate(p.b_rows):
                    mask[r0:r1, k * rk:(k + 1) * rk] = True
                B0 = torch.where(mask, B0, torch.zeros_like(B0))
        ncopy = chunk * nT if not bw else 2
        copies = [(w0, A0, B0)]
        for _ in range(ncopy - 1):
            copies.append((q.NF4Weight(p.d_out, p.d_in, w0.codes.clone(),
                                       None if w0.qscale is None else w0.qscale.clone(), w0.smax.clone()),
                           None if A0 is None else A0.clone(), None if B0 is None else B0.clone()))
        xs = {T: dev16(synth.tokens(seed_cfg, pi, T, p.d_in)[1]) for T in wl.tokens}
        dys = {T: dev16(synth.upstream_grad(seed_cfg, pi, T, p.d_out)[1]) for T in wl.tokens} if bw else {}
        outs = {T: torch.empty(T, p.d_out, dtype=torch.bfloat16, device=dev) for T in wl.tokens}
        grads = {}
        if bw:
            for T in wl.tokens:
                grads[T] = (torch.empty(T, p.d_in, dtype=torch.bfloat16, device=dev),
                            torch.empty(max(p.r, 1), p.d_in, dtype=torch.float32, device=dev),
                            torch.empty(p.d_out, max(p.r, 1), dtype=torch.float32, device=dev),
                            torch.empty(T, max(p.r, 1), dtype=torch.float32, device=dev))
        projs.append((p, copies, xs, dys, outs, grads))
    # paged AdamW state per projection and copy: the Adam moments m, v of A and B in pinned host memory, the
    # float32 master copy on the device
    opt_state = {}
    opt_stream = torch.cuda.Stream(dev) if paged else None  # default priority
    host_update = paged and args.paging == "host"
    worker = None
    if host_update:
        from bit_quantized_finetuning_amd.optim import HostAdamWWorker
        worker = HostAdamWWorker(dev, opt_stream)
    staging = {}
    if paged:
        for pi, (p, copies, *_rest) in enumerate(projs):
            for ci, (wc, A, B) in enumerate(copies):
                if A is None:
                    continue
                st = []
                for t in (A, B):
                    # the host update keeps the master copy with m and v in pinned host memory
                    master = t.float().cpu().pin_memory() if host_update else t.float()
                    st.append((t, master, torch.zeros(t.numel(), dtype=torch.float32).pin_memory(),
                               torch.zeros(t.numel(), dtype=torch.float32).pin_memory()))
                    if host_update:
                        staging[(pi, ci, len(st) - 1)] = (torch.empty(t.numel(), dtype=torch.float32).pin_memory(),
                                                          torch.empty(t.numel(), dtype=torch.bfloat16).pin_memory())
                opt_state[(pi, ci)] = st
    # DMA paging: one device page (m, v) sized for the largest parameter, reused in turn on the update stream
    # (its copies and kernels run in order there)
    page = None
    if paged and args.paging == "dma" and opt_state:
        nmax = max(st[1].numel() for sts in opt_state.values() for st in sts)
        page = [torch.empty(nmax, dtype=torch.float32, device=dev) for _ in range(2)]
    opt_on = [False]
    opt_pending = {}
    # one workspace large enough for every call, allocated (zeroed) before any capture
    ws_need = max(q.qlora_workspace_bytes(p.d_out, p.d_in, T, p.r) for p, *_ in projs for T in wl.tokens)
    q.workspace(dev, ws_need)
    torch.cuda.synchronize()

    calls = [(p, copies, xs[T], dys.get(T), outs[T], grads.get(T), T, ti)
             for p, copies, xs, dys, outs, grads in projs for ti, T in enumerate(wl.tokens)]

    def run_call(p, copies, x, dy, h, g, T, ti, k):
        ci = k % len(copies)
        wc, A, B = copies[ci]
        if not bw:
            q.qlora_forward(wc, x, A, B, p.alpha, h=h)
            return
        pi = next(i for i, pr in enumerate(projs) if pr[0] is p)
        if opt_on[0] and (pi, ci) in opt_pending:
            # the previous update of these parameters must land before the forward reads them
            pend = opt_pending.pop((pi, ci))
            if host_update:
                pend.wait()
            else:
                torch.cuda.current_stream(dev).wait_event(pend)
        dX, dA, dB, u = g
        ur = u if p.r > 0 else None
        q.qlora_forward(wc, x, A, B, p.alpha, h=h, u=ur)
        q.qlora_backward(wc, x, dy, A, B, p.alpha, u_saved=ur, dX=dX, dA=dA if p.r > 0 else None,
                         dB=dB if p.r > 0 else None)
        if opt_on[0] and (pi, ci) in opt_state and host_update:
            ready = torch.cuda.Event()
            ready.record(torch.cuda.current_stream(dev))
            jobs = HostJobs(worker)
            for k, ((t, master, m, v), grad) in enumerate(zip(opt_state[(pi, ci)], (dA, dB))):
                g_host, p_host = staging[(pi, ci, k)]
                jobs.add(worker.submit_job(1, grad.view(-1), g_host, master, m, v, t.view(-1), p_host, ready,
                                           lr=1e-4, weight_decay=0.01))
            opt_pending[(pi, ci)] = jobs
            return
        if opt_on[0] and (pi, ci) in opt_state:
            ready = torch.cuda.Event()
            ready.record(torch.cuda.current_stream(dev))
            opt_stream.wait_event(ready)
            for (t, master, m, v), grad in zip(opt_state[(pi, ci)], (dA, dB)):
                if page is None:  # zero-copy: the kernel updates the state in host memory
                    q.qlora_adamw_step(1, grad.view(-1), master.view(-1), m.view(-1), v.view(-1), t.view(-1),
                                       lr=1e-4, weight_decay=0.01, stream=opt_stream)
                    continue
                n_el = master.numel()
                dmm, dv = (b[:n_el] for b in page)
                with torch.cuda.stream(opt_stream):
                    for d, h in ((dmm, m), (dv, v)):
                        d.copy_(h, non_blocking=True)
                q.qlora_adamw_step(1, grad.view(-1), master.view(-1), dmm, dv, t.view(-1), lr=1e-4, weight_decay=0.01,
                                   stream=opt_stream)
                with torch.cuda.stream(opt_stream):
                    for d, h in ((dmm, m), (dv, v)):
                        h.copy_(d, non_blocking=True)
            done = torch.cuda.Event()
            done.record(opt_stream)
            opt_pending[(pi, ci)] = done

    def run_steps(s0, n):
        for s in range(s0, s0 + n):
            for c in calls:
                run_call(*c, s * nT + c[-1])
        if opt_on[0]:
            if host_update:
                for pend in opt_pending.values():
                    pend.wait()
            # join the update stream (also closes a graph capture's fork)
            torch.cuda.current_stream(dev).wait_stream(opt_stream)
            opt_pending.clear()

    stream = torch.cuda.current_stream(dev)

    def measure():
        """Warm up, capture the step graphs, replay once, then time exactly args.steps steps (ms)."""
        for s in range(max(args.warmup, 1)):
            run_steps(s % chunk, 1)
        torch.cuda.synchronize()
        # ---- graphs: one of `chunk` steps, and one of the remainder
        graphs = {}
        if not args.no_graph:
            side = torch.cuda.Stream(dev)  # default priority
            for n in sorted({chunk, args.steps % chunk} - {0}):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    run_steps(0, n)
                graphs[n] = g
            torch.cuda.synchronize()
            for n, g in graphs.items():       # one untimed replay of each
                g.replay()
            torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        if graphs:
            for _ in range(args.steps // chunk):
                graphs[chunk].replay()
            if args.steps % chunk:
                graphs[args.steps % chunk].replay()
        else:
            run_steps(0, args.steps)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1), bool(graphs)

    paged_info = None
    if paged:
        ms_off, _ = measure()           # the step alone
        opt_on[0] = True
        ms_total, have_graphs = measure()  # the step with the paged update
        opt_on[0] = False
        n_opt = sum(st[0].numel() for sts in opt_state.values() for st in sts) // max(len(projs[0][1]), 1)
        paged_info = {"ms_per_step_without_optimizer": round(ms_off / args.steps, 5),
                      "optimizer_throughput_loss_pct": round(100.0 * (1.0 - ms_off / ms_total), 2),
                      "optimizer": ("AdamW (lr 1e-4, wd 0.01) on the host CPU (qlora_adamw_step_host, the page's "
                                    "placement): float32 dA, dB copied to pinned host memory, master, m and v of every A "
                                    "and B in pinned host memory, the bf16 parameters copied back; a worker thread runs "
                                    "the host steps beside the next projection's kernels" if args.paging == "host" else
                                    "AdamW (lr 1e-4, wd 0.01): m and v of every A and B in pinned host memory, float32 "
                                    "master on the device, updated by qlora_adamw_step on a side stream beside the next "
                                    "projection; "
                                    + ("each state page copied to the device and back by DMA around the update"
                                       if args.paging == "dma" else "the kernel reads and writes host memory in place")),
                      "adapter_params_per_step": n_opt,
                      "host_link_bytes_per_step": (6 * n_opt if args.paging == "host" else 16 * n_opt)}
    else:
        ms_total, have_graphs = measure()
    ms_step = ms_total / args.steps
    graphs = {chunk: None} if have_graphs else {}

    fb = sum(fwd_bytes(p.d_out, p.d_in, p.r, T) for p, *_, T, _ in calls)
    ff = sum(fwd_flops(p.d_out, p.d_in, p.r, T) for p, *_, T, _ in calls)
    bb = sum(bwd_bytes(p.d_out, p.d_in, p.r, T) for p, *_, T, _ in calls) if bw else 0
    bf = sum(bwd_flops(p.d_out, p.d_in, p.r, T) for p, *_, T, _ in calls) if bw else 0
    wbytes_step = sum(weight_bytes(p.d_out, p.d_in) for p, *_ in calls) * (2 if bw else 1)
    wgbs = wbytes_step / (ms_step * 1e-3) / 1e9
    tflops = (ff + bf) / (ms_step * 1e-3) / 1e12

    if not bw:
        # every call is one launch of the weight-streaming kernel (T <= 16): its mean launch duration over
        # the timed region is the region's length over the launches in it
        launches = args.steps * len(calls)
        us_launch = ms_total * 1e3 / launches
        achieved = (fb / len(calls)) / (us_launch * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic() if wname == "llama7b_skinny" and not ABSMAX_STORAGE[0] else None,
                "kernel": "k_gemv_fwd (qlora_forward, T <= 16)",
                "bytes_per_launch": round(fb / len(calls)), "us_per_launch": round(us_launch, 3),
                "launches": launches}
        label_traffic(roof)
    else:
        achieved = (ff + bf) / (ms_step * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "whole forward + backward step (all kernels)"}

    per_call = per_call_times(torch, dev, calls, run_call, chunk) if not (args.no_graph or args.no_per_call) else []
    grouped = (grouped_times(torch, dev, q, calls, nT, chunk, args.steps, fb, wbytes_step,
                             recorded_traffic(key="grouped_traffic_bytes_per_launch")
                             if wname == "llama7b_skinny" and not ABSMAX_STORAGE[0] else None)
               if not (bw or args.no_graph) else None)

    if args.copy_calibration:
        copy_calibration(torch, dev)

    cpu = None
    if not args.no_cpu_baseline and not bw:
        cpu = cpu_baseline(args, wl, seed_cfg, wbytes_step)
    elif not args.no_cpu_baseline:
        cpu = cpu_baseline_train(args, wl, seed_cfg, ms_step, ff + bf)

    line = {
        "metric": METRIC,
        "value": round(wgbs, 1),
        "unit": "GB/s (NF4 weight bytes per second)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02^2) weights and adapters, N(0,1) tokens)",
        "config": {"workload": wl.description, "projections": [f"{p.d_out}x{p.d_in}" for p in wl.projections],
                   "tokens": list(wl.tokens), "lora_r": wl.projections[0].r, "lora_alpha": wl.projections[0].alpha,
                   "backward": bw, "graph_steps": chunk if graphs else 0,
                   "weight_storage": ("NF4 + float32 absmax per 64-weight block (4.5 bits)" if ABSMAX_STORAGE[0]
                                      else "NF4 + double-quantized block scales (4.127 bits)"),
                   "weight_copies_per_projection": len(projs[0][1]),
                   **({"layers_in_stack": wl.layers, "layers_per_step": 1} if wl.layers > 1 else {})},
        "tflops": round(tflops, 3),
        "total_GBs": round((fb + bb) / (ms_step * 1e-3) / 1e9, 1),
        "roofline": roof,
        "per_call": per_call,
        **({"grouped": grouped} if grouped else {}),
        "cpu_baseline": cpu,
    }
    if paged_info:
        line["config"]["workload"] = wl.description + ", with a paged AdamW update of every A and B"
        line["config"].update(paged_info)
    if emit:
        print(json.dumps(line), flush=True)
    return line


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_k_gemv_fwd_llama7b_skinny.json")
FWD_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_qlora_forward_65b_layer.json")


def label_traffic(roof, record=TRAFFIC_RECORD):
    """A traffic figure in a roofline object is a recorded one: say so, and from where."""
    if roof.get("traffic") is not None:
        roof["traffic_source"] = ("recorded, not measured in this run: %s (FETCH_SIZE and WRITE_SIZE counter runs, "
                                  "scaled by a copy calibration; the sources it was taken on are hash-checked)"
                                  % os.path.relpath(record, ROOT))
    return roof


def recorded_traffic(record=TRAFFIC_RECORD, key="traffic_bytes_per_launch"):
    """HBM bytes per launch recorded from FETCH_SIZE / WRITE_SIZE counter runs (the record names the command and
    the sources it was taken on), or None when the record is missing or those sources changed since."""
    import hashlib
    try:
        rec = json.load(open(record))
        h = hashlib.sha256()
        for f in rec["sources"]:
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return int(rec[key])
    except (OSError, KeyError, ValueError):
        return None


def grouped_times(torch, dev, q, calls, nT, chunk, steps, fb_step, wbytes_step, traffic=None):
    """The same step with its calls, which are independent, given to qlora_forward_many: one launch per step
    when they share a kernel variant. Graph-timed like the step, on the same rotating weight copies and inputs."""
    ws = torch.zeros(q.qlora_forward_many_workspace_bytes(len(calls)), dtype=torch.uint8, device=dev)

    def body(s):
        jobs = []
        for p, copies, x, dy, h, g, T, ti in calls:
            wc, A, B = copies[(s * nT + ti) % len(copies)]
            jobs.append({"w": wc, "x": x, "A": A, "B": B, "alpha": p.alpha, "h": h})
        q.qlora_forward_many(jobs, ws=ws)

    ms, n = _timed_graph(torch, dev, body, steps, chunk)
    achieved = fb_step / (ms * 1e-3) / 1e9
    return {"ms_per_step": round(ms, 5), "steps": n, "weight_GBs": round(wbytes_step / (ms * 1e-3) / 1e9, 1),
            "roofline": label_traffic({"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                         "kernel": ("k_gemv_fwd_many (qlora_forward_many: one launch per kernel variant among "
                                    "the step's calls)"),
                         "bytes_per_step": round(fb_step), "us_per_step": round(ms * 1e3, 3)}),
            "fallbacks": q.qlora_workspace_fallbacks(ws)}


def per_call_times(torch, dev, calls, run_call, chunk):
    """Each call shape alone: a graph of `chunk`*3 launches of it over rotating copies, replayed 5 times."""
    rows = []
    side = torch.cuda.Stream(dev)
    stream = torch.cuda.current_stream(dev)
    for c in calls:
        p, copies, x, dy, h, g, T, ti = c
        n = min(len(copies), 3 * chunk)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):
            for k in range(n):
                run_call(p, copies, x, dy, h, g, T, ti, k)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(5):
            gr.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / (5 * n)
        b = fwd_bytes(p.d_out, p.d_in, p.r, T)
        rows.append({"proj": f"{p.d_out}x{p.d_in}", "T": T, "r": p.r, "us": round(us, 2),
                     "GBs": round(b / (us * 1e-6) / 1e9, 1),
                     "weight_GBs": round(weight_bytes(p.d_out, p.d_in) / (us * 1e-6) / 1e9, 1)})
        del gr
    return rows


def cpu_baseline(args, wl, seed_cfg, wbytes_step):
    """The CPU oracle timed on a bounded sample of the same workload (host cores of this machine)."""
    import oracle
    from bit_quantized_finetuning_amd import synth

    threads, blas, model = _host_info()
    # Per projection: quantized once (not timed, as on the GPU); timed: restore + forward for every T.
    prepared = []
    for pi, p in enumerate(wl.projections):
        W = synth.weight(seed_cfg, pi, p.d_out, p.d_in, wl.weight_dtype)
        if ABSMAX_STORAGE[0]:
            codes, S = oracle.quantize_absmax(W)
            q2 = None
        else:
            codes, q2, S = oracle.quantize(W)
        (A, _), (B, _) = synth.adapters(seed_cfg, pi, p.d_out, p.d_in, p.r)
        xs = {T: synth.tokens(seed_cfg, pi, T, p.d_in)[0] for T in wl.tokens}
        prepared.append((p, codes, q2, S, A, B, xs))
    done_steps = 0
    t_start = time.perf_counter()
    while True:
        for p, codes, q2, S, A, B, xs in prepared:
            if q2 is None:
                _, wb = oracle.dequantize_absmax(codes, S, p.d_out, p.d_in)
            else:
                _, wb = oracle.dequantize(codes, q2, S, p.d_out, p.d_in)
            for T in wl.tokens:
                oracle.lora_forward(wb, xs[T], A, B, p.alpha, p.r)
        done_steps += 1
        el = time.perf_counter() - t_start
        if el >= args.cpu_seconds:
            break
    sec_step = el / done_steps
    return {"value": round(wbytes_step / sec_step / 1e9, 4), "unit": "GB/s (NF4 weight bytes per second)",
            "cores": threads, "kind": "oracle",
            "sample": f"{done_steps} full step(s) of the same workload (restore + float64 forward of every "
                      f"projection and token count; quantization untimed), {el:.1f} s",
            "ms_per_step": round(sec_step * 1e3, 1), "cpu": model, "blas": blas}


def _host_info():
    """Threads the oracle's BLAS uses, the BLAS library, and the host CPU model."""
    threads, blas = os.cpu_count(), "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] + [1])
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info}))
    except Exception:  # pragma: no cover
        pass
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return threads, blas, model


def cpu_baseline_train(args, wl, seed_cfg, ms_step_gpu, flops_step, rows=256, t_sample=128, layers=1):
    """The CPU oracle on a bounded sample of a forward + backward workload, scaled to one step.

    Sample: for each distinct projection shape, a slice of `rows` output rows of its weight (same distribution),
    quantized untimed (at model load, as on the GPU), then timed: the restore of the slice, and the float64
    forward and backward at `t_sample` tokens. The oracle's work is linear in the rows (restore, both products)
    and the products are linear in the tokens, so the step time is estimated as
        sum over projections of (restore time + product time * T / t_sample) * d_out / rows
    (the adapter terms, under 2 % of the work at these ranks, are scaled the same way)."""
    import oracle
    from bit_quantized_finetuning_amd import synth

    (T,) = wl.tokens
    shapes = {}
    for pi, p in enumerate(wl.projections):
        shapes.setdefault((p.d_out, p.d_in, p.r, p.alpha), []).append(pi)
    prepared = []
    for (d_out, d_in, r, alpha), pis in shapes.items():
        pi = pis[0]
        rr = min(rows, d_out)
        W = synth.weight(seed_cfg, pi, rr, d_in, wl.weight_dtype)
        codes, q2, S = oracle.quantize(W)
        A = B = None
        if r > 0:
            (A, _), (B, _) = synth.adapters(seed_cfg, pi, d_out, d_in, r)
            B = B[:rr]
        ts = min(t_sample, T)
        x = synth.tokens(seed_cfg, pi, ts, d_in)[0]
        dy = synth.upstream_grad(seed_cfg, pi, ts, rr)[0]
        prepared.append((len(pis), d_out, d_in, r, alpha, rr, ts, codes, q2, S, A, B, x, dy))
    t_restore = [0.0] * len(prepared)
    t_prod = [0.0] * len(prepared)
    passes = 0
    t_start = time.perf_counter()
    while True:
        for k, (units, d_out, d_in, r, alpha, rr, ts, codes, q2, S, A, B, x, dy) in enumerate(prepared):
            t0 = time.perf_counter()
            _, wb = oracle.dequantize(codes, q2, S, rr, d_in)
            t1 = time.perf_counter()
            oracle.lora_forward(wb, x, A, B, alpha, r)
            oracle.lora_backward(wb, x, dy, A, B, alpha, r)
            t2 = time.perf_counter()
            t_restore[k] += t1 - t0
            t_prod[k] += t2 - t1
        passes += 1
        el = time.perf_counter() - t_start
        if el >= args.cpu_seconds:
            break
    sec_step = 0.0
    for k, (units, d_out, d_in, r, alpha, rr, ts, *_rest) in enumerate(prepared):
        sec_step += units * (t_restore[k] + t_prod[k] * T / ts) / passes * d_out / rr
    sec_step *= layers
    threads, blas, model = _host_info()
    return {"value": round(flops_step / sec_step / 1e12, 6), "unit": "TFLOP/s (same flops per step as the GPU line)",
            "cores": threads, "kind": "oracle", "scaled": True,
            "sample": f"{passes} pass(es) over {len(prepared)} distinct projection shapes: a {rows}-row slice of "
                      f"each weight, restore + float64 forward and backward at {t_sample} tokens, {el:.1f} s; "
                      f"scaled linearly to all rows, {T} tokens and every projection of the step"
                      + (f" ({layers} layers)" if layers > 1 else ""),
            "s_per_step": round(sec_step, 2), "gpu_speedup": round(sec_step / (ms_step_gpu * 1e-3), 1),
            "cpu": model, "blas": blas}


def _timed_graph(torch, dev, body, steps, chunk):
    """Capture `body(k)` for k in 0..chunk-1 into a graph; return ms per step over `steps` steps
    (HIP events on the replay stream, a whole number of replays)."""
    side = torch.cuda.Stream(dev)  # default priority
    for k in range(chunk):
        body(k)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for k in range(chunk):
            body(k)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    reps = max(1, (steps + chunk - 1) // chunk)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (reps * chunk), reps * chunk


def _line(args, value, unit, ms_step, steps, workload, roof, cpu, extra=None, higher=True):
    line = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 5), "higher_is_better": higher, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic (seeded N(0,0.02^2) weights and adapters)",
            "config": {"workload": workload}, "roofline": roof, "cpu_baseline": cpu}
    line.update(extra or {})
    print(json.dumps(line), flush=True)


def merge_bytes(d_out, d_in, r):
    """Algorithmic HBM bytes of one merge: NF4 weight + A, B in; bf16 merged weight out."""
    return weight_bytes(d_out, d_in) + 2 * r * (d_in + d_out) + 2 * d_out * d_in


def bench_merge(args, torch, q, synth, dev):
    """Merge for export of the two LLaMA-7B projections (r = 64): one step = both merges, each one launch of
    k_merge; every launch of a graph reads its own weight copy and writes its own output."""
    wl = synth.WORKLOADS["llama7b_skinny"]
    cfg = synth.WORKLOAD_SEED["llama7b_skinny"]
    chunk = min(args.chunk, 10)
    items = []
    for pi, p in enumerate(wl.projections):
        W = torch.from_numpy(synth.weight(cfg, pi, p.d_out, p.d_in)).to(dev)
        w0 = q.qlora_quantize(W)
        del W
        (_, A_bits), (_, B_bits) = synth.adapters(cfg, pi, p.d_out, p.d_in, p.r)
        A = torch.from_numpy(np.ascontiguousarray(A_bits).view(np.int16)).view(torch.bfloat16).to(dev)
        B = torch.from_numpy(np.ascontiguousarray(B_bits).view(np.int16)).view(torch.bfloat16).to(dev)
        ws = [(q.NF4Weight(p.d_out, p.d_in, w0.codes.clone(), w0.qscale.clone(), w0.smax.clone()),
               torch.empty(p.d_out, p.d_in, dtype=torch.bfloat16, device=dev)) for _ in range(chunk)]
        items.append((p, A, B, ws))
    for _ in range(max(args.warmup, 1)):
        for p, A, B, ws in items:
            q.qlora_merge(ws[0][0], A, B, p.alpha, out=ws[0][1])

    def body(k):
        for p, A, B, ws in items:
            wc, out = ws[k]
            q.qlora_merge(wc, A, B, p.alpha, out=out)

    ms_step, steps = _timed_graph(torch, dev, body, args.steps, chunk)
    nbytes = sum(merge_bytes(p.d_out, p.d_in, p.r) for p, *_ in items)
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    us_launch = ms_step * 1e3 / len(items)
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "k_merge (qlora_merge)",
            "bytes_per_launch": round(nbytes / len(items)), "us_per_launch": round(us_launch, 3),
            "launches": steps * len(items)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:  # pragma: no cover
            threads = os.cpu_count()
        rows, prepared = 256, []
        for pi, p in enumerate(wl.projections):
            W = synth.weight(cfg, pi, rows, p.d_in)  # a 256-row weight of the same distribution
            codes, q2, S = oracle.quantize(W)
            (A, _), (B, _) = synth.adapters(cfg, pi, p.d_out, p.d_in, p.r)
            prepared.append((p, codes, q2, S, A, B[:rows]))
        done, t_start = 0, time.perf_counter()
        while True:
            for p, codes, q2, S, A, Bs in prepared:
                _, wb = oracle.dequantize(codes, q2, S, rows, p.d_in)
                oracle.lora_merge(wb, A, Bs, p.alpha, p.r)
            done += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds:
                break
        sb = sum(merge_bytes(rows, p.d_in, p.r) for p, *_ in prepared)
        cpu = {"value": round(sb * done / el / 1e9, 4), "unit": "GB/s (merge algorithmic bytes per second)",
               "cores": threads, "kind": "oracle",
               "sample": f"{done} pass(es) over {rows}-row slices of both projections (restore + float64 merge), "
                         f"{el:.1f} s"}
    _line(args, round(gbs, 1), "GB/s (merge algorithmic bytes per second)", ms_step, steps,
          "merge for export, bf16(W_hat + (alpha/r) B A), LLaMA-7B projections 4096x4096 and 11008x4096, "
          "LoRA r=64 alpha=16", roof, cpu,
          {"per_launch_us": round(us_launch, 3), "graph_steps": chunk})


def bench_quantize_stack(args, torch, q, synth, dev):
    """One pass quantizing all 280 bf16 weights of the 14B-style stack (40 layers x q, k, v, o, gate, up, down):
    one step = the whole pass, one qlora_quantize_many call (9 launches of k_quantize, 32 weights each); the
    same pass with one qlora_quantize call per weight is timed beside it. Weights come from a seeded device generator
    (N(0, 0.02^2) rounded to bf16); 13.2 G weights are too many to draw on the host."""
    wl = synth.WORKLOADS["14b_stack"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.WORKLOAD_SEED["14b_stack"])
    Ws, outs = [], []
    for layer in range(wl.layers):
        for p in wl.projections:
            W = torch.empty(p.d_out, p.d_in, dtype=torch.bfloat16, device=dev)
            W.normal_(0.0, 0.02, generator=gen)
            Ws.append(W)
            outs.append(q.NF4Weight.empty(p.d_out, p.d_in, dev))
    torch.cuda.synchronize()

    def body(k):
        q.qlora_quantize_many(Ws, outs)

    def body_single(k):
        for W, o in zip(Ws, outs):
            q.qlora_quantize(W, out=o)

    ms_step, steps = _timed_graph(torch, dev, body, args.steps, 1)
    ms_single, _ = _timed_graph(torch, dev, body_single, args.steps, 1)
    launches = -(-len(Ws) // 32)  # 32 weights per launch
    n = sum(W.numel() for W in Ws)
    nbytes = sum(2 * W.numel() + q.qlora_storage_bytes(W.shape[0], W.shape[1]) for W in Ws)
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "k_quantize<bf16> (qlora_quantize_many: 32 weights per launch)",
            "bytes_per_launch": round(nbytes / launches), "us_per_launch": round(ms_step * 1e3 / launches, 3),
            "launches": steps * launches}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:  # pragma: no cover
            threads = os.cpu_count()
        Wh = synth.weight(synth.WORKLOAD_SEED["14b_stack"], 0, 256, 5120, "bf16")
        done, t_start = 0, time.perf_counter()
        while True:
            oracle.quantize(Wh)
            done += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds:
                break
        sb = (2 * Wh.size + q.qlora_storage_bytes(256, 5120)) * done
        cpu = {"value": round(sb / el / 1e9, 4), "unit": "GB/s (quantize algorithmic bytes per second)",
               "cores": threads, "kind": "oracle",
               "sample": f"{done} quantization(s) of a 256x5120 bf16 slice, {el:.1f} s"}
    _line(args, round(gbs, 1), "GB/s (quantize algorithmic bytes per second: bf16 in, NF4 + double quant out)",
          ms_step, steps, f"one-pass quantize of the 14B-style stack: {len(Ws)} bf16 weights, {n / 1e9:.2f} G "
          "parameters", roof, cpu, {"weights": len(Ws), "params": n, "ms_per_pass": round(ms_step, 3),
                                    "ms_per_pass_one_call_per_weight": round(ms_single, 3),
                                    "GBs_one_call_per_weight": round(nbytes / (ms_single * 1e-3) / 1e9, 1)})


if __name__ == "__main__":
    main()
