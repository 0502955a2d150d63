#!/usr/bin/env python3
"""Benchmark of the QLoRA frozen-NF4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

Default workload (LLaMA-7B-shaped projections, the weight-streaming regime):
4096x4096 and 11008x4096 NF4 + double-quant weights (W ~ N(0, 0.02^2)), LoRA r=64
alpha=16 (A, B ~ N(0, 0.02^2) bf16), x ~ N(0, 1) bf16 with 1, 4 and 16 tokens.
One step = the forward h = dequant(W) x + (alpha/r) B A x of both projections at
all three token counts (6 calls). The quantization happens once before timing,
as at model load. Every step reads a different copy of the quantized weights
and adapters (16 copies, ~560 MB) so that HBM, not the 256 MB Infinity Cache,
serves the weight stream.

Printed: one JSON line with the headline metric (weight GB/s: packed codes +
scale codes + group maxima per second), the roofline of the dominant call
measured with HIP events on the stream it runs on, and the CPU oracle timed on
a bounded sample of the same workload.

Other workloads (--workload c3 / c4 / c1) time the MFMA GEMM regime (T = 4096
or 16, forward + backward) for the DESIGN/profiles record; they are not the
headline line.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4"])
    p.add_argument("--rotate", type=int, default=16, help="independent weight copies cycled through")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy (reference for HBM counter scaling)")
    return p.parse_args()


def weight_bytes(d_out, d_in):
    n = d_out * d_in
    nb = n // 64
    return n // 2 + nb + 4 * ((nb + 255) // 256)


def call_bytes(d_out, d_in, r, T, backward=False):
    """Algorithmic HBM bytes of one call: NF4 weight + adapters + activations in and out."""
    b = weight_bytes(d_out, d_in) + 2 * r * (d_in + d_out) + 2 * T * (d_in + d_out)
    if backward:
        # dY in, dX out, x in again, dA/dB out (f32)
        b += weight_bytes(d_out, d_in) + 2 * r * (d_in + d_out) + 2 * T * (d_in + d_out) + 2 * T * d_in \
            + 4 * r * (d_in + d_out)
    return b


def call_flops(d_out, d_in, r, T, backward=False):
    f = 2 * T * d_in * d_out + 2 * T * r * (d_in + d_out)
    if backward:
        f += 2 * T * d_in * d_out + 4 * T * r * (d_in + d_out)
    return f


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the layer shards as data parallel across GPUs, which is not built here).", flush=True)
        sys.exit(2)

    import torch

    from bit_quantized_finetuning_amd import qlora as q
    from bit_quantized_finetuning_amd import synth

    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    cfg = synth.CONFIG_INDEX[args.workload]

    def dev16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs: quantize once, replicate the quantized weight for MALL rotation
    projs = []
    for pi, p in enumerate(wl.projections):
        W = torch.from_numpy(synth.weight(cfg, pi, p.d_out, p.d_in, wl.weight_dtype)).to(dev)
        w0 = q.qlora_quantize(W)
        del W
        (A, A_bits), (B, B_bits) = synth.adapters(cfg, pi, p.d_out, p.d_in, p.r)
        A0, B0 = dev16(A_bits), dev16(B_bits)
        ncopy = args.rotate if not wl.backward else 2
        copies = []
        for c in range(ncopy):
            wc = q.NF4Weight(p.d_out, p.d_in, w0.codes.clone(), w0.qscale.clone(), w0.smax.clone())
            copies.append((wc, A0.clone(), B0.clone()))
        xs = {T: dev16(synth.tokens(cfg, pi, T, p.d_in)[1]) for T in wl.tokens}
        dys = {T: dev16(synth.upstream_grad(cfg, pi, T, p.d_out)[1]) for T in wl.tokens} if wl.backward else {}
        projs.append((p, copies, xs, dys))
    torch.cuda.synchronize()

    calls = []   # (proj, T)
    for p, copies, xs, dys in projs:
        for T in wl.tokens:
            calls.append((p, copies, xs[T], dys.get(T), T))

    stream = torch.cuda.current_stream(dev)
    outs = {}

    def one_call(i, p, copies, x, dy, T, step):
        wc, A, B = copies[step % len(copies)]
        key = (i, T)
        if wl.backward:
            h, u = q.qlora_forward(wc, x, A, B, p.alpha, save_u=True, h=outs.get(key))
            outs[key] = h
            q.qlora_backward(wc, x, dy, A, B, p.alpha, u_saved=u)
        else:
            h, _ = q.qlora_forward(wc, x, A, B, p.alpha, h=outs.get(key))
            outs[key] = h

    def step(s, events=None):
        for i, (p, copies, x, dy, T) in enumerate(calls):
            if events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                one_call(i, p, copies, x, dy, T, s)
                e1.record(stream)
                events.append((i, e0, e1))
            else:
                one_call(i, p, copies, x, dy, T, s)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    # timed region: whole steps (no per-call events) ...
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for s in range(args.steps):
        step(args.warmup + s)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # ... and the same steps again with HIP events around every call on its stream
    events = []
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(args.warmup + s, events)
    torch.cuda.synchronize()
    per_call_ms = [[] for _ in calls]
    for i, e0, e1 in events:
        per_call_ms[i].append(e0.elapsed_time(e1))

    bw = bool(wl.backward)
    wbytes_step = sum(weight_bytes(p.d_out, p.d_in) * (2 if bw else 1) for p, _, _, _, _ in calls)
    bytes_step = sum(call_bytes(p.d_out, p.d_in, p.r, T, bw) for p, _, _, _, T in calls)
    flops_step = sum(call_flops(p.d_out, p.d_in, p.r, T, bw) for p, _, _, _, T in calls)
    wgbs = wbytes_step / (ms_step * 1e-3) / 1e9
    tflops = flops_step / (ms_step * 1e-3) / 1e12

    call_rows = []
    for i, (p, _, _, _, T) in enumerate(calls):
        ms = float(np.mean(per_call_ms[i]))
        b = call_bytes(p.d_out, p.d_in, p.r, T, bw)
        f = call_flops(p.d_out, p.d_in, p.r, T, bw)
        call_rows.append({"proj": f"{p.d_out}x{p.d_in}", "T": T, "r": p.r, "us": round(ms * 1e3, 2),
                          "GBs": round(b / (ms * 1e-3) / 1e9, 1), "TFLOPs": round(f / (ms * 1e-3) / 1e12, 2)})

    if not bw:
        # memory-bound regime: dominant call = the forward that moves the most bytes
        tot_b = sum(call_bytes(p.d_out, p.d_in, p.r, T) for p, _, _, _, T in calls)
        tot_ms = sum(float(np.mean(per_call_ms[i])) for i in range(len(calls)))
        achieved = tot_b / (tot_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "qlora_forward T<=16 (k_lora_small + k_gemv_fwd), mean over the 6 calls",
                "per_call": call_rows}
    else:
        tot_f = sum(call_flops(p.d_out, p.d_in, p.r, T, True) for p, _, _, _, T in calls)
        tot_ms = sum(float(np.mean(per_call_ms[i])) for i in range(len(calls)))
        achieved = tot_f / (tot_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "qlora_forward + qlora_backward per projection", "per_call": call_rows}

    if args.copy_calibration:
        a = torch.empty(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if not args.no_cpu_baseline and not wl.backward:
        cpu = cpu_baseline(args, wl, cfg, calls, wbytes_step, bytes_step)

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
                   "backward": bw, "weight_copies_rotated": len(projs[0][1])},
        "tflops": round(tflops, 3),
        "total_GBs": round(bytes_step / (ms_step * 1e-3) / 1e9, 1),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(args, wl, cfg, calls, wbytes_step, bytes_step):
    """The CPU oracle timed on a bounded sample of the same workload (host cores of this machine)."""
    import oracle
    from bit_quantized_finetuning_amd import synth

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    # Per projection: quantized once (not timed, as on the GPU); timed: restore + forward for every T.
    prepared = []
    for pi, p in enumerate(wl.projections):
        W = synth.weight(cfg, pi, p.d_out, p.d_in, wl.weight_dtype)
        codes, q2, S = oracle.quantize(W)
        (A, _), (B, _) = synth.adapters(cfg, pi, p.d_out, p.d_in, p.r)
        xs = {T: synth.tokens(cfg, pi, T, p.d_in)[0] for T in wl.tokens}
        prepared.append((p, codes, q2, S, A, B, xs))
    done_steps = 0
    t_start = time.perf_counter()
    while True:
        for p, codes, q2, S, A, B, xs in prepared:
            _, wb = oracle.dequantize(codes, q2, S, p.d_out, p.d_in)
            for T in wl.tokens:
                oracle.lora_forward(wb, xs[T], A, B, p.alpha, p.r)
        done_steps += 1
        el = time.perf_counter() - t_start
        if el >= args.cpu_seconds or wl.backward:
            break
    sec_step = el / done_steps
    return {"value": round(wbytes_step / sec_step / 1e9, 4), "unit": "GB/s (NF4 weight bytes per second)",
            "cores": threads, "kind": "oracle",
            "sample": f"{done_steps} full step(s) of the same workload (restore + float64 forward of every "
                      f"projection and token count; quantization untimed), {el:.1f} s",
            "ms_per_step": round(sec_step * 1e3, 1)}


if __name__ == "__main__":
    main()
