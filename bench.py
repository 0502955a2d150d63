#!/usr/bin/env python3
"""Benchmark of the QLoRA frozen-NF4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama7b_skinny]

Default workload (LLaMA-7B-shaped projections, the weight-streaming regime):
4096x4096 and 11008x4096 NF4 + double-quant weights (W ~ N(0, 0.02^2)), LoRA r=64
alpha=16 (A, B ~ N(0, 0.02^2) bf16), x ~ N(0, 1) bf16 with 1, 4 and 16 tokens.
One step = the forward h = dequant(W) x + (alpha/r) B A x of both projections at
all three token counts (6 calls, each one launch of the weight-streaming kernel).
Quantization happens once before timing, as at model load.

Timing. The steps are captured into HIP graphs (a chunk of C steps, replayed),
so that the host's per-call cost does not leave the GPU idle between 8-15 us
kernels; HIP events on the replay stream bracket exactly K steps. Every call of
a chunk reads its own copy of the quantized weight and adapters, so between two
reads of one copy more than 600 MB of other weights stream by and HBM, not the
256 MB Infinity Cache, serves the weight stream.

Printed: one JSON line. `value` is the weight GB/s (packed codes + scale codes +
group maxima per second); `roofline` is the weight-streaming kernel's algorithmic
bytes per launch over its mean launch duration in the timed region; `cpu_baseline`
is the CPU oracle timed on a bounded sample of the same workload.

Other workloads are records, not the headline line:
  65b_skinny  the same weight-streaming forward (T = 1, 16; r = 64) on the 65B layer's
      8192x8192, 22016x8192 and 8192x22016 weights (34-93 MB per call);
  13b_4096tok / 65b_layer / linear1024 / 14b_stack  the MFMA GEMM regime
      (forward + backward; 14b_stack: one of the 40 identical layers of the
      14B-style stack, bf16 source weights, 2048 tokens, LoRA r=8 on q and v);
  14b_stack_fused  the same layer with q/k/v and gate/up each stacked into one
      call that reads its input once (q and v adapters as one block-diagonal
      rank-16 pair);
  14b_quantize  one pass quantizing all 280 bf16 weights of the 14B-style stack
      (13.2 G parameters, generated on the device from a seeded generator);
  merge_llama7b  merge for export, bf16(W_hat + (alpha/r) B A), of the two
      LLaMA-7B projections with r = 64;
  13b_paged_adamw  the 13b_4096tok step, timed without and with an AdamW update
      of every A and B whose moments m, v sit in pinned host memory (float32
      master on the device); the update of a projection runs on a side stream
      beside the next projection's forward and backward. Reported: the step with
      the update and the throughput lost to it.
  --storage absmax  any forward/backward workload on absmax-only weights (one
      float32 scale per 64-weight block, 4.5 bits) instead of double quant.
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
WORKLOAD_CHOICES = ["llama7b_skinny", "65b_skinny", "linear1024", "13b_4096tok", "65b_layer", "14b_stack", "14b_stack_fused",
                    "14b_quantize",
                    "merge_llama7b", "13b_paged_adamw"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llama7b_skinny", choices=WORKLOAD_CHOICES)
    p.add_argument("--chunk", type=int, default=20, help="steps per captured graph")
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying graphs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-per-call", action="store_true", help="skip the per-call-shape timings (profiling runs)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--storage", default="dq", choices=["dq", "absmax"],
                   help="weight storage: NF4 with double-quantized scales (4.13 bits) or float32 block absmax (4.5)")
    p.add_argument("--paging", default="zerocopy", choices=["zerocopy", "dma"],
                   help="13b_paged_adamw: update m, v in host memory in place, or copy each page to the device and back")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy (reference for HBM counter scaling)")
    return p.parse_args()


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
    paged = args.workload == "13b_paged_adamw"
    wname = "13b_4096tok" if paged else args.workload
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
    if paged:
        for pi, (p, copies, *_rest) in enumerate(projs):
            for ci, (wc, A, B) in enumerate(copies):
                if A is None:
                    continue
                st = []
                for t in (A, B):
                    master = t.float()
                    st.append((t, master, torch.zeros(t.numel(), dtype=torch.float32).pin_memory(),
                               torch.zeros(t.numel(), dtype=torch.float32).pin_memory()))
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
            torch.cuda.current_stream(dev).wait_event(opt_pending.pop((pi, ci)))
        dX, dA, dB, u = g
        ur = u if p.r > 0 else None
        q.qlora_forward(wc, x, A, B, p.alpha, h=h, u=ur)
        q.qlora_backward(wc, x, dy, A, B, p.alpha, u_saved=ur, dX=dX, dA=dA if p.r > 0 else None,
                         dB=dB if p.r > 0 else None)
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
                      "optimizer": "AdamW (lr 1e-4, wd 0.01): m and v of every A and B in pinned host memory, float32 "
                                   "master on the device, updated by qlora_adamw_step on a side stream beside the next "
                                   "projection; "
                                   + ("each state page copied to the device and back by DMA around the update"
                                      if args.paging == "dma" else "the kernel reads and writes host memory in place"),
                      "adapter_params_per_step": n_opt,
                      "host_link_bytes_per_step": 16 * n_opt}
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
                "traffic": recorded_traffic() if args.workload == "llama7b_skinny" else None,
                "kernel": "k_gemv_fwd (qlora_forward, T <= 16)",
                "bytes_per_launch": round(fb / len(calls)), "us_per_launch": round(us_launch, 3),
                "launches": launches}
    else:
        achieved = (ff + bf) / (ms_step * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "whole forward + backward step (all kernels)"}

    per_call = per_call_times(torch, dev, calls, run_call, chunk) if not (args.no_graph or args.no_per_call) else []

    if args.copy_calibration:
        # a plain device copy of known size (256 MiB read + 256 MiB written per launch), the reference that
        # scales the HBM byte counters
        a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if not args.no_cpu_baseline and not bw:
        cpu = cpu_baseline(args, wl, seed_cfg, wbytes_step)

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
        "cpu_baseline": cpu,
    }
    if paged_info:
        line["config"]["workload"] = wl.description + ", with a paged AdamW update of every A and B"
        line["config"].update(paged_info)
    print(json.dumps(line), flush=True)


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_k_gemv_fwd_llama7b_skinny.json")


def recorded_traffic():
    """HBM bytes per launch of the weight-streaming kernel from the recorded FETCH_SIZE / WRITE_SIZE runs,
    or None when the record is missing or the kernel's sources changed since the counters were taken."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_RECORD))
        h = hashlib.sha256()
        for f in rec["sources"]:
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


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

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
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
            "ms_per_step": round(sec_step * 1e3, 1)}


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
    one step = the whole pass, 280 launches of k_quantize. Weights come from a seeded device generator
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
        for W, o in zip(Ws, outs):
            q.qlora_quantize(W, out=o)

    ms_step, steps = _timed_graph(torch, dev, body, args.steps, 1)
    n = sum(W.numel() for W in Ws)
    nbytes = sum(2 * W.numel() + q.qlora_storage_bytes(W.shape[0], W.shape[1]) for W in Ws)
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "k_quantize<bf16> (qlora_quantize)",
            "bytes_per_launch": round(nbytes / len(Ws)), "us_per_launch": round(ms_step * 1e3 / len(Ws), 3),
            "launches": steps * len(Ws)}
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
          "parameters", roof, cpu, {"weights": len(Ws), "params": n, "ms_per_pass": round(ms_step, 3)})


if __name__ == "__main__":
    main()
