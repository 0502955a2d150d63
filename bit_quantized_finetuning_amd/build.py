"""Build the gfx950 HIP library libqlora.so in-tree with hipcc.

    python -m bit_quantized_finetuning_amd.build [--verbose]

Compiles every source under csrc/ (one object each, in parallel, under _build/)
and links one shared library next to this file.
Flags: correctly rounded float32 division (the quantizer's normalization must
match an IEEE divide bit for bit), no packed-FP32 instruction selection, and no
fast-math.
"""

from __future__ import annotations

import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqlora.so")

SOURCES = ["api.cpp", "quantize.hip", "lora_small.hip", "gemv.hip", "gemm.hip", "lora_grad.hip", "lora_wide.hip", "merge.hip", "adamw.hip", "adamw_host.cpp", "scratch.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3",
    "-std=c++17",
    "--offload-arch=gfx950",
    "-fPIC",
    "-shared",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source to an object (in parallel, under _build/), then link libqlora.so."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = [f for f in FLAGS if f != "-shared"] + list(extra_flags or []) + ["-I", os.path.join(ROOT, "include")]
    t0 = time.time()

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        return obj, res, cmd

    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(compile_one, SOURCES))
    msgs = []
    for obj, res, cmd in results:
        out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                        if "packed-fp32-ops' is not a recognized feature" not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{out}")
        if out.strip():
            msgs.append(out)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [r[0] for r in results]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv or "-v" in sys.argv)
