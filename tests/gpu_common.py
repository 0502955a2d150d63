"""Shared helpers for the GPU parity tests: inputs from the seeded generator, oracle
references, and the tolerance test of the floating-point outputs.

Tolerance for bf16-in / fp32-accumulate outputs and gradients (h, dX, dA, dB),
against the float64 oracle:
    relative Frobenius error      <= 5e-3
    max-abs error                 <= 1e-2 * max|ref|
Quantized codes, scale codes, group maxima and restored weights are compared bit
for bit.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from bit_quantized_finetuning_amd import synth

def product(name: str):
    """A module of the package for a GPU test module: the module itself, or (when it does not import, e.g. the
    library is not built) a stand-in whose every use fails the test loudly. Collection of the GPU test modules
    thus never depends on the library, and a GPU run without it fails instead of skipping."""
    import importlib

    try:
        return importlib.import_module(f"bit_quantized_finetuning_amd.{name}")
    except ImportError as e:  # pragma: no cover - exercised only without the library
        err = e

        class _Missing:
            def __getattr__(self, attr):
                import pytest

                pytest.fail(f"bit_quantized_finetuning_amd.{name} does not import: {err}")

        return _Missing()


REL_FRO = 5e-3
MAX_ABS = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits_to_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def assert_close(name, gpu, ref):
    g = gpu.detach().double().cpu().numpy() if torch.is_tensor(gpu) else np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / max(nr, 1e-300)
    mx = np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-300)
    say(f"    {name}: rel_fro={rel:.3e} max_abs/max|ref|={mx:.3e}")
    assert rel <= REL_FRO, f"{name}: relative Frobenius error {rel:.3e} > {REL_FRO}"
    assert mx <= MAX_ABS, f"{name}: max-abs error {mx:.3e} > {MAX_ABS} * max|ref|"


def merge_float32_slack(wb, A, B, alpha, r):
    """Bound on the float32 error of forming W_hat + s B A before the final bf16 rounding: the products
    are exact, r accumulations and the scale and add roundings each cost at most 2^-24 of the operands'
    magnitudes. Where W_hat and s B A nearly cancel this exceeds an ulp of the small result."""
    if r == 0 or A is None:
        return 0.0
    s = float(np.float32(alpha) / np.float32(r))
    return 2.0 ** -24 * (np.abs(wb) + (r + 2) * s * (np.abs(np.asarray(B, np.float64)) @ np.abs(np.asarray(A, np.float64))))


def assert_within_one_bf16_ulp(name, gpu, ref, slack=0.0, max_mismatch=1e-3):
    """gpu: bf16 tensor; ref: float64 values already rounded to bf16 (the oracle's single rounding).
    Every element within one bf16 unit in the last place of the larger magnitude plus `slack` (the
    float32 error of the library's sum, see merge_float32_slack), and at most max_mismatch of them
    off at all."""
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape
    mag = np.maximum(np.abs(g), np.abs(r))
    ulp = np.where(mag > 0, np.ldexp(1.0, np.frexp(mag)[1] - 8), 0.0)
    diff = np.abs(g - r)
    frac = float(np.mean(diff > 0))
    say(f"    {name}: max diff/ulp={np.max(np.where(ulp > 0, diff / np.where(ulp > 0, ulp, 1), 0)):.2f} "
        f"max diff/(ulp+slack)={np.max(diff / np.maximum(ulp + slack, 1e-300)):.2f} mismatch fraction={frac:.2e}")
    assert np.all(diff <= ulp + slack), f"{name}: an element is off by more than one bf16 ulp + float32 slack"
    assert frac <= max_mismatch, f"{name}: {frac:.2e} of the elements differ"


class Case:
    """Seeded inputs for one projection plus lazily computed oracle quantities."""

    def __init__(self, d_out, d_in, r, T, cfg=100, proj=0, wdtype="f32", seed=0, alpha=16.0):
        self.d_out, self.d_in, self.r, self.T, self.alpha = d_out, d_in, r, T, alpha
        self.W = synth.weight(cfg, proj, d_out, d_in, wdtype, seed)
        self.wdtype = wdtype
        if r > 0:
            (self.A, self.A_bits), (self.B, self.B_bits) = synth.adapters(cfg, proj, d_out, d_in, r, seed)
        else:
            self.A = self.B = self.A_bits = self.B_bits = None
        self.x, self.x_bits = synth.tokens(cfg, proj, T, d_in, seed)
        self.dY, self.dY_bits = synth.upstream_grad(cfg, proj, T, d_out, seed)
        self._q = None

    # oracle side -----------------------------------------------------------
    def oracle_quant(self):
        if self._q is None:
            codes, q2, S = oracle.quantize(self.W)
            w32, wb = oracle.dequantize(codes, q2, S, self.d_out, self.d_in)
            self._q = (codes, q2, S, w32, wb)
        return self._q

    def oracle_forward(self):
        wb = self.oracle_quant()[4]
        return oracle.lora_forward(wb, self.x, self.A, self.B, self.alpha, self.r)

    def oracle_backward(self):
        wb = self.oracle_quant()[4]
        return oracle.lora_backward(wb, self.x, self.dY, self.A, self.B, self.alpha, self.r)

    # device side -----------------------------------------------------------
    def device_inputs(self, device="cuda"):
        W = torch.from_numpy(self.W)
        if self.wdtype == "bf16":
            W = W.to(torch.bfloat16)
        d = {"W": W.to(device), "x": bits_to_bf16(self.x_bits, device), "dY": bits_to_bf16(self.dY_bits, device)}
        d["A"] = bits_to_bf16(self.A_bits, device) if self.r > 0 else None
        d["B"] = bits_to_bf16(self.B_bits, device) if self.r > 0 else None
        return d
