"""QLoRA linear layer forward and backward -- plain CPU oracle in float64.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.

Forward ([QLoRA-65B] "QLoRA의 수식", the two-term equation):
    h = dequant(W_NF4, c_block) x + (alpha/r) B A x
with A [r, d_in], B [d_out, r] ([QLoRA-65B] problem statement). Tokens are
rows here, so with x [T, d_in]:
    u = x A^T                       [T, r]
    h = x W_hat^T + (alpha/r) u B^T [T, d_out]
where W_hat is the bf16 restore of the quantized weight ([48GB] "restored to
bf16 before participating in matrix multiplication").

Backward ([QLoRA-65B] "QLoRA의 수식" and "명제 1": the base weight is frozen,
so no gradient is requested through the dequantization; [48GB] "QLoRA Puts the
Two Methods in Different Places": gradients pass through the restored W to A and
B). For an upstream gradient dY = dL/dh [T, d_out]:
    v  = dY B                         [T, r]
    dX = dY W_hat + (alpha/r) v A     [T, d_in]
    dA = (alpha/r) v^T x              [r, d_in]
    dB = (alpha/r) dY^T u             [d_out, r]
No dW is produced.

Merge ([48GB] "QLoRA Puts the Two Methods in Different Places": the trained A
and B cannot be added to the 4-bit weights; they are merged into the restored
16-bit weights):
    W_merged = bf16(W_hat + (alpha/r) B A)
with the sum exact in float64 and a single round-to-nearest-even to bf16.

All products are float64 matrix products of the given (bf16-exact) values;
the result is the exact value up to float64 rounding.
"""

from __future__ import annotations

import numpy as np


def _scale(alpha: float, r: int) -> float:
    # s = alpha / r is formed in float32, as the library receives it.
    return float(np.float32(alpha) / np.float32(r)) if r > 0 else 0.0


def lora_forward(W_hat: np.ndarray, x: np.ndarray, A: np.ndarray | None, B: np.ndarray | None,
                 alpha: float, r: int):
    """Return (h, u) in float64. r == 0 (or A/B None) gives the base term only."""
    Wd = np.asarray(W_hat, dtype=np.float64)
    xd = np.asarray(x, dtype=np.float64)
    h = xd @ Wd.T
    if r == 0 or A is None or B is None:
        return h, np.zeros((xd.shape[0], 0))
    Ad = np.asarray(A, dtype=np.float64)
    Bd = np.asarray(B, dtype=np.float64)
    u = xd @ Ad.T
    h = h + _scale(alpha, r) * (u @ Bd.T)
    return h, u


def lora_backward(W_hat: np.ndarray, x: np.ndarray, dY: np.ndarray, A: np.ndarray | None,
                  B: np.ndarray | None, alpha: float, r: int):
    """Return (dX, dA, dB) in float64 (dA, dB are None when r == 0). No gradient into W."""
    Wd = np.asarray(W_hat, dtype=np.float64)
    xd = np.asarray(x, dtype=np.float64)
    gd = np.asarray(dY, dtype=np.float64)
    dX = gd @ Wd
    if r == 0 or A is None or B is None:
        return dX, None, None
    Ad = np.asarray(A, dtype=np.float64)
    Bd = np.asarray(B, dtype=np.float64)
    s = _scale(alpha, r)
    u = xd @ Ad.T
    v = gd @ Bd
    dX = dX + s * (v @ Ad)
    dA = s * (v.T @ xd)
    dB = s * (gd.T @ u)
    return dX, dA, dB


def bf16_round_f64(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 in one step (nearest, ties to even), as float64.

    Finite values in the bf16 range only. A bf16 keeps 8 significant bits: with
    a = m 2^e, 0.5 <= |m| < 1, the result is rint(m 2^8) 2^(e-8) (numpy's rint
    rounds halves to even). Below the smallest normal (2^-126) the spacing is
    fixed at 2^-133.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    sub = np.ldexp(np.rint(np.ldexp(a, 133)), -133)
    return np.where(np.abs(a) < 2.0 ** -126, sub, normal)


def lora_merge(W_hat: np.ndarray, A: np.ndarray | None, B: np.ndarray | None, alpha: float, r: int) -> np.ndarray:
    """bf16(W_hat + (alpha/r) B A) as float64 values; r == 0 (or A/B None) returns W_hat rounded (unchanged)."""
    Wd = np.asarray(W_hat, dtype=np.float64)
    if r == 0 or A is None or B is None:
        return bf16_round_f64(Wd + 0.0)
    exact = Wd + _scale(alpha, r) * (np.asarray(B, dtype=np.float64) @ np.asarray(A, dtype=np.float64))
    return bf16_round_f64(exact)
