"""NF4 blockwise quantization with double quantization -- plain CPU oracle.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.

What is computed, in the pages' order:

  1. the 16-level NF4 codebook c[0..15] (normal quantiles, exact zero, dense near
     zero) -- [48GB] "Quantization Keeps the Patterns and Reduces Bits per
     Number"; [QLoRA-2023] "How it works";
  2. per block of 64 weights the scale s_k = largest |w| in the block -- same
     section of [48GB] ("split weights into blocks of 64 ... the weight with the
     largest absolute value");
  3. divide each weight by its block scale and keep the index of the nearest
     level (4 bits, two per byte) -- same section;
  4. double quantization: the block scales are themselves re-quantized to 8-bit
     codes q2 against a group maximum S, so that the scale comes back as
     (q2/256)*S with error at most S/256 -- [QLoRA-65B] "메모리 회계", the
     Double Quantization paragraph and the reconstruction equation
     w_i = c(q_i) * (q_k^(2)/256) * s_max;
  5. dequantization back to bf16 for the matmul -- [48GB] "Each weight takes
     4 bits ... restored to bf16 before participating in matrix multiplication".

The absmax-only storage (steps 1-3 and 5 without step 4) is the variant the
pages price at 4.5 bits per parameter: every block keeps its float32 scale
([QLoRA-65B] "메모리 회계", NF4 paragraph; double quantization then takes it
to 4.13). quantize_absmax / dequantize_absmax / storage_bytes_absmax.

Readings taken where the pages are silent (each also listed in the design doc):
  * codebook: 8 positive levels at Phi^-1(1/2 + (p-1/2) j/8), j=1..8, 7 negative
    levels at -Phi^-1(1/2 + (p-1/2) j/7), j=1..7, and 0, with
    p = ((1-1/30) + (1-1/32))/2, all divided by Phi^-1(p) so the ends are +-1,
    sorted ascending and rounded to float32. Absolute values: parity unpinned
    beyond the invariants the pages fix (exact 0, dense near 0, 16 levels in
    [-1, 1]) and an independent inverse-CDF route.
  * the scale is the magnitude |w| (unsigned); a zero block codes as all-zero
    (index 7).
  * nearest level: exact comparison in float64 of x = fl32(w/s) against the
    level midpoints, ties to the lower index.
  * nibble order: codes are packed per run of 8 consecutive weights into one
    little-endian 32-bit word; byte i (i = 0..3) holds element i in its low
    nibble and element i+4 in its high nibble. (The pages fix only 4-bit
    indices; this order lets a byte-select expansion produce the restored
    values in element order.)
  * double quant: groups of 256 consecutive blocks in flattened row-major order
    (the last group may be short), S_g = max s_k in float32, q2 unsigned 0..255,
    q2 = min(255, rint_half_even(fl32(s_k / S_g) * 256)), q2 = 0 when S_g = 0.
  * dequant order: s_hat = fl32(q2 * 2^-8 * S) (one rounding), then
    w_hat = fl32(c[q] * s_hat), then round-to-nearest-even to bf16.
"""

from __future__ import annotations

import math
import statistics

import numpy as np

BLOCK = 64          # weights per absmax block ([48GB] "blocks of 64")
GROUP = 256         # blocks per double-quant group (8-bit scale codes)


# ----------------------------------------------------------------------------
# 1. Codebook
# ----------------------------------------------------------------------------

def _tail_probability() -> float:
    """p = midpoint of the 15- and 16-bin half-bin tails: ((1-1/30)+(1-1/32))/2."""
    return 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))


def nf4_levels_f64(inv_cdf=None) -> np.ndarray:
    """Unrounded NF4 levels (float64, ascending).

    Normal-distribution quantiles, dense near zero, with an exact zero
    ([48GB] "Quantization Keeps the Patterns..."; [QLoRA-2023] "How it works":
    NF4 places its values where normally distributed weights fall).
    `inv_cdf` is the standard-normal quantile function; by default Wichura's
    AS241 as implemented by `statistics.NormalDist().inv_cdf`.
    """
    if inv_cdf is None:
        inv_cdf = statistics.NormalDist().inv_cdf
    p = _tail_probability()
    pos = [inv_cdf(0.5 + (p - 0.5) * j / 8.0) for j in range(1, 9)]    # 8 levels > 0
    neg = [-inv_cdf(0.5 + (p - 0.5) * j / 7.0) for j in range(1, 8)]   # 7 levels < 0
    top = inv_cdf(p)
    levels = np.array(sorted(neg + [0.0] + pos), dtype=np.float64) / top
    return levels


def nf4_codebook(inv_cdf=None) -> np.ndarray:
    """The 16 float32 NF4 levels c[0..15], ascending: c[0] = -1, c[7] = 0, c[15] = 1."""
    return nf4_levels_f64(inv_cdf).astype(np.float32)


def nf4_midpoints_f64(codebook: np.ndarray | None = None) -> np.ndarray:
    """Exact real midpoints m_j = (c_j + c_{j+1}) / 2 of adjacent float32 levels (float64 is exact here)."""
    c = (nf4_codebook() if codebook is None else codebook).astype(np.float64)
    return (c[:-1] + c[1:]) / 2.0


def nf4_thresholds_f32(codebook: np.ndarray | None = None) -> np.ndarray:
    """Float32 decision thresholds theta_j = smallest float32 strictly above m_j.

    For a float32 x, (x >= theta_j) <=> (x > m_j); so the nearest-level index can
    be taken with 15 float32 compares instead of float64 arithmetic. Used only
    by the test that checks this equivalence.
    """
    m = nf4_midpoints_f64(codebook)
    th = m.astype(np.float32)
    below = th.astype(np.float64) <= m
    th[below] = np.nextafter(th[below], np.float32(np.inf))
    return th


# ----------------------------------------------------------------------------
# bf16 rounding (own implementation; finite values only)
# ----------------------------------------------------------------------------

def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns float32 holding bf16 values."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of bf16_round(a)."""
    return (bf16_round(a).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# 2-3. Blockwise absmax, normalization, nearest level, packing
# ----------------------------------------------------------------------------

def block_absmax(w_flat_f32: np.ndarray) -> np.ndarray:
    """s_k = max |w| over block k (64 consecutive weights of the flattened row-major W), float32 exact."""
    w = np.asarray(w_flat_f32, dtype=np.float32).reshape(-1, BLOCK)
    return np.max(np.abs(w), axis=1).astype(np.float32)


def nearest_level(xn_f32: np.ndarray, codebook: np.ndarray | None = None) -> np.ndarray:
    """Index of the nearest NF4 level for normalized float32 values, ties to the lower index.

    q = #{ j in 0..14 : 2x > c_j + c_{j+1} } evaluated in float64, where both
    sides are exact ([48GB] "take the nearest level and save only the index").
    """
    c = (nf4_codebook() if codebook is None else codebook).astype(np.float64)
    sums = c[:-1] + c[1:]
    x2 = 2.0 * np.asarray(xn_f32, dtype=np.float32).astype(np.float64)
    q = np.zeros(x2.shape, dtype=np.uint8)
    for j in range(15):
        q += (x2 > sums[j]).astype(np.uint8)
    return q


def pack_codes(q: np.ndarray) -> np.ndarray:
    """Two 4-bit indices per byte: in each run of 8 elements e0..e7, byte i = e_i | e_(i+4) << 4."""
    q = np.asarray(q, dtype=np.uint8).reshape(-1, 8)
    return (q[:, 0:4] | (q[:, 4:8] << 4)).astype(np.uint8).reshape(-1)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    b = np.asarray(codes, dtype=np.uint8).reshape(-1, 4)
    q = np.empty((b.shape[0], 8), dtype=np.uint8)
    q[:, 0:4] = b & 0x0F
    q[:, 4:8] = b >> 4
    return q.reshape(-1)


# ----------------------------------------------------------------------------
# 4. Double quantization of the block scales
# ----------------------------------------------------------------------------

def double_quant(s: np.ndarray):
    """Re-quantize block scales to 8-bit codes against a per-group maximum.

    [QLoRA-65B] "메모리 회계", Double Quantization: the block scales are
    compressed to 8 bits (256 levels) with reconstruction error at most
    s_max/256, and come back as (q2/256) * s_max.
    Returns (q2 uint8 [nblocks], S float32 [ceil(nblocks/256)]).
    """
    s = np.asarray(s, dtype=np.float32)
    nb = s.size
    ng = (nb + GROUP - 1) // GROUP
    q2 = np.zeros(nb, dtype=np.uint8)
    S = np.zeros(ng, dtype=np.float32)
    for g in range(ng):
        sg = s[g * GROUP:(g + 1) * GROUP]
        Sg = np.float32(np.max(sg))
        S[g] = Sg
        if Sg == 0:
            continue                                   # q2 stays 0
        ratio = (sg / Sg).astype(np.float32)           # fl32(s_k / S_g)
        scaled = (ratio * np.float32(256.0)).astype(np.float32)   # exact (power of two)
        q2[g * GROUP:(g + 1) * GROUP] = np.minimum(np.rint(scaled), 255.0).astype(np.uint8)
    return q2, S


# ----------------------------------------------------------------------------
# Full quantizer
# ----------------------------------------------------------------------------

def quantize(W: np.ndarray):
    """Quantize W [d_out, d_in] (float32, or bf16 values held in float32) to NF4 + double quant.

    Returns (codes uint8 [n/2], q2 uint8 [n/64], S float32 [ceil(n/64/256)]).
    Steps 2-4 of the module docstring. The block codes use the exact float32
    block scale s_k; double quantization of s_k comes after ([48GB]: the scale
    "itself is further quantized").
    """
    W = np.asarray(W, dtype=np.float32)
    assert W.ndim == 2 and W.shape[1] % BLOCK == 0, "d_in must be a multiple of 64"
    w = W.reshape(-1)
    s = block_absmax(w)
    wb = w.reshape(-1, BLOCK)
    with np.errstate(divide="ignore", invalid="ignore"):
        xn = (wb / s[:, None]).astype(np.float32)      # IEEE float32 divide
    xn[s == 0, :] = 0.0
    q = nearest_level(xn).reshape(-1)
    codes = pack_codes(q)
    q2, S = double_quant(s)
    return codes, q2, S


def dequant_scales(q2: np.ndarray, S: np.ndarray) -> np.ndarray:
    """s_hat_k = fl32(q2_k * 2^-8 * S_g): the double-quant reconstruction of each block scale."""
    q2 = np.asarray(q2, dtype=np.uint8)
    g = np.arange(q2.size) // GROUP
    frac = q2.astype(np.float32) * np.float32(2.0 ** -8)           # exact
    return (frac * np.asarray(S, dtype=np.float32)[g]).astype(np.float32)


def dequantize(codes: np.ndarray, q2: np.ndarray, S: np.ndarray, d_out: int, d_in: int):
    """Restore W: w_hat_i = c(q_i) * (q2_k/256) * S_g ([QLoRA-65B] reconstruction equation).

    Returns (float32 w_hat [d_out, d_in], float32 holding the bf16-rounded w_hat).
    """
    c = nf4_codebook()
    q = unpack_codes(codes)
    sh = dequant_scales(q2, S)
    w = (c[q].reshape(-1, BLOCK) * sh[:, None]).astype(np.float32).reshape(d_out, d_in)
    return w, bf16_round(w)


def quantize_absmax(W: np.ndarray):
    """Quantize W [d_out, d_in] to NF4 with the float32 absmax of every block kept as is (no double quant).

    Returns (codes uint8 [n/2], s float32 [n/64]). The codes are those of quantize(): they come from the
    exact block scale either way; only the storage of the scale differs.
    """
    W = np.asarray(W, dtype=np.float32)
    assert W.ndim == 2 and W.shape[1] % BLOCK == 0, "d_in must be a multiple of 64"
    w = W.reshape(-1)
    s = block_absmax(w)
    wb = w.reshape(-1, BLOCK)
    with np.errstate(divide="ignore", invalid="ignore"):
        xn = (wb / s[:, None]).astype(np.float32)      # IEEE float32 divide
    xn[s == 0, :] = 0.0
    return pack_codes(nearest_level(xn).reshape(-1)), s


def dequantize_absmax(codes: np.ndarray, s: np.ndarray, d_out: int, d_in: int):
    """Restore W from absmax-only storage: w_hat_i = fl32(c(q_i) * s_k), then bf16.

    Returns (float32 w_hat [d_out, d_in], float32 holding the bf16-rounded w_hat).
    """
    c = nf4_codebook()
    q = unpack_codes(codes)
    s = np.asarray(s, dtype=np.float32)
    w = (c[q].reshape(-1, BLOCK) * s[:, None]).astype(np.float32).reshape(d_out, d_in)
    return w, bf16_round(w)


def storage_bytes_absmax(d_out: int, d_in: int) -> int:
    """Bytes of the absmax-only storage: n/2 (codes) + 4 n/64 (one float32 scale per block)."""
    n = d_out * d_in
    return n // 2 + 4 * (n // BLOCK)


def storage_bytes(d_out: int, d_in: int) -> int:
    """Bytes of the quantized weight: n/2 (codes) + n/64 (q2) + 4 * ceil(n/64/256) (S)."""
    n = d_out * d_in
    nb = n // BLOCK
    return n // 2 + nb + 4 * ((nb + GROUP - 1) // GROUP)
