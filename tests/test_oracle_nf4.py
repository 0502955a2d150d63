"""Pins for the oracle's NF4 quantizer, double quantization and dequantization (CPU only).

Every check here ties the oracle to something other than itself: invariants the
pages state, an independent inverse-normal route, brute-force nearest-level
search, the double-quant error bound, the storage figures the pages print, and
torch's own bf16 conversion.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# codebook
# ---------------------------------------------------------------------------

def test_codebook_invariants():
    c = oracle.nf4_codebook()
    g = _golden()
    assert c.dtype == np.float32 and c.size == g["nf4_levels"]["value"]
    assert np.all(np.diff(c.astype(np.float64)) > 0), "strictly increasing"
    # ends exactly +-1, exact zero (48GB: "including an exact 0")
    assert c[0] == -1.0 and c[15] == 1.0 and c[7] == 0.0
    assert np.sum(c < 0) == 7 and np.sum(c > 0) == 8
    # dense near 0, sparse at the ends: gaps grow moving away from zero on both sides
    gaps = np.diff(c.astype(np.float64))
    pos_gaps = gaps[7:]            # c7->c8, c8->c9, ..., c14->c15
    neg_gaps = gaps[:7][::-1]      # c6->c7, c5->c6, ..., c0->c1
    assert np.all(np.diff(pos_gaps) > 0)
    assert np.all(np.diff(neg_gaps) > 0)


def _inv_cdf_bisection(p: float) -> float:
    """Standard-normal quantile by bisection on Phi(x) = erfc(-x/sqrt2)/2 (independent of AS241)."""
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mid == lo or mid == hi:
            break
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_codebook_independent_inverse_cdf_routes():
    """The levels come out the same from two other quantile routes (scipy ndtri, erfc bisection)."""
    import scipy.special

    ref = oracle.nf4_levels_f64()
    via_scipy = oracle.nf4_levels_f64(lambda p: float(scipy.special.ndtri(p)))
    via_bisect = oracle.nf4_levels_f64(_inv_cdf_bisection)
    assert np.max(np.abs(ref - via_scipy)) < 1e-14
    assert np.max(np.abs(ref - via_bisect)) < 1e-13
    assert np.array_equal(via_scipy.astype(np.float32), oracle.nf4_codebook())
    assert np.array_equal(via_bisect.astype(np.float32), oracle.nf4_codebook())


def test_codebook_is_normal_quantiles():
    """Each nonzero level is a standard-normal quantile rescaled by the largest one."""
    import scipy.stats

    c = oracle.nf4_levels_f64()
    top = scipy.stats.norm.ppf(0.5 * ((1 - 1 / 30) + (1 - 1 / 32)))
    probs = scipy.stats.norm.cdf(c * top)
    # positive side: equally spaced probabilities from 1/2 (8 steps); negative side: 7 steps
    pos = np.sort(probs[c > 0])
    neg = np.sort(probs[c < 0])
    assert np.allclose(np.diff(np.concatenate([[0.5], pos])), (pos[-1] - 0.5) / 8, rtol=1e-9)
    assert np.allclose(np.diff(np.concatenate([neg, [0.5]])), (0.5 - neg[0]) / 7, rtol=1e-9)


# ---------------------------------------------------------------------------
# nearest level
# ---------------------------------------------------------------------------

def _brute_nearest(x32):
    c = oracle.nf4_codebook().astype(np.float64)
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    d = np.abs(x[:, None] - c[None, :])
    return np.argmin(d, axis=1)          # first minimum = lower index on ties


def _midpoint_neighbours(k=4):
    m = oracle.nf4_midpoints_f64()
    pts = []
    for mj in m:
        f = np.float32(mj)
        pts.append(f)
        lo = hi = f
        for _ in range(k):
            lo = np.nextafter(lo, np.float32(-np.inf))
            hi = np.nextafter(hi, np.float32(np.inf))
            pts += [lo, hi]
    return np.array(pts, dtype=np.float32)


def test_nearest_level_bruteforce():
    rs = np.random.default_rng(123)
    xs = np.concatenate([
        rs.uniform(-1, 1, 20000).astype(np.float32),
        _midpoint_neighbours(),
        oracle.nf4_codebook(),
        np.array([-1.0, 1.0, 0.0, -0.0], dtype=np.float32),
    ])
    assert np.array_equal(oracle.nearest_level(xs), _brute_nearest(xs))


def test_midpoint_ties_go_to_lower_index():
    m = oracle.nf4_midpoints_f64()
    exact = [j for j, mj in enumerate(m) if float(np.float32(mj)) == mj]
    assert len(exact) == 4, "4 of the 15 midpoints are exact float32 values"
    for j in exact:
        assert oracle.nearest_level(np.array([m[j]], dtype=np.float32))[0] == j


def test_float32_threshold_rule_matches_float64_rule():
    """q = #{j : x >= theta_j} with float32 thresholds equals the exact float64 rule on every neighbour."""
    th = oracle.nf4_thresholds_f32()
    xs = _midpoint_neighbours(k=6)
    q32 = np.sum(xs[:, None] >= th[None, :], axis=1)
    assert np.array_equal(q32, oracle.nearest_level(xs))
    assert xs.size >= 138


# ---------------------------------------------------------------------------
# full quantizer
# ---------------------------------------------------------------------------

def _brute_quantize(W):
    """Per-element brute force: block max by Python max(), divide in double then round to float32
    (exact for float32 operands), nearest of 16 by distance."""
    W = np.asarray(W, dtype=np.float32)
    flat = [float(v) for v in W.reshape(-1)]
    c = [float(v) for v in oracle.nf4_codebook()]
    q = []
    for b in range(len(flat) // 64):
        blk = flat[b * 64:(b + 1) * 64]
        s = max(abs(v) for v in blk)
        for v in blk:
            x = float(np.float32(v / s)) if s > 0 else 0.0
            best = min(range(16), key=lambda j: (abs(x - c[j]), j))
            q.append(best)
    return q


def _brute_pack(q):
    """Per 8 elements, byte i carries element i (low nibble) and element i+4 (high nibble)."""
    out = []
    for w in range(len(q) // 8):
        for i in range(4):
            out.append(q[8 * w + i] + 16 * q[8 * w + i + 4])
    return out


def test_quantize_bruteforce_tiny():
    rs = np.random.default_rng(7)
    W = (rs.standard_normal((4, 192)) * 0.02).astype(np.float32)
    W[1, 64:128] = 0.0                                  # a zero block
    W[2, 0:64] = np.linspace(-3, 5, 64)                 # spread block
    W[3, 128:192] = -np.abs(W[3, 128:192])              # all-negative block
    codes, q2, S = oracle.quantize(W)
    q = _brute_quantize(W)
    assert list(oracle.unpack_codes(codes)) == q
    assert list(codes) == _brute_pack(q)
    # word view: nibble k of little-endian word w is element 8w + (k//2) + 4*(k%2)
    words = codes.view("<u4")
    for w in range(0, words.size, 7):
        for k in range(8):
            assert (int(words[w]) >> (4 * k)) & 15 == q[8 * w + k // 2 + 4 * (k % 2)]


def test_quantize_invariants():
    rs = np.random.default_rng(11)
    W = (rs.standard_normal((32, 256)) * 0.02).astype(np.float32)
    W[5, :64] = 0.0
    codes, q2, S = oracle.quantize(W)
    q = oracle.unpack_codes(codes).reshape(-1, 64)
    w = W.reshape(-1, 64)
    for k in range(w.shape[0]):
        if np.all(w[k] == 0):
            assert np.all(q[k] == 7)
        else:
            i = int(np.argmax(np.abs(w[k])))
            assert q[k, i] == (15 if w[k, i] > 0 else 0)
    # idempotence: re-quantizing the no-DQ reconstruction c[q] * s_k returns the same codes
    c = oracle.nf4_codebook()
    s = oracle.block_absmax(W.reshape(-1))
    W2 = (c[q] * s[:, None]).astype(np.float32).reshape(W.shape)
    codes2, _, _ = oracle.quantize(W2)
    assert np.array_equal(codes, codes2)


def test_quantize_bf16_weights_widen_exactly():
    """bf16 weights are widened exactly to float32 before quantizing: identical codes either way."""
    rs = np.random.default_rng(3)
    W = (rs.standard_normal((8, 128)) * 0.02).astype(np.float32)
    Wb = torch.from_numpy(W).to(torch.bfloat16).float().numpy()
    a = oracle.quantize(Wb)
    b = oracle.quantize(Wb.astype(np.float64).astype(np.float32))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# double quantization
# ---------------------------------------------------------------------------

def test_double_quant_error_bound_exact():
    """|(q2/256) S - s| <= S/256 exactly, in rational arithmetic (QLoRA-65B, memory accounting)."""
    rs = np.random.default_rng(5)
    s = np.abs(rs.standard_normal(256 * 7 + 13)).astype(np.float32) * np.float32(0.05)
    q2, S = oracle.double_quant(s)
    bound = Fraction(_golden()["double_quant_scale_error_bound_fraction_of_smax"]["value"])
    for k in range(s.size):
        Sg = Fraction(float(S[k // 256]))
        err = abs(Fraction(int(q2[k]), 256) * Sg - Fraction(float(s[k])))
        assert err <= bound * Sg
    # every group has its maximum block at the top code
    for g in range(S.size):
        assert np.max(q2[g * 256:(g + 1) * 256]) == 255


def test_double_quant_float32_reconstruction_within_bound_plus_rounding():
    rs = np.random.default_rng(9)
    s = np.abs(rs.standard_normal(256 * 3)).astype(np.float32)
    q2, S = oracle.double_quant(s)
    sh = oracle.dequant_scales(q2, S)
    g = np.arange(s.size) // 256
    err = np.abs(sh.astype(np.float64) - s.astype(np.float64))
    ulp = np.spacing(S[g]).astype(np.float64)
    assert np.all(err <= S[g].astype(np.float64) / 256 + ulp)


def test_double_quant_outlier_block():
    """One block 1000x larger than the rest of its group: small blocks collapse to q2 = 0 but the
    absolute error bound S/256 still holds (the 'extreme distribution' caveat)."""
    s = np.full(256, 0.01, dtype=np.float32)
    s[17] = 10.0
    q2, S = oracle.double_quant(s)
    assert S[0] == np.float32(10.0) and q2[17] == 255
    assert np.all(q2[np.arange(256) != 17] == 0)
    sh = oracle.dequant_scales(q2, S)
    assert np.all(np.abs(sh - s) <= S[0] / 256 + np.spacing(S[0]))


def test_double_quant_zero_group_and_short_last_group():
    s = np.zeros(256 + 10, dtype=np.float32)
    s[256:] = np.linspace(0.1, 1.0, 10, dtype=np.float32)
    q2, S = oracle.double_quant(s)
    assert S[0] == 0 and np.all(q2[:256] == 0)
    assert S.size == 2 and S[1] == np.float32(1.0) and q2[-1] == 255


def test_double_quant_rounds_half_to_even():
    # fl32(s/S)*256 = 2.5 and 3.5 exactly -> 2 and 4
    S = np.float32(1.0)
    s = np.array([1.0, 2.5 / 256, 3.5 / 256], dtype=np.float32)
    q2, _ = oracle.double_quant(s)
    assert list(q2) == [255, 2, 4]


# ---------------------------------------------------------------------------
# dequantization
# ---------------------------------------------------------------------------

def test_dequant_matches_reconstruction_formula():
    """w_hat = c(q) * (q2/256) * s_max (QLoRA-65B reconstruction equation), within the two float32 roundings."""
    rs = np.random.default_rng(21)
    W = (rs.standard_normal((16, 1024)) * 0.02).astype(np.float32)
    codes, q2, S = oracle.quantize(W)
    w, wb = oracle.dequantize(codes, q2, S, 16, 1024)
    c = oracle.nf4_codebook().astype(np.float64)
    q = oracle.unpack_codes(codes).reshape(-1, 64)
    k = np.arange(q.shape[0])
    exact = c[q] * (q2[k].astype(np.float64) / 256.0)[:, None] * S[k // 256].astype(np.float64)[:, None]
    rel = np.abs(w.reshape(-1, 64) - exact) / np.maximum(np.abs(exact), 1e-30)
    assert np.all(rel[exact != 0] <= 2 * 2.0 ** -24 + 1e-12)
    assert np.all(w.reshape(-1, 64)[exact == 0] == 0)
    # bf16 restore agrees with torch's own round-to-nearest-even conversion
    tb = torch.from_numpy(w).to(torch.bfloat16).float().numpy()
    assert np.array_equal(wb, tb)


def test_bf16_round_matches_torch_on_ties_and_random():
    rs = np.random.default_rng(1)
    a = rs.standard_normal(100000).astype(np.float32)
    ties = (np.arange(1, 5000, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32)
    for arr in (a, ties, -ties):
        assert np.array_equal(oracle.bf16_round(arr), torch.from_numpy(arr).to(torch.bfloat16).float().numpy())


def test_nf4_quality_sanity_range():
    """Sanity range (not a pin): NF4 on N(0, 0.02^2) weights has ~9% relative Frobenius error."""
    rs = np.random.default_rng(0)
    W = (rs.standard_normal((256, 1024)) * 0.02).astype(np.float32)
    codes, q2, S = oracle.quantize(W)
    w, _ = oracle.dequantize(codes, q2, S, 256, 1024)
    rel = np.linalg.norm(w - W) / np.linalg.norm(W)
    assert 0.07 < rel < 0.11


# ---------------------------------------------------------------------------
# storage figures the pages print
# ---------------------------------------------------------------------------

def test_storage_bits_and_65b_figures():
    g = _golden()
    n = 4096 * 4096
    bits = 8 * oracle.storage_bytes(4096, 4096) / n
    assert round(bits, 2) == g["bits_per_param_double_quant"]["value"]
    # absmax-only storage: 4 bits + one fp32 per 64 weights
    assert 4 + 32 / 64 == g["bits_per_param_absmax_only"]["value"]
    N65 = 65e9
    dq_gb = N65 * bits / 8 / 1e9
    absmax_gb = N65 * 4.5 / 8 / 1e9
    assert abs(dq_gb - g["nf4_base_65b_gb"]["value"]) < 1.0
    assert abs((absmax_gb - dq_gb) - g["double_quant_saving_65b_gb"]["value"]) < 0.5


def test_storage_bytes_layout():
    assert oracle.storage_bytes(1024, 1024) == 524288 + 16384 + 256
    assert oracle.storage_bytes(11008, 4096) == 22544384 + 704512 + 4 * 2752
    # d_in = 5120: groups straddle rows, last group full
    assert oracle.storage_bytes(5120, 5120) == 13107200 + 409600 + 6400


# ---------------------------------------------------------------------------
# absmax-only storage (no double quantization): 4.5 bits per parameter
# ---------------------------------------------------------------------------

def test_absmax_storage_is_4_5_bits():
    g = _golden()
    for d_out, d_in in ((4096, 4096), (11008, 4096), (16, 64), (80, 320)):
        n = d_out * d_in
        assert 8 * oracle.storage_bytes_absmax(d_out, d_in) / n == g["bits_per_param_absmax_only"]["value"]


def test_absmax_quantize_bruteforce_tiny():
    rs = np.random.default_rng(8)
    W = (rs.standard_normal((4, 192)) * 0.02).astype(np.float32)
    W[1, 64:128] = 0.0                                  # a zero block
    W[2, 0:64] = np.linspace(-3, 5, 64)                 # spread block
    W[3, 128:192] = -np.abs(W[3, 128:192])              # all-negative block
    codes, s = oracle.quantize_absmax(W)
    assert list(oracle.unpack_codes(codes)) == _brute_quantize(W)
    flat = [float(v) for v in W.reshape(-1)]
    brute_s = [max(abs(v) for v in flat[64 * k:64 * k + 64]) for k in range(len(flat) // 64)]
    assert s.dtype == np.float32 and list(s.astype(np.float64)) == brute_s
    # same codes as the double-quant storage: the codes never see the re-coded scale
    assert np.array_equal(codes, oracle.quantize(W)[0])


def test_absmax_restore_is_lossless_on_scaled_levels():
    """Weights that are exactly a level times a power of two come back unchanged (no scale re-coding)."""
    c = oracle.nf4_codebook()
    rs = np.random.default_rng(9)
    rows = []
    for e in (-12, -7, 0, 3):
        idx = rs.integers(0, 16, 64)
        idx[rs.integers(0, 64)] = 15 if e % 2 else 0   # the block's absmax is 2^e
        rows.append(c[idx] * np.float32(2.0 ** e))
    W = np.stack(rows).astype(np.float32).reshape(4, 64)
    codes, s = oracle.quantize_absmax(W)
    assert np.array_equal(s, np.float32(2.0) ** np.array([-12, -7, 0, 3], dtype=np.float32))
    w, wb = oracle.dequantize_absmax(codes, s, 4, 64)
    assert np.array_equal(w, W)
    tb = torch.from_numpy(w).to(torch.bfloat16).float().numpy()
    assert np.array_equal(wb, tb)


def test_absmax_restore_error_within_half_the_level_gap():
    """|w_hat - w| <= s * (largest gap between adjacent levels) / 2, plus the float32 products' rounding."""
    c = oracle.nf4_codebook().astype(np.float64)
    half_gap = np.max(np.diff(c)) / 2
    rs = np.random.default_rng(10)
    W = (rs.standard_normal((32, 512)) * 0.02).astype(np.float32)
    W[3, :64] = 0.0
    codes, s = oracle.quantize_absmax(W)
    w, _ = oracle.dequantize_absmax(codes, s, 32, 512)
    err = np.abs(w.astype(np.float64) - W.astype(np.float64)).reshape(-1, 64)
    sk = s.astype(np.float64)[:, None]
    assert np.all(err <= sk * (half_gap + 2.0 ** -23))
    assert np.all(w.reshape(-1, 64)[3 * 8] == 0)
    # no worse than double quantization, whose scale carries an extra error of up to S/256
    codes2, q2, S = oracle.quantize(W)
    w2, _ = oracle.dequantize(codes2, q2, S, 32, 512)
    assert np.linalg.norm(w - W) <= np.linalg.norm(w2 - W)


def test_absmax_restore_matches_torch_float32_product():
    rs = np.random.default_rng(12)
    W = (rs.standard_normal((16, 256)) * 0.02).astype(np.float32)
    codes, s = oracle.quantize_absmax(W)
    w, wb = oracle.dequantize_absmax(codes, s, 16, 256)
    c = torch.from_numpy(oracle.nf4_codebook())
    q = torch.from_numpy(oracle.unpack_codes(codes).astype(np.int64)).view(-1, 64)
    ref = (c[q] * torch.from_numpy(s)[:, None]).view(16, 256)
    assert torch.equal(torch.from_numpy(w), ref)
    assert torch.equal(torch.from_numpy(wb), ref.to(torch.bfloat16).float())
