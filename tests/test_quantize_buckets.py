"""The quantizer's bucketed nearest-level search (quantize.hip) equals the plain threshold count.

The kernel takes x = w/s (in [-1, 1]) to one of 64 buckets from its float32 bits -- sign, binade (2^-5 .. 1 in
six steps, all smaller magnitudes in one), top two significand bits -- and counts the thresholds below the
bucket plus at most one comparison. This restates that rule on the host and checks it against the count of the
library's own 15 thresholds for every float32 in [-1, 1] (no GPU needed).
"""

import numpy as np

from bit_quantized_finetuning_amd import qlora as q


def _buckets(th):
    thd = th.astype(np.float64)
    base = np.zeros(64, np.int64)
    cand = np.full(64, np.inf, np.float32)
    for b in range(64):
        sg, e, m = b >> 5, (b >> 2) & 7, b & 3
        if e == 0:
            lo, hi = 0.0, 2.0 ** -5
        else:
            bb = 2.0 ** (e - 6)
            lo, hi = bb * (1 + m / 4), bb * (1 + (m + 1) / 4)
        if sg == 0:
            base[b] = np.sum(thd <= lo)
            c = thd[(thd > lo) & (thd < hi)]
        else:
            base[b] = np.sum(thd <= -hi)
            c = thd[(thd > -hi) & (thd <= -lo)]
        assert len(c) <= 1, f"bucket {b} holds {len(c)} thresholds"
        if len(c):
            cand[b] = np.float32(c[0])
    return base, cand


def test_bucketed_count_equals_threshold_count_on_all_float32_in_unit_interval():
    th = np.array(q.qlora_nf4_thresholds(), dtype=np.float32)
    assert np.all(np.diff(th) > 0)
    base, cand = _buckets(th)
    top = 0x3F800000  # 1.0
    mismatches = 0
    for sign in (0, 1):
        for start in range(0, top + 1, 1 << 26):
            bits = np.arange(start, min(start + (1 << 26), top + 1), dtype=np.uint32) | np.uint32(sign << 31)
            x = bits.view(np.float32)
            count = np.searchsorted(th, x, side="right")          # thresholds <= x
            e = np.clip(((bits >> 23) & 0xFF).astype(np.int32) - 121, 0, 6)
            b = ((bits >> 31).astype(np.int32) << 5) | (e << 2) | ((bits >> 21) & 3).astype(np.int32)
            mismatches += int(np.sum(count != base[b] + (x >= cand[b])))
    assert mismatches == 0


def _table2048(th):
    """The kernel's entries: (threshold or +inf, tolerance = 16 ulp of it or 0, count below) per sign, exponent
    and top two significand bits of the quotient."""
    base, cand = _buckets(th)
    i = np.arange(2048)
    sg, ex, m2 = i >> 10, (i >> 2) & 0xFF, i & 3
    e = np.clip(ex - 121, 0, 6)
    b = (sg << 5) | (e << 2) | np.where(e == 0, 0, m2)
    t = cand[b]
    tb = t.view(np.uint32)
    texp = ((tb >> 23) & 0xFF).astype(np.int64)
    tol_bits = np.where(np.isfinite(t), (texp - 19) << 23, 0).astype(np.uint32)
    return t, tol_bits.view(np.float32), base[b]


def test_approximate_quotient_rule_is_exact():
    th = np.array(q.qlora_nf4_thresholds(), dtype=np.float32)
    tbits = th.view(np.uint32).astype(np.int64)
    # every threshold has magnitude above 2^-5 and sits >= 64 ulp (bit patterns) from a quarter-binade edge
    assert np.all(np.abs(th) > 2.0 ** -5)
    low = (tbits & 0x7FFFFFFF) & ((1 << 21) - 1)
    assert np.all(np.minimum(low, (1 << 21) - low) >= 64)
    t, tol, cnt = _table2048(th)
    # quotients: a stride across [-1, 1], and every pattern within 96 ulp of each threshold and each edge
    pos = [np.arange(0, 0x3F800001, 997, dtype=np.int64)]
    for tb in (tbits & 0x7FFFFFFF):
        pos.append(np.arange(tb - 96, tb + 97))
    for edge in range(0x3D000000, 0x3F800001, 1 << 21):  # 2^-5 .. 1
        pos.append(np.arange(edge - 96, edge + 97))
    mag = np.unique(np.clip(np.concatenate(pos), 0, 0x3F800000))
    for sign in (0, 1):
        xb = (mag | (sign << 31)).astype(np.uint32)
        x = xb.view(np.float32)
        exact = np.searchsorted(th, x, side="right")
        for p in range(-4, 5):
            ya = np.clip(mag + p, 0, None) | (sign << 31)   # xa: up to 4 ulp away, same sign
            y = ya.astype(np.uint32).view(np.float32)
            idx = (ya.astype(np.uint32) >> 21).astype(np.int64)
            d = y.astype(np.float64) - t[idx].astype(np.float64)
            near = np.abs(d) <= tol[idx].astype(np.float64)
            fast = cnt[idx] + (d >= 0)
            bad = (~near) & (fast != exact)
            assert not np.any(bad), f"sign {sign}, offset {p}: {int(bad.sum())} quotients miscoded, first {x[bad][:4]}"
