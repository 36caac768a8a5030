"""Pins for the oracle's code tables (CPU only).

The pages fix the table sizes and that they are constant and shared
(gate walkthrough, section 2.4); the values follow published definitions
(QLoRA section 3 for NF4; the dynamic tree map of 8-bit Optimizers section 2
for the nested table). These tests re-derive the tables by a different route
(root finding with math.erfc, bit-pattern decoding) and check the invariants.
"""
import math

import numpy as np
import pytest

from oracle import tables


def _ppf_bisect(p: float) -> float:
    """Standard normal quantile by bisection on math.erfc (independent of scipy)."""
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_nf4_structure():
    c4 = tables.nf4_table()
    assert c4.dtype == np.float32 and c4.shape == (16,)
    assert np.all(np.diff(c4) > 0)
    assert c4[0] == -1.0 and c4[15] == 1.0 and c4[7] == 0.0
    assert np.sum(c4 > 0) == 8 and np.sum(c4 < 0) == 7


def test_nf4_values_by_independent_root_finding():
    d = tables.NF4_DELTA
    zmax = _ppf_bisect(d)
    pos_p = [d - (d - 0.5) * i / 8 for i in range(8)]     # 8 probabilities, top first
    neg_p = [d - (d - 0.5) * i / 7 for i in range(7)]
    expect = sorted([-_ppf_bisect(p) / zmax for p in neg_p] + [0.0] +
                    [_ppf_bisect(p) / zmax for p in pos_p])
    expect = np.array(expect, dtype=np.float32)
    got = tables.nf4_table()
    # both are one fp32 rounding of the same real number
    assert np.array_equal(got, expect), (got, expect)


def test_nf4_equal_probability_spacing():
    # Each positive level is the quantile of an equally spaced probability.
    c4 = tables.nf4_table_f64()
    zmax = _ppf_bisect(tables.NF4_DELTA)
    cdf = [0.5 * math.erfc(-(c * zmax) / math.sqrt(2.0)) for c in c4[8:]]
    steps = np.diff([0.5] + cdf)
    assert np.allclose(steps, (tables.NF4_DELTA - 0.5) / 8, rtol=1e-9)
    cdfn = [0.5 * math.erfc((c * zmax) / math.sqrt(2.0)) for c in c4[:7][::-1]]
    stepsn = np.diff([0.5] + cdfn)
    assert np.allclose(stepsn, (tables.NF4_DELTA - 0.5) / 7, rtol=1e-9)


def _decode_dynamic(byte: int) -> float:
    """Decode one 8-bit dynamic-tree code from its bit pattern."""
    sign = -1.0 if byte & 0x80 else 1.0
    bits = byte & 0x7F
    if bits == 0:
        return 1.0 if sign < 0 else 0.0
    e = 0
    while not (bits >> (6 - e)) & 1:   # count leading zeros in the 7 bits
        e += 1
    frac_bits = 6 - e
    j = bits & ((1 << frac_bits) - 1)
    nbins = 1 << frac_bits
    centre = 0.1 + 0.9 * (2 * j + 1) / (2 * nbins)
    return sign * centre * 10.0 ** (-e)


def test_dynamic_table_by_bit_pattern_decoding():
    dec = np.array(sorted(_decode_dynamic(b) for b in range(256)), dtype=np.float32)
    got = tables.dynamic_table()
    assert np.array_equal(dec, got)


def test_dynamic_structure():
    c8 = tables.dynamic_table()
    assert c8.shape == (256,) and c8.dtype == np.float32
    assert np.all(np.diff(c8) > 0)
    assert c8[127] == 0.0 and c8[255] == 1.0
    # negatives mirror the positives below 1.0
    assert np.array_equal(-c8[:127][::-1], c8[128:255])
    # decade populations 64, 32, ..., 1 (per sign)
    pos = c8[128:255].astype(np.float64)
    counts = [int(np.sum((pos >= 0.1 * 10.0 ** -e) & (pos < 10.0 ** -e))) for e in range(7)]
    assert counts == [64, 32, 16, 8, 4, 2, 1]
    # top bin centre and the smallest magnitude
    assert c8[254] == np.float32(0.1 + 0.9 * 127 / 128)
    assert c8[128] == np.float32(0.55e-6)


@pytest.mark.parametrize("which", ["nf4", "dyn"])
def test_midpoints_lie_between_levels(which):
    t = tables.nf4_table() if which == "nf4" else tables.dynamic_table()
    m = tables.midpoints(t)
    assert np.all(t[:-1] < m) and np.all(m < t[1:])


def test_nf4_thresholds_clear_of_the_quantiser_buckets():
    """The quantiser's division-free code search splits v/m in [-1, 1] into
    buckets of width 1/128 and assumes at most one threshold per bucket, none
    within 1/64 of a bucket width of an edge (the margin its host check
    demands). Measured: 0.0297 widths at the closest threshold."""
    m = tables.midpoints(tables.nf4_table()).astype(np.float32).astype(np.float64)
    pos = (m + 1.0) * 128.0
    frac = pos - np.floor(pos)
    assert np.min(np.minimum(frac, 1.0 - frac)) >= 1.0 / 64
    assert len(set(np.floor(pos).astype(int))) == 15


def test_table_hash_changes_with_any_bit():
    c4, c8 = tables.nf4_table(), tables.dynamic_table()
    h = tables.table_hash(c4, c8)
    c4b = c4.copy()
    c4b.view(np.uint32)[3] ^= 1
    assert tables.table_hash(c4b, c8) != h
    c8b = c8.copy()
    c8b.view(np.uint32)[200] ^= 1
    assert tables.table_hash(c4, c8b) != h
    # FNV-1a reference vector: empty input gives the offset basis
    assert tables.table_hash(np.zeros(0, np.float32), np.zeros(0, np.float32)) == 0xCBF29CE484222325
