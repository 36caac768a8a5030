"""Code tables of the NF4 double-quant format, derived from their definitions.

TEST INFRASTRUCTURE (see oracle/__init__.py). Parity unpinned by the pages for
the *values*: the gate walkthrough (section 2.4) states only that the NF4 table
holds 16 fp32 values and the nested table 256 fp32 values, both constant for
every weight and shared. The values below follow the published definitions
named in each function; tests pin the derivation (independent root finding,
bit-pattern decoding, invariants), not the choice of definition.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
from scipy.special import ndtri

# Endpoint probability of the NF4 construction. The normal quantile function is
# infinite at 0 and 1, so the outermost quantile is pulled in to the mean of the
# top-bin centres for 15 and 16 equal-probability bins:
#   delta = ((1 - 1/30) + (1 - 1/32)) / 2 = 0.96770833...
# (reading: QLoRA leaves this constant to its code; this value is the one that
# reproduces the NF4 constants QLoRA publishes).
NF4_DELTA = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))


def nf4_table_f64(delta: float = NF4_DELTA) -> np.ndarray:
    """NormalFloat-4 levels in fp64, ascending (QLoRA section 3, "4-bit NormalFloat").

    Asymmetric quantile construction: 8 equal-probability steps of the standard
    normal on the positive side and 7 on the negative side, each starting at
    probability 1/2 (quantile 0) and ending at ``delta``; the two zeros merge
    into one exact 0; everything is divided by the largest quantile so the
    range is exactly [-1, 1].
    """
    pos_p = np.linspace(delta, 0.5, 9)[:-1]      # 8 probabilities, excluding 1/2
    neg_p = np.linspace(delta, 0.5, 8)[:-1]      # 7 probabilities, excluding 1/2
    zmax = ndtri(delta)
    pos = ndtri(pos_p) / zmax
    neg = -ndtri(neg_p) / zmax
    vals = np.concatenate([neg, [0.0], pos])
    vals.sort()
    vals[0], vals[-1] = -1.0, 1.0                # exact by construction
    return vals


def nf4_table() -> np.ndarray:
    """The 16-entry NF4 table as float32 (one rounding from fp64)."""
    return nf4_table_f64().astype(np.float32)


def dynamic_table_f64() -> np.ndarray:
    """Signed dynamic-tree 8-bit map in fp64, ascending, 256 entries.

    Definition (8-bit Optimizers via Block-wise Quantization, section 2,
    "dynamic tree quantization"): after the sign bit, a run of e zero bits
    (e = 0..6) sets the decimal exponent 10**-e, the first one bit is an
    indicator, and the remaining 6-e bits index 2**(6-e) linear bins of
    [0.1, 1]; a code's value is the centre of its bin times 10**-e. The
    all-zero magnitude pattern encodes 0 with sign 0 and 1.0 with sign 1,
    which fills all 256 codes. Reading: the pages never name the nested
    table; this map is the one the pages' producer uses for nested absmax.
    """
    mags = []
    for e in range(7):
        nbins = 2 ** (6 - e)
        for j in range(nbins):
            centre = 0.1 + 0.9 * (2 * j + 1) / (2 * nbins)
            mags.append(centre * 10.0 ** (-e))
    mags = np.array(mags)
    vals = np.concatenate([-mags, mags, [0.0, 1.0]])
    vals.sort()
    return vals


def dynamic_table() -> np.ndarray:
    return dynamic_table_f64().astype(np.float32)


def midpoints(table: np.ndarray) -> np.ndarray:
    """Decision thresholds between consecutive levels, in fp32:
    m_i = fp32(fp32(t_i + t_{i+1}) * 0.5). A normalised value v gets code
    #{i : v > m_i}, i.e. the nearest level with ties going to the lower code."""
    t = table.astype(np.float32)
    return ((t[:-1] + t[1:]) * np.float32(0.5)).astype(np.float32)


def table_hash(c4: np.ndarray, c8: np.ndarray) -> int:
    """FNV-1a (64-bit) over the little-endian bytes of C4 then C8: the key a
    shard carries so that it is never dequantised with other constants."""
    h = 0xCBF29CE484222325
    for byte in c4.astype("<f4").tobytes() + c8.astype("<f4").tobytes():
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def exact_fraction(x: float) -> Fraction:
    return Fraction(float(x))
