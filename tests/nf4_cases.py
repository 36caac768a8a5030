"""Constructed weight tensors whose quantisation lands exactly on decision
thresholds, shared by the oracle pins and the GPU parity tests. The thresholds
come from the oracle's tables (the tests' side); nothing here quantises.

Gate walkthrough ("Soup layer-streamed NF4 training measured"), section 2.3:
the quantiser is deterministic; section 2.4: one constant 16-level and one
256-level table for every tensor. Nearest level with ties to the lower code,
and the offset as the exact mean of the fp32 absmax, are the readings these
cases pin at their edges.
"""
import numpy as np

from oracle import tables


def nf4_ties() -> np.ndarray:
    """[8, 256] fp32. Every 64-block has a power-of-two absmax a (2^-6 ..
    2^1, so w / a is exact) held by its first element; the others are a times
    each NF4 threshold, a times one ulp above and below it, and the negated
    thresholds: w / a lands exactly on, just above or just below a midpoint."""
    mids = tables.midpoints(tables.nf4_table())
    up = np.nextafter(mids, np.float32(2))
    dn = np.nextafter(mids, np.float32(-2))
    w = np.zeros((8, 256), np.float32)
    flat = w.reshape(-1, 64)
    for b in range(flat.shape[0]):
        a = np.float32(2.0 ** (b % 8 - 6))
        row = np.zeros(64, np.float32)
        row[0] = a if b % 2 == 0 else -a
        vals = (mids, up, dn, -mids)[b % 4]
        row[1:16] = a * vals
        row[16:31] = a * mids[::-1]
        row[31:46] = -a * up
        flat[b] = row
    return w


def nested_ties():
    """[64, 256] fp32 = one nested block of 256 absmax values with mean exactly
    1 and nested absmax exactly 1, so every centred value c = fp32(a - 1)
    is exact and c / 1 lands exactly on a threshold of the 256-level table
    wherever a = 1 +- threshold is an fp32 number. Returns (w, thresholds hit)."""
    mids = tables.midpoints(tables.dynamic_table()).astype(np.float64)
    ok = [m for m in mids if abs(m) < 1 and float(np.float32(1 + m)) - 1 == m
          and float(np.float32(1 - m)) - 1 == -m]
    absmax = [2.0, 0.0]          # c = +1 and -1: the nested absmax is 1
    for m in ok:
        if len(absmax) >= 256:
            break
        absmax += [1 + m, 1 - m]
    k = 1
    while len(absmax) < 256:     # pad with exact symmetric pairs
        absmax += [1 + k / 1024, 1 - k / 1024]
        k += 1
    w = np.zeros((256, 64), np.float32)
    w[:, 0] = np.array(absmax, np.float64).astype(np.float32)
    w[1::3, 5] = -w[1::3, 0]     # the absmax also from negative weights
    w[:, 9] = w[:, 0] * np.float32(0.5)
    return w.reshape(64, 256), ok


def offset_needs_exact_sum() -> np.ndarray:
    """[64, 256] fp32, 256 blocks: absmax 2 (127 blocks), 2 + 2^-16 (one) and
    2^-49 (128). The exact mean is 1 + 2^-24 + 2^-50, which rounds up to
    1 + 2^-23 in fp32; a plain fp64 running sum drops the 2^-49 terms (below
    half an ulp of the running total) and lands on the tie 1 + 2^-24, which
    rounds to 1.0. The values span 2^57, inside what a double-double sum of
    up to 2^21 fp32 values keeps exactly."""
    absmax = np.empty(256, np.float64)
    absmax[:127] = 2.0
    absmax[127] = 2.0 + 2.0 ** -16
    absmax[128:] = 2.0 ** -49
    w = np.zeros((256, 64), np.float32)
    w[:, 0] = absmax.astype(np.float32)
    return w.reshape(64, 256)
