"""NF4 blockwise quantisation with double-quantised absmax, and its inverse.

TEST INFRASTRUCTURE (see oracle/__init__.py).

What the pages fix (gate walkthrough, "Soup layer-streamed NF4 training
measured", sections 2.1 and 2.4): weights are quantised offline, one tensor at
a time, blockwise with block 64; each shard stores uint8-packed 4-bit codes and
the per-block absmax; with double quant the absmax is itself quantised and the
shard also carries a nested absmax and one offset. Streamed bytes per weight
are packed N/2 + absmax N/64 + nested absmax N/4096 + a 4-byte offset, about
0.516 bytes per parameter. Every weight uses the same 16-entry NF4 table and
256-entry nested table. Quantisation is deterministic across repeats and
across a CPU round trip (section 2.3).

Readings where the pages are silent:
  * flatten order: row-major W[N_out, K_in]; block b is elements [64b, 64b+64),
    nested block j is absmax blocks [256j, 256j+256); the last nested block may
    be partial;
  * code choice: v = w / absmax in fp32 (IEEE division), code = #{i : v > m_i}
    with fp32 midpoints m_i (nearest level, ties to the lower code); an
    all-zero block gets v = 0, i.e. the code of level 0;
  * packing: byte j = code[2j] << 4 | code[2j+1] (even element in the high nibble);
  * offset: the mean of the tensor's fp32 absmax values (QLoRA section 3,
    "Double Quantization": centre the constants, then quantise them
    symmetrically), evaluated as fp32(fp64(exact sum) / nb);
  * nested quantisation: c = fp32(absmax - offset); nested[j] = max|c| over
    nested block j; q8 = #{i : c/nested > m8_i} with fp32 division and fp32
    midpoints of the dynamic table; nested = 0 gives the code of 0;
  * dequantisation: a' = fp32(fp32(C8[q8] * nested) + offset) with two separate
    roundings (no fused multiply-add), W' = bf16_rne(fp32(C4[q] * a')).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import tables

BLOCK = 64
NESTED = 256


@dataclass
class QuantTensor:
    n_out: int
    k_in: int
    packed: np.ndarray   # uint8 [N/2]
    q8: np.ndarray       # uint8 [nb]
    nested: np.ndarray   # float32 [nn]
    offset: np.float32   # float32 scalar
    absmax: np.ndarray   # float32 [nb] (intermediate, not part of the shard)
    codes: np.ndarray    # uint8 [N] (intermediate, unpacked)


def n_blocks(n: int) -> int:
    return -(-n // BLOCK)


def n_nested(n: int) -> int:
    return -(-n_blocks(n) // NESTED)


def payload_bytes(n_out: int, k_in: int) -> int:
    """Streamed bytes of one tensor: packed + 8-bit absmax + fp32 nested + offset."""
    n = n_out * k_in
    return n // 2 + n_blocks(n) + 4 * n_nested(n) + 4


def codes_nearest(v: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the nearest table level for normalised values v (float32):
    #{i : v > m_i} with fp32 midpoints, i.e. ties go to the lower code."""
    mids = tables.midpoints(table)
    # searchsorted(side='left') counts the midpoints strictly below v.
    return np.searchsorted(mids, v.astype(np.float32), side="left").astype(np.uint8)


def exact_mean_f32(a: np.ndarray) -> np.float32:
    """fp32(fp64(exact sum of a) / len(a)); math.fsum is exact then rounds once."""
    s = math.fsum(a.astype(np.float64).tolist())
    return np.float32(s / len(a))


def quantize(w: np.ndarray) -> QuantTensor:
    """Quantise W[N_out, K_in] (float32) to NF4 with double-quantised absmax."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    n_out, k_in = w.shape
    n = w.size
    if n % 2:
        raise ValueError("odd element count cannot be nibble-packed")
    c4 = tables.nf4_table()
    c8 = tables.dynamic_table()

    flat = w.reshape(-1)
    nb = n_blocks(n)
    pad = nb * BLOCK - n
    blocks = np.concatenate([flat, np.zeros(pad, np.float32)]).reshape(nb, BLOCK)

    # absmax per 64-block (exact: max of magnitudes)
    absmax = np.abs(blocks).max(axis=1).astype(np.float32)

    # normalise in fp32 and pick the nearest NF4 level
    safe = np.where(absmax > 0, absmax, np.float32(1.0))
    v = (blocks / safe[:, None]).astype(np.float32)
    v[absmax == 0, :] = np.float32(0.0)
    codes = codes_nearest(v, c4).reshape(-1)[:n]

    # nibble packing: even element high
    packed = ((codes[0::2] << 4) | codes[1::2]).astype(np.uint8)

    # double quantisation of the absmax
    offset = exact_mean_f32(absmax)
    centred = (absmax - offset).astype(np.float32)
    nn = n_nested(n)
    npad = nn * NESTED - nb
    cpad = np.concatenate([centred, np.zeros(npad, np.float32)]).reshape(nn, NESTED)
    nested = np.abs(cpad).max(axis=1).astype(np.float32)
    nsafe = np.where(nested > 0, nested, np.float32(1.0))
    u = (cpad / nsafe[:, None]).astype(np.float32)
    u[nested == 0, :] = np.float32(0.0)
    q8 = codes_nearest(u, c8).reshape(-1)[:nb]

    return QuantTensor(n_out, k_in, packed, q8, nested, offset, absmax, codes)


def unpack(packed: np.ndarray) -> np.ndarray:
    out = np.empty(packed.size * 2, np.uint8)
    out[0::2] = packed >> 4
    out[1::2] = packed & 0x0F
    return out


def decoded_absmax(q: QuantTensor) -> np.ndarray:
    """a'[b] = fp32(fp32(C8[q8[b]] * nested[b >> 8]) + offset), two roundings."""
    c8 = tables.dynamic_table()
    j = np.arange(q.q8.size) // NESTED
    prod = (c8[q.q8] * q.nested[j]).astype(np.float32)
    return (prod + q.offset).astype(np.float32)


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even on the dropped 16 bits (finite x)."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def dequantize_f32(q: QuantTensor) -> np.ndarray:
    """fp32(C4[code] * a'[block]) before the bf16 rounding, shape [N_out, K_in]."""
    c4 = tables.nf4_table()
    codes = unpack(q.packed)
    a = decoded_absmax(q)
    blk = np.arange(codes.size) // BLOCK
    return (c4[codes] * a[blk]).astype(np.float32).reshape(q.n_out, q.k_in)


def dequantize_bf16(q: QuantTensor) -> np.ndarray:
    """W' as bf16 bit patterns [N_out, K_in] (the weight the GEMMs contract with)."""
    return bf16_rne_bits(dequantize_f32(q))
