"""Pins for the oracle's NF4 double-quant quantiser and dequantiser (CPU only).

Pinned against: brute force on tiny tensors (exact rational arithmetic),
special cases with known codes, the exact mean for the offset, determinism
and a byte round trip (gate walkthrough, section 2.3), idempotence of
re-quantising dequantised values, and the byte formula against the totals the
pages print (section 2.2, 2.4, 4.2, 4.3).
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import nf4, tables


def _nearest_exact(v: float, table) -> int:
    """Exact nearest level by rational distance; ties go to the lower index."""
    fv = Fraction(float(v))
    best, bestd = 0, None
    for i, t in enumerate(table):
        d = abs(fv - Fraction(float(t)))
        if bestd is None or d < bestd:
            best, bestd = i, d
    return best


def _near_midpoint(v, table) -> bool:
    """True if v lies within one fp32 ulp of an exact midpoint, where the fp32
    midpoint rule may legitimately differ from the exact nearest level."""
    for a, b in zip(table[:-1], table[1:]):
        m = (float(a) + float(b)) / 2
        if abs(float(v) - m) <= 2 * np.spacing(np.float32(m)):
            return True
    return False


def _brute_codes(w: np.ndarray):
    """Per-element brute force for the NF4 codes of a tiny tensor."""
    c4 = tables.nf4_table()
    flat = w.reshape(-1)
    out = []
    for b in range(0, flat.size, 64):
        blk = flat[b:b + 64]
        a = max(abs(float(x)) for x in blk)
        for x in blk:
            v = np.float32(x) / np.float32(a) if a > 0 else np.float32(0.0)
            out.append((_nearest_exact(v, c4), v))
    return out


@pytest.mark.parametrize("shape,seed", [((4, 64), 0), ((2, 128), 1), ((3, 192), 2)])
def test_codes_brute_force(shape, seed):
    w = np.random.Generator(np.random.PCG64(seed)).standard_normal(shape).astype(np.float32) * 0.02
    q = nf4.quantize(w)
    c4 = tables.nf4_table()
    for i, (code, v) in enumerate(_brute_codes(w)):
        if q.codes[i] != code:
            assert _near_midpoint(v, c4), (i, v, q.codes[i], code)
            # the fp32 midpoint rule decides; check it directly
            mids = tables.midpoints(c4)
            assert q.codes[i] == int(np.sum(np.float32(v) > mids))


def test_special_cases():
    w = np.zeros((2, 64), np.float32)
    w[0, 5] = 0.3       # the block maximum -> exactly +1 -> top code
    w[0, 9] = -0.3      # -absmax -> exactly -1 -> code 0
    w[0, 10] = 0.15
    q = nf4.quantize(w)
    codes = q.codes.reshape(2, 64)
    assert codes[0, 5] == 15 and codes[0, 9] == 0
    assert np.all(codes[1] == 7)            # all-zero block -> level 0 (index 7)
    assert codes[0, 0] == 7                  # zero inside a non-zero block
    c4 = tables.nf4_table()
    assert codes[0, 10] == int(np.argmin(np.abs(c4 - np.float32(0.5))))
    assert q.absmax[1] == 0.0


def test_exact_midpoint_goes_to_lower_code():
    c4 = tables.nf4_table()
    mids = tables.midpoints(c4)
    w = np.zeros((1, 64), np.float32)
    w[0, 0] = 1.0                            # absmax 1 -> v equals w exactly
    w[0, 1:16] = mids                        # every decision threshold exactly
    w[0, 16:31] = np.nextafter(mids, np.float32(2))   # one ulp above each
    q = nf4.quantize(w)
    assert q.codes[1:16].tolist() == list(range(15))
    assert q.codes[16:31].tolist() == list(range(1, 16))


def test_single_nonzero_block_and_zero_nested():
    # 512 zero blocks -> two nested blocks; only one block has any weight.
    w = np.zeros((1, 64 * 512), np.float32)
    w[0, 70] = 0.1
    q = nf4.quantize(w)
    assert q.absmax[1] == np.float32(0.1) and np.count_nonzero(q.absmax) == 1
    assert q.offset == np.float32(0.1 / 512)
    c8 = tables.dynamic_table()
    # centred values: -offset everywhere except block 1
    assert q.nested[0] == np.float32(np.float32(0.1) - q.offset)
    assert q.q8[1] == 255                    # c/nested == 1 -> the 1.0 level
    assert q.nested[1] == q.offset           # all centred values equal -offset
    assert np.all(q.q8[256:] == 0) and c8[0] < 0   # -1 normalised -> lowest code
    # partial nested block (576x576: 5184 blocks -> 21 nested, the last holds 64)
    w2 = synth.weight(0, "q", 576, 576)
    q2 = nf4.quantize(w2)
    assert q2.nested.size == 21 and q2.q8.size == 5184


def test_all_zero_tensor():
    q = nf4.quantize(np.zeros((4, 64), np.float32))
    assert np.all(q.codes == 7)
    assert q.offset == 0.0 and np.all(q.nested == 0)
    assert np.all(q.q8 == 127)               # index of level 0 in the nested table
    assert np.all(nf4.dequantize_bf16(q) == 0)


def test_offset_is_exact_mean():
    w = synth.weight(3, "k", 192, 576)
    q = nf4.quantize(w)
    exact = sum(Fraction(float(a)) for a in q.absmax) / len(q.absmax)
    assert q.offset == np.float32(float(exact))
    # and the absmax themselves are the per-block maxima
    assert np.array_equal(q.absmax, np.abs(w.reshape(-1, 64)).max(axis=1))


def test_packing_roundtrip_and_order():
    w = synth.weight(1, "v", 192, 576)
    q = nf4.quantize(w)
    assert np.array_equal(nf4.unpack(q.packed), q.codes)
    assert q.packed[0] == (q.codes[0] << 4) | q.codes[1]


def test_determinism_and_byte_roundtrip():
    w = synth.weight(2, "o", 576, 576)
    q1, q2 = nf4.quantize(w), nf4.quantize(w.copy())
    for f in ("packed", "q8", "nested"):
        assert getattr(q1, f).tobytes() == getattr(q2, f).tobytes()
    assert q1.offset == q2.offset
    # through bytes and back (a host round trip)
    w_rt = np.frombuffer(w.tobytes(), dtype=np.float32).reshape(w.shape)
    q3 = nf4.quantize(w_rt)
    assert q3.packed.tobytes() == q1.packed.tobytes()


def test_dequant_per_element_brute_force():
    w = synth.weight(0, "k", 20, 2048)         # 640 blocks -> 3 nested blocks, last partial
    q = nf4.quantize(w)
    c4, c8 = tables.nf4_table(), tables.dynamic_table()
    deq = nf4.dequantize_bf16(q).reshape(-1)
    codes = nf4.unpack(q.packed)
    rng = np.random.Generator(np.random.PCG64(9))
    for e in rng.integers(0, codes.size, 400):
        b = e // 64
        a = np.float32(np.float32(c8[q.q8[b]]) * np.float32(q.nested[b // 256]))
        a = np.float32(a + q.offset)
        val = np.float32(c4[codes[e]] * a)
        bits = int(np.array([val], np.float32).view(np.uint32)[0])
        # round half to even by exact integer reasoning
        lo = bits & 0xFFFF
        hi = bits >> 16
        if lo > 0x8000 or (lo == 0x8000 and (hi & 1)):
            hi += 1
        assert deq[e] == hi, e


def test_requantise_is_idempotent():
    w = synth.weight(4, "gate", 64, 576)
    q = nf4.quantize(w)
    deq = nf4.dequantize_f32(q).reshape(-1, 64)
    a = nf4.decoded_absmax(q)
    v = (deq / np.where(a > 0, a, 1)[:, None]).astype(np.float32)
    again = nf4.codes_nearest(v, tables.nf4_table()).reshape(-1)
    assert np.array_equal(again, q.codes)


def test_dequant_error_bound():
    w = synth.weight(5, "up", 128, 576)
    q = nf4.quantize(w)
    deq = nf4.bf16_to_f32(nf4.dequantize_bf16(q)).reshape(-1, 64).astype(np.float64)
    c4 = tables.nf4_table().astype(np.float64)
    half_gap = np.max(np.diff(c4)) / 2
    a_true = q.absmax.astype(np.float64)
    a_dec = nf4.decoded_absmax(q).astype(np.float64)
    bound = a_true * half_gap + np.abs(a_dec - a_true) + np.abs(a_dec) * 2.0 ** -8
    err = np.abs(deq - w.reshape(-1, 64)).max(axis=1)
    assert np.all(err <= bound * (1 + 1e-6))
    # double quant loses little: decoded absmax within the nested grid's half gap
    c8 = tables.dynamic_table().astype(np.float64)
    nested = np.repeat(q.nested.astype(np.float64), 256)[: a_true.size]
    assert np.all(np.abs(a_dec - a_true) <= nested * np.max(np.diff(c8)) / 2 + 1e-9)


def test_bf16_round_to_nearest_even():
    x = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF, 0xBF808000, 0xBF818000],
                 np.uint32).view(np.float32)
    got = nf4.bf16_rne_bits(x)
    assert got.tolist() == [0x3F80, 0x3F82, 0x3F81, 0x3F80, 0xBF80, 0xBF82]


def test_payload_formula_matches_page_totals(golden):
    # per tensor N/2 + N/64 + 4*N/16384 + 4 bytes
    assert nf4.payload_bytes(576, 576) == 165888 + 5184 + 21 * 4 + 4
    from oracle.stack import layer_shard_payload
    per135 = layer_shard_payload(synth.SHAPES["135m"])
    per8 = layer_shard_payload(synth.SHAPES["8b"])
    assert per135 == 1_825_668 and per8 == 112_513_052
    g = golden
    s135 = per135 * g["store_135m_gb"]["layers"] / 1e9
    s8 = per8 * g["store_8b_gb"]["layers"] / 1e9
    assert round(s135, 3) == g["store_135m_gb"]["value"]
    assert round(s8, 2) == g["store_8b_gb"]["value"]
    emb = 2 * g["embed_lm_head_8b_gb"]["vocab"] * g["embed_lm_head_8b_gb"]["hidden"] * 2 / 1e9
    assert round(emb, 2) == g["embed_lm_head_8b_gb"]["value"]
    assert round(s8 + emb, 2) == g["shard_set_8b_gb"]["value"]
    params8 = sum(a * b for a, b in synth.SHAPES["8b"].values())
    assert round(per8 / params8, 3) == g["bytes_per_param_approx"]["value"]


def test_nf4_ties_at_every_threshold():
    """Weights that divide exactly onto each NF4 threshold (power-of-two
    absmax) take the lower code; one ulp above takes the upper code, one ulp
    below the lower; the exact-rational brute force agrees away from the
    thresholds."""
    from tests.nf4_cases import nf4_ties
    w = nf4_ties()
    q = nf4.quantize(w)
    codes = q.codes.reshape(-1, 64)
    for b in range(codes.shape[0]):
        kind = b % 4
        got = codes[b, 1:16].tolist()
        if kind in (0, 2):        # on the threshold, or one ulp below: the lower code
            assert got == list(range(15)), (b, got)
        elif kind == 1:           # one ulp above: the upper code
            assert got == list(range(1, 16)), (b, got)
        else:                     # negated thresholds: mirror of the lower code rule
            assert got == [int(np.searchsorted(tables.midpoints(tables.nf4_table()), -m, "left"))
                           for m in tables.midpoints(tables.nf4_table())]
        assert codes[b, 16:31].tolist() == list(range(14, -1, -1))


def test_nested_ties_take_the_lower_code():
    from tests.nf4_cases import nested_ties
    w, hit = nested_ties()
    assert len(hit) >= 16
    q = nf4.quantize(w)
    assert q.offset == np.float32(1.0) and q.nested.tolist() == [1.0]
    mids = tables.midpoints(tables.dynamic_table()).astype(np.float64)
    c = (q.absmax.astype(np.float64) - 1.0)
    for b, cv in enumerate(c):
        on = np.nonzero(mids == cv)[0]
        if on.size:               # exactly on threshold i: code i (the lower level)
            assert q.q8[b] == on[0], (b, cv)
    assert sum(np.any(mids == cv) for cv in c) >= 2 * min(len(hit), 127)


def test_offset_needs_the_exact_sum():
    from tests.nf4_cases import offset_needs_exact_sum
    w = offset_needs_exact_sum()
    q = nf4.quantize(w)
    assert q.offset == np.float32(1 + 2.0 ** -23)
    # a plain running fp64 sum would give the tie, which rounds to 1.0
    run = 0.0
    for a in q.absmax.astype(np.float64):
        run += a
    assert np.float32(run / 256) == np.float32(1.0)
