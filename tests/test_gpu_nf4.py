"""GPU parity of the sharder and the dequantiser against the oracle: bit-exact.

Gate walkthrough ("Soup layer-streamed NF4 training measured"), section 2.2
check 0: the offline shard bytes are identical to the resident quantised
weight (packed + absmax + nested absmax); section 2.3: the quantiser is
deterministic across repeats.
"""
import numpy as np
import pytest
import torch

import layer_streamed_nf4_amd as L
import synth
from oracle import nf4
from tests.gpu_helpers import (bits_to_f32, dev_bf16bits, host_u16, quantize_on_gpu, require_gpu,
                               sections, stream)

pytestmark = pytest.mark.gpu

SHAPES = [
    ("q", 576, 576),      # config 1 / 135M q,o: 21 nested blocks, the last partial
    ("k", 192, 576),      # 135M k,v: 6.75 nested blocks
    ("gate", 1536, 576),
    ("down", 576, 1536),
    ("q", 4096, 4096),    # 8B q,o
    ("v", 1024, 4096),    # 8B k,v
    ("gate", 14336, 4096),  # 8B gate,up
    ("down", 4096, 14336),  # 8B down
    ("q", 8, 64),         # one nested block holding 8 absmax
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _compare(w, shard, d):
    ref = nf4.quantize(w)
    packed, q8, nested, offset = sections(shard, d)
    assert offset.view(np.uint32) == np.float32(ref.offset).view(np.uint32), (offset, ref.offset)
    assert np.array_equal(nested.view(np.uint32), ref.nested.view(np.uint32))
    assert np.array_equal(q8, ref.q8)
    assert np.array_equal(packed, ref.packed)
    return ref


@pytest.mark.parametrize("proj,n,k", SHAPES)
def test_quantize_and_dequant_bit_exact(proj, n, k):
    print(f"quantize {proj} {n}x{k}", flush=True)
    w = synth.weight(7, proj, n, k)
    shard, d, status = quantize_on_gpu(w, base=512)
    assert status == 0
    ref = _compare(w, shard, d)
    out = torch.empty((n, k), dtype=torch.int16, device="cuda")
    L.nf4_dequant(shard.data_ptr(), d, out.data_ptr(), stream())
    got = host_u16(out)
    assert np.array_equal(got, nf4.dequantize_bf16(ref))


def test_quantize_bf16_input():
    w32 = synth.weight(3, "o", 576, 576)
    bits = (w32.view(np.uint32) >> 16).astype(np.uint16)     # a bf16 weight
    shard, d, status = quantize_on_gpu(bits, dtype=L.DTYPE_BF16)
    assert status == 0
    _compare(bits_to_f32(bits), shard, d)


def test_special_weights():
    w = np.zeros((64, 1024), np.float32)
    w[0, :64] = np.linspace(-1, 1, 64, dtype=np.float32)
    w[1, 5] = 3.0                        # one non-zero element in a block
    w[2, :] = -0.5                        # constant negative rows
    w[3, 64:128] = 1e-30                  # tiny magnitudes
    shard, d, status = quantize_on_gpu(w)
    assert status == 0
    _compare(w, shard, d)


def test_non_finite_weight_is_flagged():
    w = synth.weight(1, "k", 64, 128)
    w[3, 7] = np.inf
    _, _, status = quantize_on_gpu(w)
    assert status == 1


def test_quantize_deterministic_and_roundtrip():
    w = synth.weight(11, "v", 1024, 4096)
    s1, d, _ = quantize_on_gpu(w)
    s2, _, _ = quantize_on_gpu(w)
    assert torch.equal(s1, s2)
    # device -> host -> device keeps the bytes, and the dequantised weight
    back = s1.cpu().to("cuda")
    o1 = torch.empty((1024, 4096), dtype=torch.int16, device="cuda")
    o2 = torch.empty_like(o1)
    L.nf4_dequant(s1.data_ptr(), d, o1.data_ptr(), stream())
    L.nf4_dequant(back.data_ptr(), d, o2.data_ptr(), stream())
    assert torch.equal(o1, o2)


def test_flipped_nibble_is_detected():
    # a single corrupted nibble must break bit-exactness (the check has teeth)
    w = synth.weight(2, "q", 576, 576)
    shard, d, _ = quantize_on_gpu(w)
    ref = nf4.quantize(w)
    h = shard.cpu()
    h[d.off_packed + 1234] ^= 0x10
    packed = h.numpy()[d.off_packed:d.off_packed + 576 * 576 // 2]
    assert not np.array_equal(packed, ref.packed)
    out = torch.empty((576, 576), dtype=torch.int16, device="cuda")
    L.nf4_dequant(h.to("cuda").data_ptr(), d, out.data_ptr(), stream())
    assert not np.array_equal(host_u16(out), nf4.dequantize_bf16(ref))


def test_threshold_ties_bit_exact():
    """Weights on, one ulp above and one ulp below every NF4 threshold; absmax
    values whose centred form lands exactly on thresholds of the 256-level
    table; and absmax values whose mean needs the exact sum (a plain fp64
    running sum rounds the offset the other way): the device sharder gives the
    oracle's bytes in every case, and the offset of the last is 1 + 2^-23."""
    from tests.nf4_cases import nested_ties, nf4_ties, offset_needs_exact_sum
    for w in (nf4_ties(), nested_ties()[0], offset_needs_exact_sum()):
        shard, d, status = quantize_on_gpu(w)
        assert status == 0
        ref = _compare(w, shard, d)
        out = torch.empty(w.shape, dtype=torch.int16, device="cuda")
        L.nf4_dequant(shard.data_ptr(), d, out.data_ptr(), stream())
        assert np.array_equal(host_u16(out), nf4.dequantize_bf16(ref))
    _, _, _, offset = sections(quantize_on_gpu(offset_needs_exact_sum())[0],
                               L.nf4s_tensor_layout(64, 256))
    assert offset == np.float32(1 + 2.0 ** -23)
