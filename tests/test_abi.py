"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, reports the same code tables and byte accounting as the
oracle, and refuses bad arguments on the host before launching anything.

The oracle is imported only to compare constants; no value flows from the
library into the oracle.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import layer_streamed_nf4_amd as L
from oracle import nf4, tables

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "nf4stream.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_library_exports_every_declared_function():
    names = _header_functions()
    assert len(names) >= 20
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


def test_tables_match_oracle_bit_for_bit():
    c4, c8 = L.nf4_code_tables()
    assert c4.view(np.uint32).tolist() == tables.nf4_table().view(np.uint32).tolist()
    assert c8.view(np.uint32).tolist() == tables.dynamic_table().view(np.uint32).tolist()
    assert L.nf4s_table_hash() == tables.table_hash(tables.nf4_table(), tables.dynamic_table())


@pytest.mark.parametrize("shape", [(576, 576), (192, 576), (1536, 576), (576, 1536),
                                   (4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336),
                                   (27648, 5120), (8, 64)])
def test_shard_bytes_match_oracle(shape):
    assert L.nf4_shard_bytes(*shape) == nf4.payload_bytes(*shape)


def test_tensor_layout_sections():
    d = L.nf4s_tensor_layout(576, 576, 512)
    assert d.off_packed == 512
    for off in (d.off_q8, d.off_nested, d.off_offset, d.end):
        assert off % 256 == 0
    assert d.off_q8 >= d.off_packed + 576 * 576 // 2
    assert d.off_nested >= d.off_q8 + 5184
    assert d.off_offset >= d.off_nested + 21 * 4
    assert d.end >= d.off_offset + 4
    assert (d.method, d.blocksize, d.nested_block, d.double_quant) == (1, 64, 256, 1)


@pytest.mark.parametrize("n_out,k_in", [(576, 100), (0, 64), (7, 64), (64, -64)])
def test_layout_rejects_bad_shapes(n_out, k_in):
    with pytest.raises(L.Nf4sError) as e:
        L.nf4s_tensor_layout(n_out, k_in)
    assert e.value.code == L.ESHAPE


def test_layout_rejects_misaligned_base():
    with pytest.raises(L.Nf4sError) as e:
        L.nf4s_tensor_layout(64, 64, 100)
    assert e.value.code == L.EALIGN


def test_workspace_queries_depend_on_shape_only():
    a = L.nf4s_workspace_bytes(L.OP_LINEAR_FWD, 512, 4096, 4096)
    b = L.nf4s_workspace_bytes(L.OP_LINEAR_FWD, 512, 4096, 4096)
    assert a == b and a % 4 == 0
    # the absmax (5184 fp32, padded to 256 B) and one double-double partial
    # of the offset sum per 64 absmax values (81 of them; 14336 at 8B gate)
    assert L.nf4s_workspace_bytes(L.OP_QUANTIZE, 0, 576, 576) == 20736 + 81 * 16
    assert L.nf4s_workspace_bytes(L.OP_QUANTIZE, 0, 14336, 4096) == 917504 * 4 + 14336 * 16
    with pytest.raises(L.Nf4sError) as e:
        L.nf4s_workspace_bytes(99, 1, 64, 64)
    assert e.value.code == L.EINVAL
    # GEMM rows: at most 2^23 (the tile grid's y dimension stays below 65535)
    assert L.nf4s_workspace_bytes(L.OP_LINEAR_FWD, 1 << 23, 64, 64) >= 0
    for op in (L.OP_LINEAR_FWD, L.OP_LINEAR_BWD):
        with pytest.raises(L.Nf4sError) as e:
            L.nf4s_workspace_bytes(op, (1 << 23) + 1, 64, 64)
        assert e.value.code == L.ESHAPE


FAKE = 1 << 40  # a 256-byte aligned address that is never dereferenced


def _desc(n=64, k=64):
    return L.nf4s_tensor_layout(n, k)


def test_descriptor_key_mismatches_are_refused():
    d = _desc()
    d.double_quant = 0      # the sharder/reader double-quant flag disagreement
    with pytest.raises(L.Nf4sError) as e:
        L.nf4_dequant(FAKE, d, FAKE)
    assert e.value.code == L.EKEY
    d = _desc()
    d.blocksize = 32
    with pytest.raises(L.Nf4sError) as e:
        L.streamed_linear_fwd(FAKE, d, FAKE, 16, FAKE, None, None, 0, 0.0, None, 0)
    assert e.value.code == L.EKEY
    d = _desc()
    d.table_hash ^= 1
    with pytest.raises(L.Nf4sError) as e:
        L.streamed_linear_bwd(FAKE, d, FAKE, 16, FAKE, None, None, 0, None, 0)
    assert e.value.code == L.ETABLE
    d = _desc()
    d.off_q8 += 256
    with pytest.raises(L.Nf4sError) as e:
        L.nf4_dequant(FAKE, d, FAKE)
    assert e.value.code == L.EKEY


def test_pointer_and_argument_errors():
    d = _desc()
    with pytest.raises(L.Nf4sError) as e:
        L.nf4_dequant(None, d, FAKE)
    assert e.value.code == L.EINVAL
    with pytest.raises(L.Nf4sError) as e:
        L.nf4_dequant(FAKE + 16, d, FAKE)        # shard base must be 256-B aligned
    assert e.value.code == L.EALIGN
    with pytest.raises(L.Nf4sError) as e:
        L.streamed_linear_fwd(FAKE, d, FAKE + 2, 16, FAKE, None, None, 0, 0.0, None, 0)
    assert e.value.code == L.EALIGN
    with pytest.raises(L.Nf4sError) as e:     # LoRA operands come together
        L.streamed_linear_fwd(FAKE, d, FAKE, 16, FAKE, FAKE, None, 16, 2.0, None, 0)
    assert e.value.code == L.EINVAL
    with pytest.raises(L.Nf4sError) as e:     # rank out of range
        L.streamed_linear_fwd(FAKE, d, FAKE, 16, FAKE, FAKE, FAKE, 65, 2.0, None, 0)
    assert e.value.code == L.EINVAL
    with pytest.raises(L.Nf4sError) as e:
        L.streamed_linear_fwd(FAKE, d, FAKE, 0, FAKE, None, None, 0, 0.0, None, 0)
    assert e.value.code == L.ESHAPE
    with pytest.raises(L.Nf4sError) as e:     # non-finite LoRA scale
        L.streamed_linear_fwd(FAKE, d, FAKE, 16, FAKE, FAKE, FAKE, 16, float("nan"), None, 0)
    assert e.value.code == L.EINVAL
    with pytest.raises(L.Nf4sError) as e:
        L.nf4_quantize_shard(FAKE, 7, 64, 64, FAKE, d, None, FAKE, 1 << 20)
    assert e.value.code == L.EINVAL
    with pytest.raises(L.Nf4sError) as e:     # missing workspace
        L.nf4_quantize_shard(FAKE, L.DTYPE_F32, 64, 64, FAKE, d, None, None, 0)
    assert e.value.code == L.EWORKSPACE
    with pytest.raises(L.Nf4sError) as e:     # descriptor for another shape
        L.nf4_quantize_shard(FAKE, L.DTYPE_F32, 128, 64, FAKE, d, None, FAKE, 1 << 20)
    assert e.value.code in (L.ESHAPE,)
    with pytest.raises(L.Nf4sError) as e:
        L.lora_fwd(FAKE, 16, 100, FAKE, 16, FAKE, FAKE, 1 << 20)
    assert e.value.code == L.ESHAPE
    with pytest.raises(L.Nf4sError) as e:
        L.lora_bwd(FAKE, FAKE, FAKE, 16, 64, 64, FAKE, 16, 2.0, FAKE, FAKE, FAKE, 2, FAKE, 1 << 30)
    assert e.value.code == L.EINVAL


def test_linear_workspace_is_required_when_split():
    d = L.nf4s_tensor_layout(4096, 4096)
    need = L.nf4s_workspace_bytes(L.OP_LINEAR_FWD, 512, 4096, 4096)
    assert need > 0                            # 64 output tiles: the contraction is split
    with pytest.raises(L.Nf4sError) as e:
        L.streamed_linear_fwd(FAKE, d, FAKE, 512, FAKE, None, None, 0, 0.0, FAKE, need - 4)
    assert e.value.code == L.EWORKSPACE


def test_prefetch_and_pool_argument_errors():
    with pytest.raises(L.Nf4sError) as e:
        L.layer_prefetch(FAKE, 1024, FAKE, 2048, None)      # shard larger than the slot
    assert e.value.code == L.ESLOT
    with pytest.raises(L.Nf4sError) as e:
        L.layer_prefetch(FAKE + 8, 1024, FAKE, 512, None)
    assert e.value.code == L.EALIGN
    with pytest.raises(L.Nf4sError) as e:
        L.nf4s_pool_create([FAKE], 1024, 1, 2)               # pool of one slot
    assert e.value.code == L.ESLOT
    with pytest.raises(L.Nf4sError) as e:
        L.nf4s_pool_create([FAKE] * 9, 1024, 1, 2)
    assert e.value.code == L.ESLOT
    with pytest.raises(L.Nf4sError) as e:
        L.nf4s_pool_create([FAKE, FAKE], 1024, 1, 1)         # copy stream == compute stream
    assert e.value.code == L.EINVAL
    with pytest.raises(L.Nf4sError) as e:
        L.nf4s_pool_create([FAKE, FAKE + 4096], 0, 1, 2)     # empty slots
    assert e.value.code == L.ESLOT
    # slots that share memory would let a copy overwrite a layer another
    # slot's reader still holds
    for slots in ([FAKE, FAKE], [FAKE, FAKE + 256], [FAKE + 4096, FAKE + 8192, FAKE + 4352]):
        with pytest.raises(L.Nf4sError) as e:
            L.nf4s_pool_create(slots, 1024, 1, 2)
        assert e.value.code == L.EINVAL, slots


def test_packed_activation_bytes():
    assert L.nf4s_packed_activation_bytes(512, 4096) == 512 * 4096 * 2
    assert L.nf4s_packed_activation_bytes(300, 136) == 512 * 192 * 2
    assert L.nf4s_packed_activation_bytes(1, 8) == 256 * 64 * 2
    for M, K in ((0, 64), (16, 0), (16, 12), (-1, 64)):
        assert L.nf4s_packed_activation_bytes(M, K) == 0


def test_pack_and_packed_call_errors():
    with pytest.raises(L.Nf4sError) as e:
        L.nf4s_pack_activation(FAKE, 16, 12, FAKE, 1 << 20)          # K not a multiple of 8
    assert e.value.code == L.ESHAPE
    with pytest.raises(L.Nf4sError) as e:
        L.nf4s_pack_activation(FAKE, 0, 64, FAKE, 1 << 20)
    assert e.value.code == L.ESHAPE
    with pytest.raises(L.Nf4sError) as e:
        L.nf4s_pack_activation(FAKE, 16, 64, FAKE + 16, 1 << 20)     # packed buffer 256-B aligned
    assert e.value.code == L.EALIGN
    with pytest.raises(L.Nf4sError) as e:
        L.nf4s_pack_activation(FAKE, 16, 64, FAKE, 1024)             # buffer too small
    assert e.value.code == L.EWORKSPACE
    d = _desc()
    with pytest.raises(L.Nf4sError) as e:
        L.streamed_linear_fwd_packed(FAKE, d, FAKE + 16, 16, FAKE, None, None, 0, 0.0, None, 0)
    assert e.value.code == L.EALIGN
    d.table_hash ^= 1
    with pytest.raises(L.Nf4sError) as e:
        L.streamed_linear_bwd_packed(FAKE, d, FAKE, 16, FAKE, None, None, 0, None, 0)
    assert e.value.code == L.ETABLE


def test_packed_workspace_is_split_partials_only():
    # the forward runs on 512 x 128 tiles where they fill the chip unsplit
    # (gate at M = 1024: 112 x 2 tiles), else on 256 x 128 tiles: gate at
    # M = 512 then has 112 x 2 tiles, again unsplit; no scratch either way
    assert L.nf4s_workspace_bytes(L.OP_LINEAR_FWD_PACKED, 1024, 14336, 4096) == 0
    assert L.nf4s_workspace_bytes(L.OP_LINEAR_FWD_PACKED, 512, 14336, 4096) == 0
    # q at M = 512: 32 x 2 tiles of 256 x 128, split in four
    need = L.nf4s_workspace_bytes(L.OP_LINEAR_FWD_PACKED, 512, 4096, 4096)
    assert need == 4 * 512 * 4096 * 4
    assert need > 0 and need % (512 * 4096 * 4) == 0
    full = L.nf4s_workspace_bytes(L.OP_LINEAR_FWD, 512, 4096, 4096)
    assert full == need + L.nf4s_packed_activation_bytes(512, 4096)
    # backward tiles are 256 x 128: dx of gate at M = 512 (32 x 2 tiles) splits
    assert L.nf4s_workspace_bytes(L.OP_LINEAR_BWD_PACKED, 512, 14336, 4096) > 0


def _err(fn, *args):
    with pytest.raises(L.Nf4sError) as e:
        fn(*args)
    return e.value.code


def test_decoder_argument_errors():
    """The decoder entry points validate on the host before any launch."""
    assert _err(L.nf4s_rope, None, 4, 2, 2, 16, 1e4, 0) == L.EINVAL
    assert _err(L.nf4s_rope, FAKE, 6, 4, 2, 16, 1e4, 0) == L.ESHAPE        # rows % seq
    assert _err(L.nf4s_rope, FAKE, 6, 3, 1, 25, 1e4, 0) == L.ESHAPE        # odd head size
    assert _err(L.nf4s_rope, FAKE, 6, 3, 1, 12, 1e4, 0) == L.ESHAPE        # not a multiple of 8
    assert _err(L.nf4s_rmsnorm_fwd, FAKE, FAKE, 4, 12, 1e-5, FAKE, FAKE) == L.ESHAPE  # width % 8
    assert _err(L.nf4s_rmsnorm_fwd, FAKE + 8, FAKE, 4, 16, 1e-5, FAKE, FAKE) == L.EALIGN
    assert _err(L.nf4s_rope, FAKE, 6, 3, 1, 16, 1.0, 0) == L.EINVAL        # theta
    assert _err(L.nf4s_rope, FAKE + 4, 6, 3, 1, 16, 1e4, 0) == L.EALIGN
    assert _err(L.nf4s_attention_fwd, FAKE, FAKE, FAKE, 1, 4, 3, 2, 16, FAKE, None, FAKE) == L.ESHAPE
    assert _err(L.nf4s_attention_fwd, FAKE, FAKE, FAKE, 0, 4, 4, 2, 16, FAKE, None, FAKE) == L.ESHAPE
    assert _err(L.nf4s_attention_fwd, FAKE, FAKE, FAKE, 1, 4, 4, 2, 16, FAKE, None, FAKE) == L.ESHAPE
    assert _err(L.nf4s_attention_bwd, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 4, 2, 32, FAKE, FAKE,
                FAKE, None, 0) == L.EWORKSPACE
    assert _err(L.nf4s_attention_bwd, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 4, 2, 32, FAKE, FAKE,
                FAKE, FAKE, 1 << 30, 0, FAKE + 16) == L.EALIGN                  # packed dv
    assert _err(L.nf4s_rmsnorm_bwd, [], FAKE, FAKE, FAKE, 4, 8, 0, FAKE) == L.EINVAL
    assert _err(L.nf4s_rmsnorm_bwd, [FAKE] * 4, FAKE, FAKE, FAKE, 4, 8, 0, FAKE) == L.EINVAL
    assert _err(L.nf4s_rmsnorm_bwd, [FAKE], FAKE, FAKE, FAKE, 4, 8, 2, FAKE) == L.EINVAL
    # a packed copy needs the bf16 one; both 16-byte aligned
    assert _err(L.nf4s_rmsnorm_bwd, [FAKE], FAKE, FAKE, FAKE, 4, 8, 0, FAKE, 0, None, FAKE) == L.EINVAL
    assert _err(L.nf4s_rmsnorm_bwd, [FAKE], FAKE, FAKE, FAKE, 4, 8, 0, FAKE, 0, FAKE + 2) == L.EALIGN
    assert _err(L.nf4s_rmsnorm_fwd, FAKE, FAKE, 4, 8, 0.0, FAKE, FAKE) == L.EINVAL   # eps
    assert _err(L.nf4s_rmsnorm_fwd, FAKE, FAKE, 0, 8, 1e-5, FAKE, FAKE) == L.ESHAPE
    assert _err(L.nf4s_adamw, FAKE, FAKE, FAKE, FAKE, 16, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0) == L.EINVAL
    assert _err(L.nf4s_adamw, FAKE, FAKE, FAKE, FAKE, 16, 1e-3, 1.0, 0.999, 1e-8, 0.0, 1) == L.EINVAL
    assert _err(L.nf4s_cross_entropy, FAKE, FAKE, 8, 100, FAKE, FAKE, FAKE, 4) == L.EWORKSPACE
    assert _err(L.nf4s_cross_entropy, FAKE, FAKE + 4, 8, 100, FAKE, FAKE, FAKE, 1 << 20) == L.EALIGN
    assert _err(L.nf4s_embed, FAKE, 0, 64, FAKE, 4, FAKE) == L.ESHAPE
    assert _err(L.nf4s_swiglu_fwd, FAKE, FAKE, 0, 8, FAKE) == L.ESHAPE
    assert _err(L.nf4s_swiglu_fwd, FAKE, FAKE, 4, 12, FAKE) == L.ESHAPE            # width % 8
    assert _err(L.nf4s_swiglu_fwd, FAKE, FAKE, 4, 16, FAKE, 0, FAKE + 16) == L.EALIGN  # packed 256-B
    assert _err(L.nf4s_swiglu_bwd, FAKE, FAKE, FAKE, 4, 16, FAKE, FAKE + 8) == L.EALIGN
    assert _err(L.nf4s_swiglu_bwd, FAKE, FAKE, FAKE, 4, 16, FAKE, FAKE, 0, None, FAKE + 64) == L.EALIGN
    # a row-major result may be NULL only when its packed form is asked for
    assert _err(L.nf4s_swiglu_bwd, FAKE, FAKE, FAKE, 4, 16, None, FAKE) == L.EINVAL
    assert _err(L.nf4s_swiglu_bwd, FAKE, FAKE, FAKE, 4, 16, FAKE, None, 0, FAKE, None) == L.EINVAL
    assert _err(L.nf4s_rmsnorm_fwd, FAKE, FAKE, 4, 16, 1e-5, FAKE, FAKE, 0, FAKE + 32) == L.EALIGN
    assert _err(L.nf4s_residual_add, FAKE, FAKE, 16, None) == L.EINVAL
    assert _err(L.nf4s_to_bf16, FAKE + 2, 2, 8, FAKE) == L.EALIGN
    assert _err(L.nf4s_to_bf16, FAKE, 2, 10, FAKE) == L.ESHAPE                     # width % 8
    assert _err(L.nf4s_to_bf16, FAKE, 2, 8, FAKE, 0, FAKE + 128) == L.EALIGN
    # the dense (lm_head) GEMM: whole 64-blocks along k_in, split partials required
    assert _err(L.dense_linear_fwd_packed, FAKE, 256, 100, FAKE, 16, FAKE, None, 0) == L.ESHAPE
    need = L.nf4s_workspace_bytes(L.OP_DENSE_BWD_PACKED, 512, 128256, 4096)
    assert need > 0
    assert _err(L.dense_linear_bwd_packed, FAKE, 128256, 4096, FAKE, 512, FAKE, None, 0) == L.EWORKSPACE


def test_decoder_workspace_sizes():
    assert L.nf4s_workspace_bytes(L.OP_ATTENTION_BWD, 512, 32, 128) == 512 * 32 * 4 * (1 + 2 * 128)
    assert L.nf4s_workspace_bytes(L.OP_CROSS_ENTROPY, 512, 0, 0) == 512 * 4
    assert L.nf4s_workspace_bytes(L.OP_DENSE_FWD_PACKED, 512, 128256, 4096) == 0   # 2004 tiles
    with pytest.raises(L.Nf4sError):
        L.nf4s_workspace_bytes(L.OP_ATTENTION_BWD, 0, 32, 128)
    with pytest.raises(L.Nf4sError):
        L.nf4s_workspace_bytes(L.OP_ATTENTION_BWD, 512, 32, 16)


def test_grouped_forward_workspace():
    # q, k, v of the 8B layer at M = 512: 48 x 2 tiles of 256 x 128 (512-row
    # tiles would need a split), the contraction split in two, partials for
    # all three outputs
    assert L.grouped_workspace_bytes([4096, 1024, 1024], 4096, 512) == 2 * 512 * 6144 * 4
    # gate and up: 224 tiles of 512 x 128 fill the chip, no split, no scratch
    assert L.grouped_workspace_bytes([14336, 14336], 4096, 512) == 0
    # a group of one plans like the single call
    assert L.grouped_workspace_bytes([4096], 4096, 512) == \
        L.nf4s_workspace_bytes(L.OP_LINEAR_FWD_PACKED, 512, 4096, 4096)
    assert _err(L.grouped_workspace_bytes, [64] * 4, 64, 16) == L.EINVAL
    assert _err(L.grouped_workspace_bytes, [], 64, 16) == L.EINVAL
    assert _err(L.grouped_workspace_bytes, [64, 60], 64, 16) == L.ESHAPE
    assert _err(L.grouped_workspace_bytes, [64, 64], 64, 0) == L.ESHAPE


def test_forward_plans():
    """Which forward kernel a shape runs on: 512 x 128 tiles where they fill
    the chip unsplit (gate + up of the 8B layer at 512 rows: 224 tiles), else
    256 x 128 tiles, split while the grid is short of the CUs."""
    g8, k8 = [14336, 14336], 4096
    assert L.linear_fwd_plan(g8, k8, 512) == (512, 128, 1)
    assert L.linear_fwd_plan(g8, k8, 2048) == (512, 128, 1)
    assert L.linear_fwd_plan(g8, k8, 512, swiglu=True) == (512, 128, 1)
    assert L.linear_fwd_plan([14336], k8, 512) == (256, 128, 1)      # 112 tiles of 512 would split
    assert L.linear_fwd_plan([4096, 1024, 1024], k8, 512) == (256, 128, 2)
    assert L.linear_fwd_plan([4096, 1024, 1024], k8, 2048) == (512, 128, 1)
    assert L.linear_fwd_plan([4096], 14336, 512) == (256, 128, 4)
    assert L.linear_fwd_plan([576, 200, 136], 576, 700) == (512, 128, 1)  # 9 steps: never split
    assert _err(L.linear_fwd_plan, [14336, 1024], k8, 512, True) == L.EINVAL
    assert _err(L.linear_fwd_plan, [4096, 4096], k8, 512, True) == L.ESHAPE   # would split
    assert _err(L.linear_fwd_plan, [64] * 4, 64, 16) == L.EINVAL
    assert _err(L.linear_fwd_plan, [64, 60], 64, 16) == L.ESHAPE


def test_grouped_forward_argument_errors():
    d = [L.nf4s_tensor_layout(64, 128, 0)]
    d.append(L.nf4s_tensor_layout(32, 128, d[0].end))
    fwd = L.streamed_linear_fwd_grouped
    ys = [FAKE, FAKE]
    # only error paths: every call below is refused before any launch
    assert _err(fwd, FAKE, [d[0]] * 4, FAKE, 16, [FAKE] * 4, None, None, 0, 0.0, None, 0) == L.EINVAL
    other = L.nf4s_tensor_layout(64, 64, d[1].end)
    assert _err(fwd, FAKE, [d[0], other], FAKE, 16, ys, None, None, 0, 0.0, None, 0) == L.ESHAPE
    assert _err(fwd, FAKE, d, FAKE, 16, ys, [FAKE, None], [None, None], 16, 2.0, None, 0) == L.EINVAL
    assert _err(fwd, FAKE, d, FAKE, 16, ys, [FAKE, None], [FAKE, None], 0, 2.0, None, 0) == L.EINVAL
    assert _err(fwd, FAKE, d, FAKE + 16, 16, ys, None, None, 0, 0.0, None, 0) == L.EALIGN
    assert _err(fwd, FAKE, d, FAKE, 16, [FAKE, FAKE + 2], None, None, 0, 0.0, None, 0) == L.EALIGN
    assert _err(fwd, FAKE, d, FAKE, 0, ys, None, None, 0, 0.0, None, 0) == L.ESHAPE
    bad = L.nf4s_tensor_layout(32, 128, d[0].end)
    bad.table_hash ^= 1
    assert _err(fwd, FAKE, [d[0], bad], FAKE, 16, ys, None, None, 0, 0.0, None, 0) == L.ETABLE
    # q, k, v at 8B widths and M = 512 split the contraction: workspace required
    q = [L.nf4s_tensor_layout(4096, 4096, 0)]
    q.append(L.nf4s_tensor_layout(1024, 4096, q[0].end))
    q.append(L.nf4s_tensor_layout(1024, 4096, q[1].end))
    assert _err(fwd, FAKE, q, FAKE, 512, [FAKE] * 3, None, None, 0, 0.0, FAKE, 1024) == L.EWORKSPACE


def test_grouped_lora_workspace():
    ns, k, M = [4096, 1024], 4096, 512
    single_f = sum(L.nf4s_workspace_bytes(L.OP_LORA_FWD, M, n, k) for n in ns)
    single_b = sum(L.nf4s_workspace_bytes(L.OP_LORA_BWD, M, n, k) for n in ns)
    assert L.lora_grouped_workspace_bytes(ns, k, M, False) == single_f
    assert L.lora_grouped_workspace_bytes(ns, k, M, True) == single_b
    # backward partials: ceil(n_out / 512) chunks of M x 64 fp32 per adapter
    assert single_b == (8 + 2) * M * 64 * 4
    assert _err(L.lora_grouped_workspace_bytes, [64] * 4, 64, 16, True) == L.EINVAL
    assert _err(L.lora_grouped_workspace_bytes, [], 64, 16, True) == L.EINVAL
    assert _err(L.lora_grouped_workspace_bytes, [64, 60], 64, 16, True) == L.ESHAPE
    assert _err(L.lora_grouped_workspace_bytes, [64], 100, 16, False) == L.ESHAPE
    assert _err(L.lora_grouped_workspace_bytes, [64], 64, 0, False) == L.ESHAPE


def test_grouped_lora_argument_errors():
    # only error paths: every call below is refused before any launch
    fwd, bwd = L.lora_fwd_grouped, L.lora_bwd_grouped
    two = [FAKE, FAKE]
    assert _err(fwd, FAKE, 16, 64, [FAKE] * 4, 16, [FAKE] * 4, FAKE, 1 << 30) == L.EINVAL
    assert _err(fwd, FAKE, 16, 100, two, 16, two, FAKE, 1 << 30) == L.ESHAPE
    assert _err(fwd, FAKE, 0, 64, two, 16, two, FAKE, 1 << 30) == L.ESHAPE
    assert _err(fwd, FAKE, 16, 64, two, 65, two, FAKE, 1 << 30) == L.EINVAL
    assert _err(fwd, FAKE, 16, 64, [FAKE, FAKE + 2], 16, two, FAKE, 1 << 30) == L.EALIGN
    assert _err(fwd, FAKE, 16, 64, two, 16, [FAKE, None], FAKE, 1 << 30) == L.EINVAL
    assert _err(fwd, FAKE, 16, 64, two, 16, two, FAKE, 16) == L.EWORKSPACE
    ok = dict(x=FAKE, dys=two, us=two, M=16, k_in=64, n_outs=[64, 128], Bs=two, r=16, scale=2.0,
              dAs=two, dBs=two, du_outs=two, accumulate=0, ws=FAKE, ws_bytes=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return _err(bwd, a["x"], a["dys"], a["us"], a["M"], a["k_in"], a["n_outs"], a["Bs"], a["r"],
                    a["scale"], a["dAs"], a["dBs"], a["du_outs"], a["accumulate"], a["ws"],
                    a["ws_bytes"])
    assert call(n_outs=[64, 60]) == L.ESHAPE
    assert call(accumulate=2) == L.EINVAL
    assert call(scale=float("nan")) == L.EINVAL
    assert call(dys=[FAKE, FAKE + 8]) == L.EALIGN
    assert call(dBs=[FAKE, FAKE + 2]) == L.EALIGN
    assert call(du_outs=[None, FAKE]) == L.EINVAL
    assert call(ws_bytes=64) == L.EWORKSPACE


def test_grouped_backward_workspace():
    # q, k, v of the 8B layer at M = 512: 64 tiles of 256 x 128; q's 64 steps
    # in two splits, k and v one each: 256 workgroups of at most 32 steps,
    # four fp32 partials of 512 x 4096
    assert L.grouped_bwd_workspace_bytes([4096, 1024, 1024], 4096, 512) == 4 * 512 * 4096 * 4
    # gate and up: 224 steps each on 32 tiles of 512 x 128, four splits of
    # 56 steps each: eight partials
    assert L.grouped_bwd_workspace_bytes([14336, 14336], 4096, 512) == 8 * 512 * 4096 * 4
    # at M = 2048: 128 tiles of 512 x 128, one split each
    assert L.grouped_bwd_workspace_bytes([14336, 14336], 4096, 2048) == 2 * 2048 * 4096 * 4
    # a group of one plans like the single call
    for n, k, M in ((4096, 4096, 512), (40, 64, 100), (14336, 4096, 2048)):
        assert L.grouped_bwd_workspace_bytes([n], k, M) == \
            L.nf4s_workspace_bytes(L.OP_LINEAR_BWD_PACKED, M, n, k)
    assert _err(L.grouped_bwd_workspace_bytes, [64] * 4, 64, 16) == L.EINVAL
    assert _err(L.grouped_bwd_workspace_bytes, [], 64, 16) == L.EINVAL
    assert _err(L.grouped_bwd_workspace_bytes, [64, 72], 64, 16) == L.ESHAPE
    assert _err(L.grouped_bwd_workspace_bytes, [64, 64], 100, 16) == L.ESHAPE
    assert _err(L.grouped_bwd_workspace_bytes, [64, 64], 64, 0) == L.ESHAPE


def test_grouped_backward_argument_errors():
    d = [L.nf4s_tensor_layout(64, 128, 0)]
    d.append(L.nf4s_tensor_layout(128, 128, d[0].end))
    bwd = L.streamed_linear_bwd_grouped
    two = [FAKE, FAKE]
    # only error paths: every call below is refused before any launch
    assert _err(bwd, FAKE, [d[0]] * 4, [FAKE] * 4, 16, FAKE, None, None, 0, None, 0) == L.EINVAL
    other = L.nf4s_tensor_layout(64, 64, d[1].end)
    assert _err(bwd, FAKE, [d[0], other], two, 16, FAKE, None, None, 0, None, 0) == L.ESHAPE
    odd = L.nf4s_tensor_layout(72, 128, d[1].end)
    assert _err(bwd, FAKE, [d[0], odd], two, 16, FAKE, None, None, 0, None, 0) == L.ESHAPE
    assert _err(bwd, FAKE, d, [FAKE, FAKE + 16], 16, FAKE, None, None, 0, None, 0) == L.EALIGN
    assert _err(bwd, FAKE, d, two, 16, FAKE + 2, None, None, 0, None, 0) == L.EALIGN
    assert _err(bwd, FAKE, d, two, 16, FAKE, [FAKE, None], [None, None], 16, None, 0) == L.EINVAL
    assert _err(bwd, FAKE, d, two, 16, FAKE, [FAKE, None], [FAKE, None], 0, None, 0) == L.EINVAL
    assert _err(bwd, FAKE, d, two, 0, FAKE, None, None, 0, None, 0) == L.ESHAPE
    bad = L.nf4s_tensor_layout(128, 128, d[0].end)
    bad.table_hash ^= 1
    assert _err(bwd, FAKE, [d[0], bad], two, 16, FAKE, None, None, 0, None, 0) == L.ETABLE
    q = [L.nf4s_tensor_layout(4096, 4096, 0)]
    q.append(L.nf4s_tensor_layout(1024, 4096, q[0].end))
    assert _err(bwd, FAKE, q, two, 512, FAKE, None, None, 0, FAKE, 1024) == L.EWORKSPACE


def test_residual_forward_argument_errors():
    d = L.nf4s_tensor_layout(64, 128, 0)
    f = L.streamed_linear_fwd_residual
    # only error paths: every call below is refused before any launch
    assert _err(f, FAKE, d, FAKE, 16, FAKE, None, None, 0, 0.0, None, FAKE, None, 0) == L.EINVAL
    assert _err(f, FAKE, d, FAKE, 16, FAKE, None, None, 0, 0.0, FAKE, FAKE + 4, None, 0) == L.EALIGN
    assert _err(f, FAKE, d, FAKE + 16, 16, FAKE, None, None, 0, 0.0, FAKE, FAKE, None, 0) == L.EALIGN
    assert _err(f, FAKE, d, FAKE, 16, FAKE, FAKE, None, 16, 2.0, FAKE, FAKE, None, 0) == L.EINVAL
    assert _err(f, FAKE, d, FAKE, 0, FAKE, None, None, 0, 0.0, FAKE, FAKE, None, 0) == L.ESHAPE
    o = L.nf4s_tensor_layout(4096, 4096, 0)
    assert _err(f, FAKE, o, FAKE, 512, FAKE, None, None, 0, 0.0, FAKE, FAKE, FAKE, 64) == L.EWORKSPACE


def test_rope_pair_argument_errors():
    f = L.nf4s_rope_pair
    assert _err(f, FAKE, 4, FAKE, 2, 8, 4, 32, 1.0, 0) == L.EINVAL        # theta
    assert _err(f, FAKE, 4, FAKE, 2, 8, 3, 32, 1e4, 0) == L.ESHAPE        # rows % seq
    assert _err(f, FAKE, 4, FAKE, 0, 8, 4, 32, 1e4, 0) == L.ESHAPE        # heads
    assert _err(f, FAKE, 4, FAKE + 2, 2, 8, 4, 32, 1e4, 0) == L.EALIGN
    assert _err(f, FAKE, 4, None, 2, 8, 4, 32, 1e4, 0) == L.EINVAL
    assert _err(f, FAKE, 4, FAKE, 2, 8, 4, 32, 1e4, 2) == L.EINVAL        # inverse
    assert _err(f, FAKE, 4, FAKE, 2, 8, 4, 32, 1e4, 0, 0, FAKE + 64) == L.EALIGN   # packed copy
    assert _err(f, FAKE, 4, FAKE, 2, 8, 4, 32, 1e4, 0, 0, None, FAKE + 8) == L.EALIGN


def test_fused_swiglu_refuses_split_shapes_and_bad_arguments():
    # q-sized weights at M = 512: 64 tiles of 512 rows, the contraction would be split
    assert not L.nf4s_swiglu_fused_supported(512, 4096, 4096)
    assert L.nf4s_swiglu_fused_supported(512, 14336, 4096)
    assert not L.nf4s_swiglu_fused_supported(512, 14336 + 8, 4096)   # not whole 64-column tiles
    d0 = L.nf4s_tensor_layout(4096, 4096)
    d1 = L.nf4s_tensor_layout(4096, 4096, d0.end)
    with pytest.raises(L.Nf4sError) as e:
        L.streamed_linear_fwd_swiglu(FAKE, d0, d1, FAKE, 512, FAKE, None, 0, None, None, 0, 0.0)
    assert e.value.code == L.ESHAPE
    g0 = L.nf4s_tensor_layout(14336, 4096)
    g1 = L.nf4s_tensor_layout(14336, 4096, g0.end)
    with pytest.raises(L.Nf4sError) as e:                               # no output at all
        L.streamed_linear_fwd_swiglu(FAKE, g0, g1, FAKE, 512, None, None, 0, None, None, 0, 0.0)
    assert e.value.code == L.EINVAL
    with pytest.raises(L.Nf4sError) as e:                               # packed output too small
        L.streamed_linear_fwd_swiglu(FAKE, g0, g1, FAKE, 512, None, FAKE, 1024, None, None, 0, 0.0)
    assert e.value.code == L.EWORKSPACE
    with pytest.raises(L.Nf4sError) as e:                               # gate and up differ
        L.streamed_linear_fwd_swiglu(FAKE, g0, d1, FAKE, 512, FAKE, None, 0, None, None, 0, 0.0)
    assert e.value.code == L.ESHAPE
