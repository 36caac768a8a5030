"""Python binding of libnf4stream (the layer-streamed NF4 + LoRA hot path).

Argument marshalling only: every function forwards to the C ABI declared in
include/nf4stream.h with the same name, raises Nf4sError on a negative status,
and computes nothing itself. Device pointers and streams are plain integers
(``tensor.data_ptr()``, ``torch.cuda.Stream().cuda_stream``). There is no
fallback: if the HIP library is missing, importing a function that needs it
raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf4stream.so")

OK, EINVAL, ESHAPE, EALIGN, ETABLE, EKEY, ESLOT, ENOTPINNED, EHIP, EWORKSPACE = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9)
DTYPE_F32, DTYPE_BF16 = 0, 1
OP_QUANTIZE, OP_LINEAR_FWD, OP_LINEAR_BWD, OP_LORA_BWD, OP_LORA_FWD = 1, 2, 3, 4, 5
OP_LINEAR_FWD_PACKED, OP_LINEAR_BWD_PACKED = 6, 7
OP_DENSE_FWD_PACKED, OP_DENSE_BWD_PACKED, OP_ATTENTION_BWD, OP_CROSS_ENTROPY = 8, 9, 10, 11
METHOD_NF4 = 1

EXPORTS = (
    "nf4s_version", "nf4s_last_error", "nf4_shard_bytes", "nf4s_tensor_layout",
    "nf4_code_tables", "nf4s_table_hash", "nf4s_workspace_bytes", "nf4_quantize_shard",
    "nf4_dequant", "streamed_linear_fwd", "streamed_linear_bwd", "lora_fwd", "lora_bwd",
    "layer_prefetch", "nf4s_event_create", "nf4s_event_destroy", "nf4s_event_record",
    "nf4s_stream_wait_event", "nf4s_pool_create", "nf4s_pool_destroy", "nf4s_pool_set_layer",
    "nf4s_pool_prefetch", "nf4s_pool_acquire", "nf4s_pool_release", "nf4s_pool_stats",
    "nf4s_pool_set_debug", "streamed_linear_fwd_noalloc", "nf4s_swiglu_fused_supported",
    "streamed_linear_fwd_swiglu", "nf4s_packed_activation_bytes", "nf4s_pack_activation", "streamed_linear_fwd_packed",
    "streamed_linear_bwd_packed", "dense_linear_fwd_packed", "dense_linear_bwd_packed",
    "nf4s_grouped_workspace_bytes", "streamed_linear_fwd_grouped", "nf4s_linear_fwd_plan",
    "nf4s_lora_grouped_workspace_bytes", "lora_fwd_grouped", "lora_bwd_grouped",
    "nf4s_grouped_bwd_workspace_bytes", "streamed_linear_bwd_grouped", "streamed_linear_fwd_residual",
    "nf4s_rope_pair",
    "nf4s_embed", "nf4s_rmsnorm_fwd", "nf4s_rmsnorm_bwd", "nf4s_rope", "nf4s_attention_fwd",
    "nf4s_attention_bwd", "nf4s_swiglu_fwd", "nf4s_swiglu_bwd", "nf4s_residual_add",
    "nf4s_to_bf16", "nf4s_cross_entropy", "nf4s_adamw", "nf4s_token_nll", "nf4s_dpo_loss",
    "nf4s_logit_grad",
)


class Nf4sError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"nf4stream error {code}: {msg}")
        self.code = code


class TensorDesc(ctypes.Structure):
    _fields_ = [
        ("n_out", ctypes.c_int64), ("k_in", ctypes.c_int64),
        ("method", ctypes.c_int32), ("blocksize", ctypes.c_int32),
        ("nested_block", ctypes.c_int32), ("double_quant", ctypes.c_int32),
        ("off_packed", ctypes.c_uint64), ("off_q8", ctypes.c_uint64),
        ("off_nested", ctypes.c_uint64), ("off_offset", ctypes.c_uint64),
        ("end", ctypes.c_uint64), ("table_hash", ctypes.c_uint64),
    ]

    def copy(self):
        d = TensorDesc()
        ctypes.pointer(d)[0] = self
        return d


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIG = {
    "nf4s_version": (ctypes.c_char_p, []),
    "nf4s_last_error": (ctypes.c_char_p, []),
    "nf4_shard_bytes": (ctypes.c_uint64, [_I64, _I64]),
    "nf4s_tensor_layout": (ctypes.c_int, [_I64, _I64, ctypes.c_uint64, ctypes.POINTER(TensorDesc)]),
    "nf4_code_tables": (ctypes.c_int, [_P, _P]),
    "nf4s_table_hash": (ctypes.c_uint64, []),
    "nf4s_workspace_bytes": (ctypes.c_int, [ctypes.c_int, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)]),
    "nf4_quantize_shard": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _P, ctypes.POINTER(TensorDesc),
                                          _P, _P, ctypes.c_size_t, _P]),
    "nf4_dequant": (ctypes.c_int, [_P, ctypes.POINTER(TensorDesc), _P, _P]),
    "streamed_linear_fwd": (ctypes.c_int, [_P, ctypes.POINTER(TensorDesc), _P, _I64, _P, _P, _P,
                                           ctypes.c_int, ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "streamed_linear_bwd": (ctypes.c_int, [_P, ctypes.POINTER(TensorDesc), _P, _I64, _P, _P, _P,
                                           ctypes.c_int, _P, ctypes.c_size_t, _P]),
    "nf4s_swiglu_fused_supported": (ctypes.c_int, [_I64, _I64, _I64]),
    "streamed_linear_fwd_swiglu": (ctypes.c_int, [_P, ctypes.POINTER(TensorDesc), ctypes.POINTER(TensorDesc),
                                                  _P, _I64, _P, _P, ctypes.c_size_t, _P, _P, ctypes.c_int,
                                                  ctypes.c_float, _P]),
    "streamed_linear_fwd_noalloc": (ctypes.c_int, [_P, ctypes.POINTER(TensorDesc), _P, _I64, _P, _P, _P,
                                                   ctypes.c_int, ctypes.c_float, _P]),
    "lora_fwd": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.c_int, _P, _P, ctypes.c_size_t, _P]),
    "lora_bwd": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int, ctypes.c_float,
                                _P, _P, _P, ctypes.c_int, _P, ctypes.c_size_t, _P]),
    "layer_prefetch": (ctypes.c_int, [_P, ctypes.c_size_t, _P, ctypes.c_size_t, _P, _P, _P]),
    "nf4s_event_create": (ctypes.c_int, [ctypes.POINTER(_P)]),
    "nf4s_event_destroy": (ctypes.c_int, [_P]),
    "nf4s_event_record": (ctypes.c_int, [_P, _P]),
    "nf4s_stream_wait_event": (ctypes.c_int, [_P, _P]),
    "nf4s_pool_create": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(_P), ctypes.c_size_t, _P, _P,
                                        ctypes.POINTER(_P)]),
    "nf4s_pool_destroy": (ctypes.c_int, [_P]),
    "nf4s_pool_set_layer": (ctypes.c_int, [_P, ctypes.c_int, _P, ctypes.c_size_t]),
    "nf4s_pool_prefetch": (ctypes.c_int, [_P, ctypes.c_int]),
    "nf4s_pool_acquire": (ctypes.c_int, [_P, ctypes.c_int, ctypes.POINTER(_P)]),
    "nf4s_pool_release": (ctypes.c_int, [_P, ctypes.c_int]),
    "nf4s_pool_stats": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)]),
    "nf4s_pool_set_debug": (ctypes.c_int, [_P, ctypes.c_int]),
    "nf4s_packed_activation_bytes": (ctypes.c_uint64, [_I64, _I64]),
    "nf4s_pack_activation": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "streamed_linear_fwd_packed": (ctypes.c_int, [_P, ctypes.POINTER(TensorDesc), _P, _I64, _P, _P,
                                                  _P, ctypes.c_int, ctypes.c_float, _P,
                                                  ctypes.c_size_t, _P]),
    "streamed_linear_bwd_packed": (ctypes.c_int, [_P, ctypes.POINTER(TensorDesc), _P, _I64, _P, _P,
                                                  _P, ctypes.c_int, _P, ctypes.c_size_t, _P]),
    "nf4s_grouped_workspace_bytes": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P]),
    "nf4s_linear_fwd_plan": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, ctypes.c_int, _P, _P, _P]),
    "streamed_linear_fwd_grouped": (ctypes.c_int, [_P, ctypes.POINTER(TensorDesc), ctypes.c_int, _P,
                                                   _I64, _P, _P, _P, ctypes.c_int, ctypes.c_float,
                                                   _P, ctypes.c_size_t, _P]),
    "nf4s_rope_pair": (ctypes.c_int, [_P, ctypes.c_int, _P, ctypes.c_int, _I64, _I64, ctypes.c_int,
                                      ctypes.c_double, ctypes.c_int, _P, _P, _P]),
    "streamed_linear_fwd_residual": (ctypes.c_int, [_P, ctypes.POINTER(TensorDesc), _P, _I64, _P, _P, _P,
                                                    ctypes.c_int, ctypes.c_float, _P, _P, _P,
                                                    ctypes.c_size_t, _P]),
    "nf4s_grouped_bwd_workspace_bytes": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P]),
    "streamed_linear_bwd_grouped": (ctypes.c_int, [_P, ctypes.POINTER(TensorDesc), ctypes.c_int, _P,
                                                   _I64, _P, _P, _P, ctypes.c_int, _P,
                                                   ctypes.c_size_t, _P]),
    "nf4s_lora_grouped_workspace_bytes": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, ctypes.c_int,
                                                         _P]),
    "lora_fwd_grouped": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.c_int, ctypes.c_int, _P, _P,
                                        ctypes.c_size_t, _P]),
    "lora_bwd_grouped": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_float, _P, _P, _P, ctypes.c_int, _P, ctypes.c_size_t,
                                        _P]),
    "dense_linear_fwd_packed": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P, ctypes.c_size_t, _P]),
    "dense_linear_bwd_packed": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P, ctypes.c_size_t, _P]),
    "nf4s_embed": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P]),
    "nf4s_rmsnorm_fwd": (ctypes.c_int, [_P, _P, _I64, _I64, ctypes.c_float, _P, _P, _P, _P]),
    "nf4s_rmsnorm_bwd": (ctypes.c_int, [ctypes.POINTER(_P), ctypes.c_int, _P, _P, _P, _I64, _I64,
                                        ctypes.c_int, _P, _P, _P, _P]),
    "nf4s_rope": (ctypes.c_int, [_P, _I64, _I64, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                 ctypes.c_int, _P]),
    "nf4s_attention_fwd": (ctypes.c_int, [_P, _P, _P, _I64, _I64, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, _P, _P, _P, _P, _P]),
    "nf4s_attention_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "nf4s_swiglu_fwd": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P]),
    "nf4s_swiglu_bwd": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P, _P, _P, _P]),
    "nf4s_residual_add": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
    "nf4s_to_bf16": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "nf4s_cross_entropy": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P, ctypes.c_size_t, _P]),
    "nf4s_adamw": (ctypes.c_int, [_P, _P, _P, _P, _I64, ctypes.c_float, ctypes.c_float,
                                  ctypes.c_float, ctypes.c_float, ctypes.c_float, _I64, _P]),
    "nf4s_token_nll": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P]),
    "nf4s_dpo_loss": (ctypes.c_int, [_P, _P, _P, _I64, _I64, ctypes.c_float, _P, _P, _P]),
    "nf4s_logit_grad": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]),
}


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m layer_streamed_nf4_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc != OK:
        raise Nf4sError(rc, lib().nf4s_last_error().decode())
    return rc


def nf4s_version() -> str:
    return lib().nf4s_version().decode()


def nf4_shard_bytes(n_out: int, k_in: int) -> int:
    return int(lib().nf4_shard_bytes(n_out, k_in))


def nf4s_tensor_layout(n_out: int, k_in: int, base: int = 0) -> TensorDesc:
    d = TensorDesc()
    _check(lib().nf4s_tensor_layout(n_out, k_in, base, ctypes.byref(d)))
    return d


def nf4_code_tables():
    c4 = np.zeros(16, np.float32)
    c8 = np.zeros(256, np.float32)
    _check(lib().nf4_code_tables(c4.ctypes.data, c8.ctypes.data))
    return c4, c8


def nf4s_table_hash() -> int:
    return int(lib().nf4s_table_hash())


def nf4s_workspace_bytes(op: int, M: int, n_out: int, k_in: int) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().nf4s_workspace_bytes(op, M, n_out, k_in, ctypes.byref(b)))
    return int(b.value)


def nf4_quantize_shard(w, dtype, n_out, k_in, shard, desc, status, ws, ws_bytes, stream=0):
    _check(lib().nf4_quantize_shard(w, dtype, n_out, k_in, shard, ctypes.byref(desc), status, ws,
                                    ws_bytes, stream))


def nf4_dequant(shard, desc, w_bf16, stream=0):
    _check(lib().nf4_dequant(shard, ctypes.byref(desc), w_bf16, stream))


def streamed_linear_fwd(shard, desc, x, M, y, lora_u, lora_B, r, scale, ws, ws_bytes, stream=0):
    _check(lib().streamed_linear_fwd(shard, ctypes.byref(desc), x, M, y, lora_u, lora_B, r, scale,
                                     ws, ws_bytes, stream))


NOALLOC_SCRATCH_BYTES = 64 << 20


def streamed_linear_fwd_noalloc(shard, desc, x, M, y, lora_u, lora_B, r, scale, stream=0):
    _check(lib().streamed_linear_fwd_noalloc(shard, ctypes.byref(desc), x, M, y, lora_u, lora_B, r,
                                             scale, stream))


def streamed_linear_bwd(shard, desc, dy, M, dx, lora_du, lora_A, r, ws, ws_bytes, stream=0):
    _check(lib().streamed_linear_bwd(shard, ctypes.byref(desc), dy, M, dx, lora_du, lora_A, r, ws,
                                     ws_bytes, stream))


def nf4s_packed_activation_bytes(M, K):
    return int(lib().nf4s_packed_activation_bytes(M, K))


def nf4s_pack_activation(a, M, K, packed, packed_bytes, stream=0):
    _check(lib().nf4s_pack_activation(a, M, K, packed, packed_bytes, stream))


def streamed_linear_fwd_packed(shard, desc, x_packed, M, y, lora_u, lora_B, r, scale, ws, ws_bytes,
                               stream=0):
    _check(lib().streamed_linear_fwd_packed(shard, ctypes.byref(desc), x_packed, M, y, lora_u, lora_B,
                                            r, scale, ws, ws_bytes, stream))


def streamed_linear_bwd_packed(shard, desc, dy_packed, M, dx, lora_du, lora_A, r, ws, ws_bytes,
                               stream=0):
    _check(lib().streamed_linear_bwd_packed(shard, ctypes.byref(desc), dy_packed, M, dx, lora_du,
                                            lora_A, r, ws, ws_bytes, stream))


def grouped_workspace_bytes(n_outs, k_in, M):
    """Workspace of streamed_linear_fwd_grouped for weights of n_outs outputs."""
    arr = (ctypes.c_int64 * len(n_outs))(*n_outs)
    out = ctypes.c_size_t()
    _check(lib().nf4s_grouped_workspace_bytes(len(n_outs), ctypes.cast(arr, ctypes.c_void_p), k_in, M,
                                              ctypes.byref(out)))
    return out.value


def linear_fwd_plan(n_outs, k_in, M, swiglu=False):
    """(tile rows, tile columns, splits) of the forward launch for these shapes."""
    arr = (ctypes.c_int64 * len(n_outs))(*n_outs)
    v = [ctypes.c_int() for _ in range(3)]
    _check(lib().nf4s_linear_fwd_plan(len(n_outs), ctypes.cast(arr, ctypes.c_void_p), k_in, M, int(swiglu),
                                      *(ctypes.byref(x) for x in v)))
    return tuple(x.value for x in v)


def _ptr_array(ptrs):
    if ptrs is None:
        return None
    return ctypes.cast((ctypes.c_void_p * len(ptrs))(*[p or None for p in ptrs]), ctypes.c_void_p)


def streamed_linear_fwd_grouped(shard, descs, x_packed, M, ys, lora_us, lora_Bs, r, scale, ws,
                                ws_bytes, stream=0):
    """One launch of the forward of len(descs) weights reading x_packed.

    descs: TensorDesc list; ys: device pointers; lora_us / lora_Bs: None or
    lists of device pointers (None entries: no adapter on that weight).
    """
    n = len(descs)
    darr = (TensorDesc * n)(*descs)
    _check(lib().streamed_linear_fwd_grouped(shard, darr, n, x_packed, M, _ptr_array(ys),
                                             _ptr_array(lora_us), _ptr_array(lora_Bs), r, scale, ws,
                                             ws_bytes, stream))


def nf4s_swiglu_fused_supported(M, width, k_in) -> bool:
    return bool(lib().nf4s_swiglu_fused_supported(M, width, k_in))


def streamed_linear_fwd_swiglu(shard, d_gate, d_up, x_packed, M, out, out_packed, out_packed_bytes,
                               lora_us, lora_Bs, r, scale, stream=0):
    """out (and/or out_packed) = bf16(silu(g) * u) of the gate and up projections."""
    _check(lib().streamed_linear_fwd_swiglu(shard, ctypes.byref(d_gate), ctypes.byref(d_up), x_packed, M,
                                            out, out_packed, out_packed_bytes, _ptr_array(lora_us),
                                            _ptr_array(lora_Bs), r, scale, stream))


def streamed_linear_fwd_residual(shard, desc, x_packed, M, y, lora_u, lora_B, r, scale, h_in, h_out, ws,
                                 ws_bytes, stream=0):
    """y = the forward of desc on x_packed (bf16) and h_out = h_in + y (fp32)."""
    _check(lib().streamed_linear_fwd_residual(shard, ctypes.byref(desc), x_packed, M, y, lora_u, lora_B,
                                              r, scale, h_in, h_out, ws, ws_bytes, stream))


def grouped_bwd_workspace_bytes(n_outs, k_in, M):
    """Workspace of streamed_linear_bwd_grouped for weights of n_outs outputs."""
    arr = (ctypes.c_int64 * len(n_outs))(*n_outs)
    out = ctypes.c_size_t()
    _check(lib().nf4s_grouped_bwd_workspace_bytes(len(n_outs), ctypes.cast(arr, ctypes.c_void_p), k_in,
                                                  M, ctypes.byref(out)))
    return out.value


def streamed_linear_bwd_grouped(shard, descs, dy_packed, M, dx, lora_dus, lora_As, r, ws, ws_bytes,
                                stream=0):
    """dx = sum of the backward of len(descs) weights (one launch).

    dy_packed: device pointers of the packed dy_i; lora_dus / lora_As: None or
    lists of device pointers (None entries: no adapter on that weight).
    """
    n = len(descs)
    darr = (TensorDesc * n)(*descs)
    _check(lib().streamed_linear_bwd_grouped(shard, darr, n, _ptr_array(dy_packed), M, dx,
                                             _ptr_array(lora_dus), _ptr_array(lora_As), r, ws,
                                             ws_bytes, stream))


def dense_linear_fwd_packed(w, n_out, k_in, x_packed, M, y, ws, ws_bytes, stream=0):
    _check(lib().dense_linear_fwd_packed(w, n_out, k_in, x_packed, M, y, ws, ws_bytes, stream))


def dense_linear_bwd_packed(w, n_out, k_in, dy_packed, M, dx, ws, ws_bytes, stream=0):
    _check(lib().dense_linear_bwd_packed(w, n_out, k_in, dy_packed, M, dx, ws, ws_bytes, stream))


def nf4s_embed(table, vocab, hidden, ids, T, h, stream=0):
    _check(lib().nf4s_embed(table, vocab, hidden, ids, T, h, stream))


def nf4s_rmsnorm_fwd(x, w, T, H, eps, y, rstd, stream=0, packed=None):
    _check(lib().nf4s_rmsnorm_fwd(x, w, T, H, eps, y, rstd, packed, stream))


def nf4s_rmsnorm_bwd(dys, x, w, rstd, T, H, accumulate, dh, stream=0, y=None, packed=None):
    """dys: a sequence of 1..3 device pointers (bf16 [T, H] gradients);
    y / packed: optional bf16 copies of the resulting dh (row-major / packed)."""
    arr = (_P * len(dys))(*dys)
    _check(lib().nf4s_rmsnorm_bwd(arr, len(dys), x, w, rstd, T, H, accumulate, dh, y, packed, stream))


def nf4s_rope_pair(q, q_heads, k, k_heads, T, S, head_dim, theta, inverse, stream=0, q_packed=None,
                   k_packed=None):
    _check(lib().nf4s_rope_pair(q, q_heads, k, k_heads, T, S, head_dim, theta, inverse, q_packed, k_packed,
                                stream))


def nf4s_rope(x, T, S, heads, head_dim, theta, inverse, stream=0):
    _check(lib().nf4s_rope(x, T, S, heads, head_dim, theta, inverse, stream))


def nf4s_attention_fwd(q, k, v, B, S, heads, kv_heads, head_dim, o, o_f32, lse, stream=0, packed=None):
    _check(lib().nf4s_attention_fwd(q, k, v, B, S, heads, kv_heads, head_dim, o, o_f32, lse, packed,
                                    stream))


def nf4s_attention_bwd(q, k, v, o_f32, dout, lse, B, S, heads, kv_heads, head_dim, dq, dk, dv, ws,
                       ws_bytes, stream=0, dv_packed=None):
    _check(lib().nf4s_attention_bwd(q, k, v, o_f32, dout, lse, B, S, heads, kv_heads, head_dim, dq,
                                    dk, dv, dv_packed, ws, ws_bytes, stream))


def nf4s_swiglu_fwd(g, u, T, width, out, stream=0, packed=None):
    _check(lib().nf4s_swiglu_fwd(g, u, T, width, out, packed, stream))


def nf4s_swiglu_bwd(ds, g, u, T, width, dg, du, stream=0, dg_packed=None, du_packed=None):
    _check(lib().nf4s_swiglu_bwd(ds, g, u, T, width, dg, du, dg_packed, du_packed, stream))


def nf4s_residual_add(h, y, n, out, stream=0):
    _check(lib().nf4s_residual_add(h, y, n, out, stream))


def nf4s_to_bf16(x, T, width, y, stream=0, packed=None):
    _check(lib().nf4s_to_bf16(x, T, width, y, packed, stream))


def nf4s_cross_entropy(logits, targets, T, V, loss, dlogits, ws, ws_bytes, stream=0):
    _check(lib().nf4s_cross_entropy(logits, targets, T, V, loss, dlogits, ws, ws_bytes, stream))


def nf4s_adamw(p, g, m, v, n, lr, beta1, beta2, eps, weight_decay, step, stream=0):
    _check(lib().nf4s_adamw(p, g, m, v, n, lr, beta1, beta2, eps, weight_decay, step, stream))


def nf4s_token_nll(logits, targets, T, V, nll, stream=0):
    _check(lib().nf4s_token_nll(logits, targets, T, V, nll, stream))


def nf4s_dpo_loss(nll_policy, nll_ref, mask, pairs, S, beta, loss, seq_coef, stream=0):
    _check(lib().nf4s_dpo_loss(nll_policy, nll_ref, mask, pairs, S, beta, loss, seq_coef, stream))


def nf4s_logit_grad(logits, targets, seq_coef, mask, T, S, V, dlogits, stream=0):
    _check(lib().nf4s_logit_grad(logits, targets, seq_coef, mask, T, S, V, dlogits, stream))


def lora_fwd(x, M, k_in, A, r, u_out, ws, ws_bytes, stream=0):
    _check(lib().lora_fwd(x, M, k_in, A, r, u_out, ws, ws_bytes, stream))


def lora_bwd(x, dy, u, M, k_in, n_out, B, r, scale, dA, dB, du_out, accumulate, ws, ws_bytes,
             stream=0):
    _check(lib().lora_bwd(x, dy, u, M, k_in, n_out, B, r, scale, dA, dB, du_out, accumulate, ws,
                          ws_bytes, stream))


def _i64_array(vals):
    return ctypes.cast((ctypes.c_int64 * len(vals))(*vals), ctypes.c_void_p)


def lora_grouped_workspace_bytes(n_outs, k_in, M, backward):
    """Workspace of lora_fwd_grouped / lora_bwd_grouped (any rank up to the maximum)."""
    out = ctypes.c_size_t()
    _check(lib().nf4s_lora_grouped_workspace_bytes(len(n_outs), _i64_array(n_outs), k_in, M,
                                                   int(bool(backward)), ctypes.byref(out)))
    return out.value


def lora_fwd_grouped(x, M, k_in, As, r, u_outs, ws, ws_bytes, stream=0):
    """u_outs[i] = x.As[i]^T for the adapters reading x, in one launch per kernel."""
    _check(lib().lora_fwd_grouped(x, M, k_in, _ptr_array(As), len(As), r, _ptr_array(u_outs), ws,
                                  ws_bytes, stream))


def lora_bwd_grouped(x, dys, us, M, k_in, n_outs, Bs, r, scale, dAs, dBs, du_outs, accumulate, ws,
                     ws_bytes, stream=0):
    """lora_bwd of each adapter reading x (lists of device pointers), one launch per kernel."""
    _check(lib().lora_bwd_grouped(x, _ptr_array(dys), _ptr_array(us), M, k_in, _i64_array(n_outs),
                                  _ptr_array(Bs), len(Bs), r, scale, _ptr_array(dAs), _ptr_array(dBs),
                                  _ptr_array(du_outs), accumulate, ws, ws_bytes, stream))


def layer_prefetch(slot, slot_bytes, host_src, nbytes, copy_stream, wait_free=None, record_ready=None):
    _check(lib().layer_prefetch(slot, slot_bytes, host_src, nbytes, copy_stream, wait_free,
                                record_ready))


def nf4s_event_create() -> int:
    ev = _P()
    _check(lib().nf4s_event_create(ctypes.byref(ev)))
    return ev.value


def nf4s_event_destroy(ev):
    _check(lib().nf4s_event_destroy(ev))


def nf4s_event_record(ev, stream):
    _check(lib().nf4s_event_record(ev, stream))


def nf4s_stream_wait_event(stream, ev):
    _check(lib().nf4s_stream_wait_event(stream, ev))


def nf4s_pool_create(slots, slot_bytes, copy_stream, compute_stream) -> int:
    arr = (_P * len(slots))(*slots)
    out = _P()
    _check(lib().nf4s_pool_create(len(slots), arr, slot_bytes, copy_stream, compute_stream,
                                  ctypes.byref(out)))
    return out.value


def nf4s_pool_destroy(pool):
    _check(lib().nf4s_pool_destroy(pool))


def nf4s_pool_set_layer(pool, layer, host_src, nbytes):
    _check(lib().nf4s_pool_set_layer(pool, layer, host_src, nbytes))


def nf4s_pool_prefetch(pool, layer):
    _check(lib().nf4s_pool_prefetch(pool, layer))


def nf4s_pool_acquire(pool, layer) -> int:
    out = _P()
    _check(lib().nf4s_pool_acquire(pool, layer, ctypes.byref(out)))
    return out.value


def nf4s_pool_release(pool, layer):
    _check(lib().nf4s_pool_release(pool, layer))


POOL_POISON_ON_RELEASE = 1


def nf4s_pool_set_debug(pool, flags):
    _check(lib().nf4s_pool_set_debug(pool, flags))


def nf4s_pool_stats(pool):
    c = ctypes.c_uint64(0)
    b = ctypes.c_uint64(0)
    _check(lib().nf4s_pool_stats(pool, ctypes.byref(c), ctypes.byref(b)))
    return int(c.value), int(b.value)
