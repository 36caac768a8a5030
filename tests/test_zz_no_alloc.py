"""streamed_linear_fwd_noalloc: the forward entry point that allocates nothing
(its scratch is a library-owned device array) against streamed_linear_fwd with
a caller workspace -- the same kernels, so the same bits -- on two calls in a
row, the second smaller, and against the oracle; a size past the array is
refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import layer_streamed_nf4_amd as L
import synth
from oracle import linear, nf4
from tests.gpu_helpers import bits_to_f32, dev_bf16bits, dev_f32, host_u16, quantize_on_gpu, require_gpu, stream, ws_tensor

R, S = 16, 2.0
FAKE = 1 << 40


def test_noalloc_refuses_sizes_past_its_scratch():
    """No GPU needed: the size check runs on the host before any HIP call."""
    d = L.nf4s_tensor_layout(4096, 14336)
    need = L.nf4s_workspace_bytes(L.OP_LINEAR_FWD, 8192, 4096, 14336)
    assert need > L.NOALLOC_SCRATCH_BYTES
    with pytest.raises(L.Nf4sError) as e:
        L.streamed_linear_fwd_noalloc(FAKE, d, FAKE, 8192, FAKE, None, None, 0, 0.0)
    assert e.value.code == L.EWORKSPACE
    # every 8B projection up to M = 2048 fits
    for n, k in ((4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)):
        for M in (1, 512, 2048):
            assert L.nf4s_workspace_bytes(L.OP_LINEAR_FWD, M, n, k) <= L.NOALLOC_SCRATCH_BYTES


def _case(proj, n, k, M, layer):
    w = synth.weight(layer, proj, n, k)
    shard, d, status = quantize_on_gpu(w)
    assert status == 0
    a, b = synth.lora_pair(layer, proj, n, k)
    x = synth.activation((M, k), layer, 0)
    return dict(w=w, shard=shard, d=d, a=a, b=b, x=x, n=n, k=k, M=M)


def _both(c):
    s = stream()
    n, k, M = c["n"], c["k"], c["M"]
    x, A, B = dev_bf16bits(c["x"]), dev_f32(c["a"]), dev_f32(c["b"])
    u = torch.empty((M, R), dtype=torch.float32, device="cuda")
    wl = ws_tensor(L.nf4s_workspace_bytes(L.OP_LORA_FWD, M, n, k))
    L.lora_fwd(x.data_ptr(), M, k, A.data_ptr(), R, u.data_ptr(), wl.data_ptr(), wl.numel(), s)
    y_ws = torch.full((M, n), -1, dtype=torch.int16, device="cuda")
    y_na = torch.full((M, n), -1, dtype=torch.int16, device="cuda")
    ws = ws_tensor(L.nf4s_workspace_bytes(L.OP_LINEAR_FWD, M, n, k))
    L.streamed_linear_fwd(c["shard"].data_ptr(), c["d"], x.data_ptr(), M, y_ws.data_ptr(), u.data_ptr(),
                          B.data_ptr(), R, S, ws.data_ptr(), ws.numel(), s)
    L.streamed_linear_fwd_noalloc(c["shard"].data_ptr(), c["d"], x.data_ptr(), M, y_na.data_ptr(),
                                  u.data_ptr(), B.data_ptr(), R, S, s)
    torch.cuda.synchronize()
    return host_u16(y_ws), host_u16(y_na)


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_twice_then_smaller():
    require_gpu()
    # 8B o projection at M = 512: the contraction is split four ways, so the
    # scratch holds the packed x and fp32 partials; then a smaller call that
    # reuses the array holding the first call's partials
    for proj, n, k, M, layer in (("o", 4096, 4096, 512, 2), ("q", 576, 576, 300, 5)):
        print(f"noalloc {proj} {n}x{k} M={M}", flush=True)
        c = _case(proj, n, k, M, layer)
        y_ws, y_na = _both(c)
        assert np.array_equal(y_ws, y_na), proj
        wq = bits_to_f32(nf4.dequantize_bf16(nf4.quantize(c["w"]))).astype(np.float64)
        y_ref, _ = linear.forward(bits_to_f32(c["x"]).astype(np.float64), wq, c["a"], c["b"], S)
        assert linear.rel_err(bits_to_f32(y_na), y_ref) <= 5e-3
