"""The gate + up forward with the SwiGLU epilogue (streamed_linear_fwd_swiglu)
against the unfused launches it replaces and against the oracle.

"Soup layer-streamed NF4 training measured", section 2.1: the decoder layer
around the streamed linears is unmodified, so the fused launch must give the
bits of streamed_linear_fwd_grouped on (gate, up) followed by nf4s_swiglu_fwd,
row-major and in fragment order, with and without adapters, for whole and
ragged row tiles.
"""
import numpy as np
import pytest
import torch

import layer_streamed_nf4_amd as L
import synth
from oracle import decoder as D, linear, nf4
from tests.gpu_helpers import (bits_to_f32, dev_bf16bits, dev_f32, host_u16, packed_rows_below, require_gpu,
                               stream, ws_tensor)

pytestmark = pytest.mark.gpu
R, S = 16, 2.0


def _setup(width, k, M, layer):
    descs, end = [], 0
    for n in (width, width):
        descs.append(L.nf4s_tensor_layout(n, k, end))
        end = descs[-1].end
    shard = torch.zeros(end, dtype=torch.uint8, device="cuda")
    ws = []
    for p, d in zip(("gate", "up"), descs):
        w = synth.weight(layer, p, width, k)
        wq = ws_tensor(L.nf4s_workspace_bytes(L.OP_QUANTIZE, 0, width, k))
        wd = dev_f32(w)
        L.nf4_quantize_shard(wd.data_ptr(), L.DTYPE_F32, width, k, shard.data_ptr(), d, None, wq.data_ptr(),
                             wq.numel(), stream())
        ws.append((wq, wd))
    torch.cuda.synchronize()
    x = synth.activation((M, k), layer, 0)
    return shard, descs, x


def _run(width, k, M, layer, lora):
    require_gpu()
    s = stream()
    shard, descs, x = _setup(width, k, M, layer)
    xd = dev_bf16bits(x)
    xp = ws_tensor(L.nf4s_packed_activation_bytes(M, k))
    L.nf4s_pack_activation(xd.data_ptr(), M, k, xp.data_ptr(), xp.numel(), s)
    keep, us, Bs = [], [None, None], [None, None]
    pairs = {}
    for i, p in enumerate(("gate", "up")):
        if p in lora:
            a, b = synth.lora_pair(layer, p, width, k)
            pairs[p] = (a, b)
            A, B = dev_f32(a), dev_f32(b)
            u = torch.empty((M, R), dtype=torch.float32, device="cuda")
            wl = ws_tensor(L.nf4s_workspace_bytes(L.OP_LORA_FWD, M, width, k))
            L.lora_fwd(xd.data_ptr(), M, k, A.data_ptr(), R, u.data_ptr(), wl.data_ptr(), wl.numel(), s)
            keep += [A, B, u, wl]
            us[i], Bs[i] = u.data_ptr(), B.data_ptr()
    r, sc = (R, S) if lora else (0, 0.0)
    pk_bytes = L.nf4s_packed_activation_bytes(M, width)
    # fused
    out = torch.full((M, width), -1, dtype=torch.int16, device="cuda")
    out_pk = torch.full((pk_bytes,), 0x7F, dtype=torch.uint8, device="cuda")
    L.streamed_linear_fwd_swiglu(shard.data_ptr(), descs[0], descs[1], xp.data_ptr(), M, out.data_ptr(),
                                 out_pk.data_ptr(), pk_bytes, us, Bs, r, sc, s)
    # unfused: grouped launch, then the elementwise kernel
    g = torch.empty((M, width), dtype=torch.int16, device="cuda")
    u_ = torch.empty((M, width), dtype=torch.int16, device="cuda")
    wsg = ws_tensor(L.grouped_workspace_bytes([width, width], k, M))
    L.streamed_linear_fwd_grouped(shard.data_ptr(), descs, xp.data_ptr(), M, [g.data_ptr(), u_.data_ptr()],
                                  us, Bs, r, sc, wsg.data_ptr(), wsg.numel(), s)
    ref = torch.empty((M, width), dtype=torch.int16, device="cuda")
    ref_pk = torch.full((pk_bytes,), 0x7F, dtype=torch.uint8, device="cuda")
    L.nf4s_swiglu_fwd(g.data_ptr(), u_.data_ptr(), M, width, ref.data_ptr(), s, packed=ref_pk.data_ptr())
    torch.cuda.synchronize()
    return dict(x=x, out=host_u16(out), out_pk=out_pk.cpu().numpy(), ref=host_u16(ref),
                ref_pk=ref_pk.cpu().numpy(), g=host_u16(g), u=host_u16(u_), pairs=pairs)


@pytest.mark.parametrize("M,lora,layer,shape", [(512, (), 1, "8b"), (512, ("gate", "up"), 2, "8b"),
                                                (700, ("up",), 3, "8b"), (2048, ("gate", "up"), 4, "8b"),
                                                # 135M widths: 24 tiles of 64 + 64 columns for 512
                                                # rows, a contraction of 9 steps (never split)
                                                (300, ("gate",), 5, "135m"), (512, ("up",), 6, "135m")])
def test_fused_swiglu_equals_grouped_then_swiglu(M, lora, layer, shape):
    width, k = synth.SHAPES[shape]["gate"]
    print(f"fused swiglu {shape} M={M} lora={lora}", flush=True)
    assert L.nf4s_swiglu_fused_supported(M, width, k)
    got = _run(width, k, M, layer, lora)
    assert np.array_equal(got["out"], got["ref"])
    a = packed_rows_below(got["out_pk"], M, width)
    b = packed_rows_below(got["ref_pk"], M, width)
    assert np.array_equal(a, b)
    if M in (700, 300):
        # against the oracle: silu(g) * u of its own fp64 products, bf16-rounded where the path rounds
        x = bits_to_f32(got["x"]).astype(np.float64)
        gu = {}
        for p in ("gate", "up"):
            w = bits_to_f32(nf4.dequantize_bf16(nf4.quantize(synth.weight(layer, p, width, k)))).astype(np.float64)
            a_, b_ = got["pairs"].get(p, (None, None))
            gu[p], _ = linear.forward(x, w, a_, b_, S if p in got["pairs"] else 0.0)
        ref = D.bf16(D.silu(D.bf16(gu["gate"])) * D.bf16(gu["up"]))
        sw = bits_to_f32(got["out"]).astype(np.float64)
        err = np.abs(sw - ref)
        assert np.all(err <= 2.0 ** -6 * np.abs(ref) + 2.0 ** -9 * np.max(np.abs(ref))), float(np.max(err))
