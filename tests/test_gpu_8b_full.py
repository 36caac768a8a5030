"""Full-size, element-wise parity of one Llama-8B-shaped layer's streamed
linears against the oracle, in exactly the launches the decoder step makes.

Gate walkthrough ("Soup layer-streamed NF4 training measured"), section 2.2:
the shipped path is checked on its real shapes. Per layer the decoder runs
  forward:  q, k, v as one grouped launch (adapters on the targets among them),
            o into the residual stream, gate and up as one grouped launch,
            down into the residual stream;
  backward: the adapter gradients of each input group, then down alone (its
            packed dy written by the norm backward), gate + up and q + k + v
            each as one contraction when every member would split alone (else
            one call per projection), o alone.
Every output element of every launch is compared with an fp64 product of the
oracle's own dequantised weights (5e-3 of the largest magnitude for bf16
outputs, 1e-5 for the fp32 adapter results); the residual stream must equal
h_in + the bf16 output exactly. M = 512 is the B1 S512 step with adapters on
q and v; M = 2048 is the B4 step with adapters on all seven projections.
"""
import numpy as np
import pytest
import torch

import layer_streamed_nf4_amd as L
import synth
from layer_streamed_nf4_amd.stack import PROJ, ShardSet
from oracle import linear, nf4
from tests.gpu_helpers import bits_to_f32, dev_bf16bits, dev_f32, host_u16, require_gpu, stream, ws_tensor

pytestmark = pytest.mark.gpu
TOL = 5e-3
R, ALPHA = 16, 32
S = ALPHA / R
LAYER = 9
SHAPES = synth.SHAPES["8b"]
GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


@pytest.fixture(scope="module")
def layer():
    require_gpu()
    print("8b layer: quantise on the device, dequantise in the oracle", flush=True)
    sh = ShardSet(SHAPES, 1, lambda i, p: dev_f32(synth.weight(LAYER, p, *SHAPES[p])), pinned=False,
                  keep_device=True)
    W = {p: bits_to_f32(nf4.dequantize_bf16(nf4.quantize(synth.weight(LAYER, p, *SHAPES[p]))))
         .astype(np.float64) for p in PROJ}
    lora = {p: synth.lora_pair(LAYER, p, *SHAPES[p]) for p in PROJ}
    return dict(base=sh.device[0], descs=sh.layout.descs, W=W, lora=lora)


def _rel(got, ref):
    return linear.rel_err(got, ref)


def _packed(x, M, K, keep):
    xp = ws_tensor(L.nf4s_packed_activation_bytes(M, K))
    L.nf4s_pack_activation(x.data_ptr(), M, K, xp.data_ptr(), xp.numel(), stream())
    keep.append(xp)
    return xp


def _grouped_bwd_used(ps, M):
    """The decoder's rule: one contraction when every member would split alone."""
    k = SHAPES[ps[0]][1]
    return len(ps) > 1 and all(L.nf4s_workspace_bytes(L.OP_LINEAR_BWD_PACKED, M, SHAPES[p][0], k) > 0
                               for p in ps)


@pytest.mark.parametrize("M,targets", [(512, ("q", "v")), (2048, PROJ)])
def test_8b_layer_linears_full_size(layer, M, targets):
    s = stream()
    keep = []
    base = layer["base"].data_ptr()
    descs = layer["descs"]
    A = {p: dev_f32(layer["lora"][p][0]) for p in targets}
    B = {p: dev_f32(layer["lora"][p][1]) for p in targets}
    results = {}

    # ---- forward, one input per group -------------------------------------
    for gi, ps in enumerate(GROUPS):
        k = SHAPES[ps[0]][1]
        x = synth.activation((M, k), 3, gi)
        xd = dev_bf16bits(x)
        xp = _packed(xd, M, k, keep)
        tg = [p for p in ps if p in targets]
        u = {p: torch.empty((M, R), dtype=torch.float32, device="cuda") for p in tg}
        if tg:
            wl = ws_tensor(L.lora_grouped_workspace_bytes([SHAPES[p][0] for p in tg], k, M, False))
            L.lora_fwd_grouped(xd.data_ptr(), M, k, [A[p].data_ptr() for p in tg], R,
                               [u[p].data_ptr() for p in tg], wl.data_ptr(), wl.numel(), s)
            keep.append(wl)
        ys = {p: torch.empty((M, SHAPES[p][0]), dtype=torch.int16, device="cuda") for p in ps}
        us = [u[p].data_ptr() if p in tg else None for p in ps]
        Bs = [B[p].data_ptr() if p in tg else None for p in ps]
        r, sc = (R, S) if tg else (0, 0.0)
        h_in = h_out = None
        if len(ps) > 1:
            ws = ws_tensor(L.grouped_workspace_bytes([SHAPES[p][0] for p in ps], k, M))
            L.streamed_linear_fwd_grouped(base, [descs[p] for p in ps], xp.data_ptr(), M,
                                          [ys[p].data_ptr() for p in ps], us, Bs, r, sc,
                                          ws.data_ptr(), ws.numel(), s)
        else:
            (p,) = ps
            ws = ws_tensor(L.nf4s_workspace_bytes(L.OP_LINEAR_FWD_PACKED, M, SHAPES[p][0], k))
            h_in = dev_f32(synth.weight(LAYER + 100 + gi, p, M, SHAPES[p][0], sigma=1.0))
            h_out = torch.empty_like(h_in)
            L.streamed_linear_fwd_residual(base, descs[p], xp.data_ptr(), M, ys[p].data_ptr(), us[0],
                                           Bs[0], r, sc, h_in.data_ptr(), h_out.data_ptr(),
                                           ws.data_ptr(), ws.numel(), s)
        torch.cuda.synchronize()
        xf = bits_to_f32(x).astype(np.float64)
        for p in ps:
            a, b = (layer["lora"][p] if p in tg else (None, None))
            y_ref, u_ref = linear.forward(xf, layer["W"][p], a, b, S if p in tg else 0.0)
            y = bits_to_f32(host_u16(ys[p]))
            results[("y", p)] = _rel(y, y_ref)
            assert results[("y", p)] <= TOL, (p, results[("y", p)])
            if p in tg:
                assert _rel(u[p].cpu().numpy(), u_ref) <= 1e-5, p
            if h_in is not None:
                want = (h_in.cpu().numpy() + y).astype(np.float32)
                assert np.array_equal(h_out.cpu().numpy().view(np.uint32), want.view(np.uint32)), p
        del ws, xd

    # ---- backward -----------------------------------------------------------
    for gi, ps in enumerate(reversed(GROUPS)):
        k = SHAPES[ps[0]][1]
        x = synth.activation((M, k), 3, len(GROUPS) - 1 - gi)       # the forward's input
        xd = dev_bf16bits(x)
        dys = {p: synth.activation((M, SHAPES[p][0]), 4, 10 * gi + j) for j, p in enumerate(ps)}
        dyd = {p: dev_bf16bits(v) for p, v in dys.items()}
        tg = [p for p in ps if p in targets]
        u = {p: torch.empty((M, R), dtype=torch.float32, device="cuda") for p in tg}
        du = {p: torch.empty((M, R), dtype=torch.float32, device="cuda") for p in tg}
        dA = {p: torch.empty((R, k), dtype=torch.float32, device="cuda") for p in tg}
        dB = {p: torch.empty((SHAPES[p][0], R), dtype=torch.float32, device="cuda") for p in tg}
        if tg:
            ns = [SHAPES[p][0] for p in tg]
            wl = ws_tensor(max(L.lora_grouped_workspace_bytes(ns, k, M, False),
                               L.lora_grouped_workspace_bytes(ns, k, M, True)))
            L.lora_fwd_grouped(xd.data_ptr(), M, k, [A[p].data_ptr() for p in tg], R,
                               [u[p].data_ptr() for p in tg], wl.data_ptr(), wl.numel(), s)
            L.lora_bwd_grouped(xd.data_ptr(), [dyd[p].data_ptr() for p in tg], [u[p].data_ptr() for p in tg],
                               M, k, ns, [B[p].data_ptr() for p in tg], R, S,
                               [dA[p].data_ptr() for p in tg], [dB[p].data_ptr() for p in tg],
                               [du[p].data_ptr() for p in tg], 0, wl.data_ptr(), wl.numel(), s)
            keep.append(wl)
        dyps = {p: _packed(dyd[p], M, SHAPES[p][0], keep) for p in ps}
        dxs = {}
        if _grouped_bwd_used(ps, M):
            dx = torch.empty((M, k), dtype=torch.int16, device="cuda")
            ws = ws_tensor(L.grouped_bwd_workspace_bytes([SHAPES[p][0] for p in ps], k, M))
            L.streamed_linear_bwd_grouped(base, [descs[p] for p in ps], [dyps[p].data_ptr() for p in ps], M,
                                          dx.data_ptr(), [du[p].data_ptr() if p in tg else None for p in ps],
                                          [A[p].data_ptr() if p in tg else None for p in ps],
                                          R if tg else 0, ws.data_ptr(), ws.numel(), s)
            dxs[ps] = dx
        else:
            for p in ps:
                dx = torch.empty((M, k), dtype=torch.int16, device="cuda")
                ws = ws_tensor(L.nf4s_workspace_bytes(L.OP_LINEAR_BWD_PACKED, M, SHAPES[p][0], k))
                L.streamed_linear_bwd_packed(base, descs[p], dyps[p].data_ptr(), M, dx.data_ptr(),
                                             du[p].data_ptr() if p in tg else None,
                                             A[p].data_ptr() if p in tg else None, R if p in tg else 0,
                                             ws.data_ptr(), ws.numel(), s)
                torch.cuda.synchronize()
                dxs[(p,)] = dx
        torch.cuda.synchronize()
        xf = bits_to_f32(x).astype(np.float64)
        grads = {}
        for p in ps:
            a, b = (layer["lora"][p] if p in tg else (None, None))
            grads[p] = linear.backward(xf, bits_to_f32(dys[p]).astype(np.float64), layer["W"][p], a, b,
                                       S if p in tg else 0.0)
            if p in tg:
                assert _rel(du[p].cpu().numpy(), grads[p]["du"]) <= 1e-5, p
                assert _rel(dA[p].cpu().numpy(), grads[p]["dA"]) <= 1e-5, p
                assert _rel(dB[p].cpu().numpy(), grads[p]["dB"]) <= 1e-5, p
        for key, dx in dxs.items():
            ref = sum(grads[p]["dx"] for p in key)
            got = bits_to_f32(host_u16(dx))
            results[("dx",) + key] = _rel(got, ref)
            assert results[("dx",) + key] <= TOL, (key, results[("dx",) + key])
        del ws, xd
    print("8b full-size errors (M=%d): " % M + ", ".join(f"{'/'.join(k)} {v:.2e}" for k, v in results.items()),
          flush=True)
