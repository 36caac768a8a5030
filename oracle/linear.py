"""Frozen NF4 linear with a LoRA adapter: forward, backward and adapter grads.

TEST INFRASTRUCTURE (see oracle/__init__.py). Plain matrix products in fp64.

What the pages fix: the frozen base linears run as NF4 weights with bf16
compute (gate walkthrough, section 2.1: "NF4 double quant + bf16 compute";
LoRA r=16 on q_proj, v_proj). The base is frozen, so the backward produces
dL/dx = dL/dy . W and no weight gradient (section 4.4: the decoder counts
2 forward + 2 recompute + 2 dL/dx, not the 8 of a trainable weight; English
article, "The Principle of Layer Streaming": dL/dx = W^T dL/dy). The adapter
gradients must be non-zero in every layer (section 2.2, check 2), and with
B = 0 the gradient of A is structurally zero (section 2.5).

Readings: W'[N_out, K_in] is the dequantised bf16 weight; the LoRA update is
the plain one, y += s * (x A^T) B^T with s = alpha / r (no rsLoRA, dropout 0,
no bias -- llama projections have none). Loss convention for checks:
L = <dy, y>.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def forward(x, w, a=None, b=None, scale=0.0):
    """y = x W'^T + s (x A^T) B^T.

    x [M, K_in], w [N_out, K_in] (values of W'), a [r, K_in], b [N_out, r].
    Returns (y [M, N_out], u [M, r] or None) in fp64.
    """
    x, w = _f64(x), _f64(w)
    y = x @ w.T
    u = None
    if a is not None:
        u = x @ _f64(a).T
        y = y + scale * (u @ _f64(b).T)
    return y, u


def backward(x, dy, w, a=None, b=None, scale=0.0):
    """Gradients of L = <dy, y> for the forward above.

    Returns dict with dx [M, K_in] and, with an adapter, du = s dy B [M, r],
    dA = du^T x [r, K_in], dB = s dy^T (x A^T) [N_out, r]. No dW (frozen base).
    """
    x, dy, w = _f64(x), _f64(dy), _f64(w)
    dx = dy @ w
    out = {"dx": dx}
    if a is not None:
        a, b = _f64(a), _f64(b)
        u = x @ a.T
        du = scale * (dy @ b)
        out["du"] = du
        out["dA"] = du.T @ x
        out["dB"] = scale * (dy.T @ u)
        out["dx"] = dx + du @ a
    return out


def loss(x, dy, w, a=None, b=None, scale=0.0):
    y, _ = forward(x, w, a, b, scale)
    return float(np.sum(_f64(dy) * y))


def rel_err(got, ref):
    """max |got - ref| / max |ref| (the parity metric for GEMM/LoRA outputs)."""
    got, ref = _f64(got), _f64(ref)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / den)
