"""Llama-style decoder around the streamed NF4 linears: forward, backward, AdamW.

TEST INFRASTRUCTURE (see oracle/__init__.py). Plain fp64 NumPy, one function
per operation, written from the textbook definitions; no blocking or fusion.

What the pages fix ("Soup layer-streamed NF4 training measured", sections
2.1, 2.2 and 4.3; "Fine-Tune 8B Models on 4GB VRAM", "Boundary Conditions
List"): a llama-architecture decoder (SmolLM2-135M: 30 layers, tied
embeddings) whose decoder-layer linears are the streamed NF4 weights with bf16
compute and LoRA r16 on q_proj and v_proj; embeddings and lm_head stay resident
and unquantised (bf16); every layer body is checkpointed, so the backward
recomputes it; the check is on logits, a 25-step loss curve and the LoRA
gradients.

Readings where the pages are silent (llama's published definitions):
  * RMSNorm: y = x / sqrt(mean(x^2) + eps) * w;
  * rotary embedding in the rotate-half form: for head dimension d, pair
    (j, j + d/2) of a row at position t is rotated by t * theta^(-2j/d);
    positions count within each sequence (rows are batch-major, b*S + t);
  * causal softmax attention with grouped KV heads (head h reads KV head
    h // (heads / kv_heads)), scale 1/sqrt(d);
  * SwiGLU MLP: down(silu(gate(x)) * up(x)), silu(z) = z / (1 + e^-z);
  * pre-norm residual blocks, a final RMSNorm, logits = h E^T, mean token
    cross-entropy against given next-token targets;
  * precision of the training step ("bf16 compute"): every tensor that feeds
    a matrix product or the attention is bf16 -- the norm outputs, q/k/v after
    RoPE, the attention output, the SwiGLU product, the logits, and in the
    backward the gradients entering each product -- while the residual stream,
    norms, softmaxes and reductions are computed in higher precision. With
    exact=True no rounding happens at all (used by the finite-difference pins);
  * the optimiser of the adapters is plain AdamW (decoupled weight decay,
    bias-corrected moments) in fp32; the pages' paged 8-bit AdamW is an
    allocation strategy of a library, not part of the step's arithmetic.

Preference step ("Soup v0.72.4 technical analysis", sections 3.1-3.3): the
reference model is the same frozen base with the adapters switched off, the
policy the base with them on; no second model. The pages name DPO without
writing its loss; reading: the DPO objective of Rafailov et al. (2023),
    L = -mean_p log sigmoid(beta * ((lp_c - lr_c) - (lp_r - lr_r))),
with lp / lr the policy / reference log-probability of a sequence, the sum of
its masked per-token log-probabilities log softmax(z_t)[target_t], and
sequences ordered chosen, rejected per pair.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import nf4

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass
class Config:
    hidden: int
    inter: int
    heads: int
    kv_heads: int
    head_dim: int
    vocab: int
    layers: int
    rope_theta: float
    eps: float
    targets: tuple = ("q", "v")
    r: int = 16
    alpha: int = 32

    @property
    def scale(self) -> float:
        return self.alpha / self.r


@dataclass
class Params:
    """embed/lm_head [V, H] (bf16 values), norm weights [H], frozen linear
    weights W[l][p] = W' values [N_out, K_in], adapters lora[l][p] = (A, B)."""
    embed: np.ndarray
    lm_head: np.ndarray
    w_attn: list
    w_mlp: list
    w_final: np.ndarray
    W: list
    lora: list


def bf16(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (via fp32, nearest-even) and return as fp64."""
    return nf4.bf16_to_f32(nf4.bf16_rne_bits(np.asarray(x, dtype=np.float64).astype(np.float32))).astype(np.float64)


def _r(x, exact):
    return np.asarray(x, dtype=np.float64) if exact else bf16(x)


# ---- operations --------------------------------------------------------------

def rmsnorm(x, w, eps):
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * rstd * w, rstd


def rmsnorm_bwd(dy, x, w, rstd):
    """dL/dx of y = x * rstd(x) * w."""
    g = dy * w
    return rstd * g - x * rstd ** 3 * np.mean(g * x, axis=-1, keepdims=True)


def rope_tables(seq, d, theta):
    inv = theta ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.arange(seq, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x, cos, sin, inverse=False):
    """x [B, S, heads, d]; rotate pair (j, j + d/2) by the position's angle
    (by minus the angle when inverse)."""
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    c = cos[None, :, None, :]
    s = (-sin if inverse else sin)[None, :, None, :]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q, k, v, kv_group):
    """q [B, S, H, d], k/v [B, S, Hkv, d] -> o [B, S, H, d], P [B, H, S, S]."""
    B, S, H, d = q.shape
    o = np.empty_like(q)
    P = np.empty((B, H, S, S))
    mask = np.triu(np.ones((S, S), dtype=bool), 1)
    for h in range(H):
        kh, vh = k[:, :, h // kv_group], v[:, :, h // kv_group]
        s = np.einsum("bid,bjd->bij", q[:, :, h], kh) / np.sqrt(d)
        s = np.where(mask[None], -np.inf, s)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=-1, keepdims=True)
        P[:, h] = p
        o[:, :, h] = np.einsum("bij,bjd->bid", p, vh)
    return o, P


def attention_bwd(do, q, k, v, P, kv_group):
    B, S, H, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(H):
        g = h // kv_group
        p = P[:, h]
        dv[:, :, g] += np.einsum("bij,bid->bjd", p, do[:, :, h])
        dp = np.einsum("bid,bjd->bij", do[:, :, h], v[:, :, g])
        ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
        dq[:, :, h] = np.einsum("bij,bjd->bid", ds, k[:, :, g]) / np.sqrt(d)
        dk[:, :, g] += np.einsum("bij,bid->bjd", ds, q[:, :, h]) / np.sqrt(d)
    return dq, dk, dv


def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu_bwd(ds, g, u):
    sg = 1.0 / (1.0 + np.exp(-g))
    return ds * u * (sg * (1.0 + g * (1.0 - sg))), ds * g * sg


def cross_entropy(logits, targets):
    """Mean token cross-entropy and its gradient; logits [T, V], targets [T]."""
    m = logits.max(axis=-1, keepdims=True)
    z = logits - m
    lse = np.log(np.sum(np.exp(z), axis=-1, keepdims=True))
    T = logits.shape[0]
    loss = float(np.mean(lse[:, 0] - z[np.arange(T), targets]))
    p = np.exp(z - lse)
    p[np.arange(T), targets] -= 1.0
    return loss, p / T


def adamw(p, g, m, v, t, lr, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0):
    """One AdamW step (t counts from 1); returns new (p, m, v)."""
    m = beta1 * m + (1 - beta1) * g
    v = beta2 * v + (1 - beta2) * g * g
    mhat = m / (1 - beta1 ** t)
    vhat = v / (1 - beta2 ** t)
    p = p * (1 - lr * wd) - lr * mhat / (np.sqrt(vhat) + eps)
    return p, m, v


# ---- the model -----------------------------------------------------------------

def _lin(x, P: Params, l, p, cfg, adapters=True):
    y = x @ P.W[l][p].T
    if adapters and p in cfg.targets:
        a, b = P.lora[l][p]
        y = y + cfg.scale * ((x @ a.T) @ b.T)
    return y


def _lin_bwd(x, dy, P: Params, l, p, cfg, grads):
    dx = dy @ P.W[l][p]
    if p in cfg.targets:
        a, b = P.lora[l][p]
        du = cfg.scale * (dy @ b)
        grads[(l, p)] = (du.T @ x, cfg.scale * (dy.T @ (x @ a.T)))
        dx = dx + du @ a
    return dx


def layer_forward(P: Params, l, h, B, S, cfg: Config, cos, sin, exact=False, adapters=True):
    """Layer l of the decoder from its input residual h [B*S, H]: returns
    (h_out, cache of the layer's activations)."""
    T = B * S
    grp = cfg.heads // cfg.kv_heads
    c = {"h_in": h}
    n1, c["rstd1"] = rmsnorm(h, P.w_attn[l], cfg.eps)
    n1 = _r(n1, exact)
    q = _r(_lin(n1, P, l, "q", cfg, adapters), exact).reshape(B, S, cfg.heads, cfg.head_dim)
    k = _r(_lin(n1, P, l, "k", cfg, adapters), exact).reshape(B, S, cfg.kv_heads, cfg.head_dim)
    v = _r(_lin(n1, P, l, "v", cfg, adapters), exact).reshape(B, S, cfg.kv_heads, cfg.head_dim)
    qr, kr = _r(rope(q, cos, sin), exact), _r(rope(k, cos, sin), exact)
    o, Pm = attention(qr, kr, v, grp)
    o = _r(o, exact).reshape(T, -1)
    h = h + _r(_lin(o, P, l, "o", cfg, adapters), exact)
    c.update(n1=n1, qr=qr, kr=kr, v=v, P=Pm, o=o, h_mid=h)
    n2, c["rstd2"] = rmsnorm(h, P.w_mlp[l], cfg.eps)
    n2 = _r(n2, exact)
    g = _r(_lin(n2, P, l, "gate", cfg, adapters), exact)
    u = _r(_lin(n2, P, l, "up", cfg, adapters), exact)
    sw = _r(silu(g) * u, exact)
    h = h + _r(_lin(sw, P, l, "down", cfg, adapters), exact)
    c.update(n2=n2, g=g, u=u, sw=sw)
    return h, c


def forward(P: Params, ids, targets, cfg: Config, exact=False, adapters=True):
    """Returns (loss, logits [B*S, V], cache). adapters=False evaluates the
    frozen base alone (the reference model of a preference step)."""
    B, S = ids.shape
    cos, sin = rope_tables(S, cfg.head_dim, cfg.rope_theta)
    h = P.embed[ids.reshape(-1)].astype(np.float64)
    cache = {"layers": []}
    for l in range(cfg.layers):
        h, c = layer_forward(P, l, h, B, S, cfg, cos, sin, exact, adapters)
        cache["layers"].append(c)
    hn, rstd_f = rmsnorm(h, P.w_final, cfg.eps)
    hn = _r(hn, exact)
    logits = _r(hn @ P.lm_head.T, exact)
    loss, dlogits = cross_entropy(logits, targets.reshape(-1))
    cache.update(h_final=h, rstd_f=rstd_f, hn=hn, dlogits=dlogits, shape=(B, S), cos=cos, sin=sin)
    return loss, logits, cache


def backward(P: Params, cache, cfg: Config, exact=False):
    """Gradients of the mean cross-entropy: {(layer, proj): (dA, dB)} for the
    adapters and dh0 = dL/d(embedding rows) [B*S, H]."""
    B, S = cache["shape"]
    cos, sin = cache["cos"], cache["sin"]
    grads = {}
    dl = _r(cache["dlogits"], exact)
    dhn = _r(dl @ P.lm_head, exact)
    dh = rmsnorm_bwd(dhn, cache["h_final"], P.w_final, cache["rstd_f"])
    for l in range(cfg.layers - 1, -1, -1):
        dh = layer_backward(P, l, cache["layers"][l], dh, B, S, cfg, cos, sin, grads, exact)
    return {"lora": grads, "dh0": dh}


def layer_backward(P: Params, l, c, dh, B, S, cfg: Config, cos, sin, grads, exact=False):
    """Backward of layer l from dL/dh_out (fp64 [B*S, H]) and the layer's
    cached activations: returns dL/dh_in and adds the layer's adapter
    gradients to grads."""
    T = B * S
    grp = cfg.heads // cfg.kv_heads
    dd = _r(dh, exact)
    dsw = _r(_lin_bwd(c["sw"], dd, P, l, "down", cfg, grads), exact)
    dg, du = swiglu_bwd(dsw, c["g"], c["u"])
    dg, du = _r(dg, exact), _r(du, exact)
    dn2 = (_r(_lin_bwd(c["n2"], dg, P, l, "gate", cfg, grads), exact)
           + _r(_lin_bwd(c["n2"], du, P, l, "up", cfg, grads), exact))
    dh = dh + rmsnorm_bwd(dn2, c["h_mid"], P.w_mlp[l], c["rstd2"])
    dao = _r(dh, exact)
    do = _r(_lin_bwd(c["o"], dao, P, l, "o", cfg, grads), exact)
    do = do.reshape(B, S, cfg.heads, cfg.head_dim)
    dqr, dkr, dv = attention_bwd(do, c["qr"], c["kr"], c["v"], c["P"], grp)
    dq = _r(rope(_r(dqr, exact), cos, sin, inverse=True), exact).reshape(T, -1)
    dk = _r(rope(_r(dkr, exact), cos, sin, inverse=True), exact).reshape(T, -1)
    dv = _r(dv, exact).reshape(T, -1)
    dn1 = (_r(_lin_bwd(c["n1"], dq, P, l, "q", cfg, grads), exact)
           + _r(_lin_bwd(c["n1"], dk, P, l, "k", cfg, grads), exact)
           + _r(_lin_bwd(c["n1"], dv, P, l, "v", cfg, grads), exact))
    dh = dh + rmsnorm_bwd(dn1, c["h_in"], P.w_attn[l], c["rstd1"])
    return dh


# ---- preference step -------------------------------------------------------------

def token_nll(logits, targets):
    """Per-token negative log-probability of the target: logsumexp(z_t) - z_t[target_t]."""
    m = logits.max(axis=-1, keepdims=True)
    lse = (m + np.log(np.sum(np.exp(logits - m), axis=-1, keepdims=True)))[:, 0]
    return lse - logits[np.arange(logits.shape[0]), targets]


def log_sigmoid(x):
    return -(np.maximum(-x, 0.0) + np.log1p(np.exp(-np.abs(x))))


def dpo_loss(nll_policy, nll_ref, mask, seq, beta):
    """DPO over sequences of length seq ordered chosen, rejected per pair.
    Returns (loss, coef) with coef[s] = dL/d(nll summed over sequence s's
    masked tokens) -- the weight of (softmax - onehot) in that sequence's
    logit gradient."""
    lp = -(mask * nll_policy).reshape(-1, seq).sum(axis=1)
    lr = -(mask * nll_ref).reshape(-1, seq).sum(axis=1)
    n = lp.size // 2
    delta = beta * ((lp[0::2] - lr[0::2]) - (lp[1::2] - lr[1::2]))
    loss = float(-np.mean(log_sigmoid(delta)))
    g = -(1.0 / n) * np.exp(log_sigmoid(-delta))   # dL/d delta = -sigmoid(-delta)/n
    coef = np.empty(2 * n)
    coef[0::2] = -beta * g     # d lp_c = -d nll_c
    coef[1::2] = beta * g
    return loss, coef


def dpo_step(P: Params, ids, targets, mask, cfg: Config, beta, exact=False):
    """Reference forward (adapters off), policy forward and backward for the
    DPO loss. ids/targets [2 * pairs, S] ordered chosen, rejected per pair;
    mask [2 * pairs, S] weights of the response tokens. Returns (loss,
    {"lora": ..., "dh0": ...}, policy logits)."""
    S = ids.shape[1]
    _, ref_logits, _ = forward(P, ids, targets, cfg, exact, adapters=False)
    _, logits, cache = forward(P, ids, targets, cfg, exact)
    t = targets.reshape(-1)
    m = mask.reshape(-1).astype(np.float64)
    loss, coef = dpo_loss(token_nll(logits, t), token_nll(ref_logits, t), m, S, beta)
    z = logits - logits.max(axis=-1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=-1, keepdims=True)
    p[np.arange(t.size), t] -= 1.0
    w = np.repeat(coef, S) * m
    cache["dlogits"] = p * w[:, None]
    return loss, backward(P, cache, cfg, exact), logits
