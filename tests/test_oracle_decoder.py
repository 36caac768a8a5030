"""Pins of the decoder oracle (CPU): finite differences of the loss in exact
fp64, closed forms, invariants, and an independent log-sum-exp.

"Soup layer-streamed NF4 training measured", sections 2.1-2.2: a llama decoder
(SmolLM2-135M) whose streamed linears carry LoRA on q/v; the checks are on
logits, loss and the adapter gradients. The definitions pinned here are the
llama ones listed in oracle/decoder.py.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

import synth
from oracle import decoder as D


def _cfg(**kw):
    c = dict(synth.DECODER["tiny"])
    c.pop("tied")
    c.update(kw)
    return D.Config(**c)


def _params(cfg, seed=0, b_scale=0.3):
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = synth.SHAPES["tiny"]
    W = [{p: rng.standard_normal(shapes[p]) * 0.15 for p in D.PROJ} for _ in range(cfg.layers)]
    lora = [{p: (rng.standard_normal((cfg.r, shapes[p][1])) * 0.1,
                 rng.standard_normal((shapes[p][0], cfg.r)) * b_scale) for p in cfg.targets}
            for _ in range(cfg.layers)]
    emb = rng.standard_normal((cfg.vocab, cfg.hidden)) * 0.5
    return D.Params(embed=emb, lm_head=emb, w_attn=[1 + 0.1 * rng.standard_normal(cfg.hidden) for _ in range(cfg.layers)],
                    w_mlp=[1 + 0.1 * rng.standard_normal(cfg.hidden) for _ in range(cfg.layers)],
                    w_final=1 + 0.1 * rng.standard_normal(cfg.hidden), W=W, lora=lora)


def _batch(cfg, B=2, S=8, seed=3):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.integers(0, cfg.vocab, size=(B, S)), rng.integers(0, cfg.vocab, size=(B, S)))


def test_finite_differences_adapters_and_embedding():
    """Central differences of the exact-fp64 loss agree with the backward for
    adapter entries of every layer and target, and for embedding rows."""
    cfg = _cfg()
    P = _params(cfg)
    ids, tg = _batch(cfg)
    loss, _, cache = D.forward(P, ids, tg, cfg, exact=True)
    g = D.backward(P, cache, cfg, exact=True)
    rng = np.random.Generator(np.random.PCG64(11))
    eps = 1e-5
    for (l, p), (dA, dB) in g["lora"].items():
        a, b = P.lora[l][p]
        for arr, grad in ((a, dA), (b, dB)):
            for _ in range(3):
                idx = tuple(rng.integers(0, s) for s in arr.shape)
                old = arr[idx]
                arr[idx] = old + eps
                lp = D.forward(P, ids, tg, cfg, exact=True)[0]
                arr[idx] = old - eps
                lm = D.forward(P, ids, tg, cfg, exact=True)[0]
                arr[idx] = old
                fd = (lp - lm) / (2 * eps)
                assert abs(fd - grad[idx]) <= 1e-6 + 1e-4 * abs(fd), (l, p, idx, fd, grad[idx])
    # embedding: perturb h0 at one position through a separate copy of the row
    dh0 = g["dh0"]
    tok = 5
    pos = 3
    emb2 = P.embed.copy()
    for j in (0, 17, 63):
        ids2 = ids.copy().reshape(-1)
        ids2[pos] = cfg.vocab - 1          # a row used at this position only
        assert np.sum(ids2 == cfg.vocab - 1) == 1
        ids2 = ids2.reshape(ids.shape)
        emb2[:] = P.embed
        Q = D.Params(**{**P.__dict__, "embed": emb2, "lm_head": P.lm_head})
        _, _, c2 = D.forward(Q, ids2, tg, cfg, exact=True)
        g2 = D.backward(Q, c2, cfg, exact=True)["dh0"]
        emb2[cfg.vocab - 1, j] += eps
        lp = D.forward(Q, ids2, tg, cfg, exact=True)[0]
        emb2[cfg.vocab - 1, j] -= 2 * eps
        lm = D.forward(Q, ids2, tg, cfg, exact=True)[0]
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - g2[pos, j]) <= 1e-6 + 1e-4 * abs(fd), (j, fd, g2[pos, j])
    assert np.isfinite(loss) and dh0.shape == (ids.size, cfg.hidden) and tok


def test_rmsnorm_closed_form_and_gradient():
    c = 0.7
    w = np.array([1.0, 2.0, -0.5, 3.0])
    y, rstd = D.rmsnorm(np.full((1, 4), c), w, 1e-5)
    assert np.allclose(y, w * c / math.sqrt(c * c + 1e-5), rtol=0, atol=1e-15)
    rng = np.random.Generator(np.random.PCG64(1))
    x = rng.standard_normal((3, 8))
    w = rng.standard_normal(8)
    dy = rng.standard_normal((3, 8))
    _, rstd = D.rmsnorm(x, w, 1e-5)
    dx = D.rmsnorm_bwd(dy, x, w, rstd)
    e = 1e-6
    for i, j in ((0, 0), (1, 5), (2, 7)):
        xp, xm = x.copy(), x.copy()
        xp[i, j] += e
        xm[i, j] -= e
        fd = (np.sum(dy * D.rmsnorm(xp, w, 1e-5)[0]) - np.sum(dy * D.rmsnorm(xm, w, 1e-5)[0])) / (2 * e)
        assert abs(fd - dx[i, j]) < 1e-7


def test_rope_is_a_rotation():
    S, d = 9, 16
    cos, sin = D.rope_tables(S, d, 10000.0)
    rng = np.random.Generator(np.random.PCG64(2))
    x = rng.standard_normal((2, S, 3, d))
    y = D.rope(x, cos, sin)
    assert np.array_equal(y[:, 0], x[:, 0])                       # position 0: identity
    h = d // 2
    assert np.allclose(x[..., :h] ** 2 + x[..., h:] ** 2, y[..., :h] ** 2 + y[..., h:] ** 2)
    assert np.allclose(D.rope(y, cos, sin, inverse=True), x)      # inverse rotation
    # complex form: (x1 + i x2) e^{i t theta^(-2j/d)}
    t, j = 5, 3
    ang = t * 10000.0 ** (-2 * j / d)
    z = (x[0, t, 1, j] + 1j * x[0, t, 1, j + h]) * np.exp(1j * ang)
    assert abs(z.real - y[0, t, 1, j]) < 1e-12 and abs(z.imag - y[0, t, 1, j + h]) < 1e-12


def test_attention_special_cases_and_gqa():
    rng = np.random.Generator(np.random.PCG64(4))
    B, S, H, Hkv, d = 2, 6, 4, 2, 8
    q = rng.standard_normal((B, S, H, d))
    k = rng.standard_normal((B, S, Hkv, d))
    v = rng.standard_normal((B, S, Hkv, d))
    o, P = D.attention(q, k, v, H // Hkv)
    for h in range(H):
        assert np.allclose(o[:, 0, h], v[:, 0, h // 2])           # causal: row 0 sees key 0 only
    assert np.allclose(np.triu(P[0, 0], 1), 0) and np.allclose(P.sum(-1), 1)
    o0, _ = D.attention(np.zeros_like(q), k, v, H // Hkv)         # q = 0: uniform over the prefix
    for t in range(S):
        assert np.allclose(o0[:, t, 1], v[:, : t + 1, 0].mean(axis=1))
    kr, vr = np.repeat(k, 2, axis=2), np.repeat(v, 2, axis=2)     # grouped == repeated heads
    o2, _ = D.attention(q, kr, vr, 1)
    assert np.allclose(o, o2)


def test_attention_gradient_by_finite_differences():
    rng = np.random.Generator(np.random.PCG64(5))
    B, S, H, Hkv, d = 1, 5, 4, 2, 4
    q, k, v = (rng.standard_normal((B, S, n, d)) for n in (H, Hkv, Hkv))
    do = rng.standard_normal((B, S, H, d))
    o, P = D.attention(q, k, v, 2)
    dq, dk, dv = D.attention_bwd(do, q, k, v, P, 2)
    e = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for idx in ((0, 4, 1, 2), (0, 2, 0, 0)):
            if idx[2] >= arr.shape[2]:
                continue
            old = arr[idx]
            arr[idx] = old + e
            lp = np.sum(do * D.attention(q, k, v, 2)[0])
            arr[idx] = old - e
            lm = np.sum(do * D.attention(q, k, v, 2)[0])
            arr[idx] = old
            assert abs((lp - lm) / (2 * e) - grad[idx]) < 1e-6


def test_cross_entropy_uniform_and_against_logsumexp():
    V = 1000
    loss, g = D.cross_entropy(np.zeros((4, V)), np.array([1, 2, 3, 999]))
    assert abs(loss - math.log(V)) < 1e-12
    assert np.allclose(g.sum(axis=1), 0)
    rng = np.random.Generator(np.random.PCG64(6))
    z = rng.standard_normal((5, 37)) * 3
    t = rng.integers(0, 37, size=5)
    loss, g = D.cross_entropy(z, t)
    ref = np.mean(logsumexp(z, axis=1) - z[np.arange(5), t])
    assert abs(loss - ref) < 1e-12
    e = 1e-6
    zp, zm = z.copy(), z.copy()
    zp[2, 7] += e
    zm[2, 7] -= e
    assert abs((D.cross_entropy(zp, t)[0] - D.cross_entropy(zm, t)[0]) / (2 * e) - g[2, 7]) < 1e-8


def test_swiglu_gradient():
    rng = np.random.Generator(np.random.PCG64(7))
    g, u, ds = (rng.standard_normal(6) * 2 for _ in range(3))
    dg, du = D.swiglu_bwd(ds, g, u)
    e = 1e-6
    assert np.allclose((D.silu(g + e) * u - D.silu(g - e) * u) / (2 * e) * ds, dg, atol=1e-8)
    assert np.allclose(D.silu(g) * ds, du)
    assert D.silu(np.array(0.0)) == 0.0


def test_adamw_first_step_closed_form():
    p = np.array([0.5, -1.0, 2.0])
    g = np.array([0.1, -0.3, 0.0])
    lr, wd, eps = 1e-3, 0.01, 1e-8
    p1, m, v = D.adamw(p, g, np.zeros(3), np.zeros(3), 1, lr, wd=wd, eps=eps)
    assert np.allclose(p1, p * (1 - lr * wd) - lr * g / (np.abs(g) + eps))


def test_bf16_rounding_points():
    """The rounded step stays close to the exact one and rounds where stated."""
    cfg = _cfg()
    P = _params(cfg)
    ids, tg = _batch(cfg)
    le, _, _ = D.forward(P, ids, tg, cfg, exact=True)
    lr_, logits, cache = D.forward(P, ids, tg, cfg, exact=False)
    assert abs(le - lr_) < 0.05 * abs(le)
    for x in (logits, cache["hn"], cache["layers"][0]["n1"], cache["layers"][1]["sw"]):
        assert np.array_equal(D.bf16(x), x)


# ---- preference step (DPO) ----------------------------------------------------------

def _pref_batch(cfg, pairs=2, S=10, prompt=4, seed=8, share_prompt=True):
    """Chosen/rejected sequences (sharing a prompt unless told otherwise);
    mask = response targets."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = rng.integers(0, cfg.vocab, size=(2 * pairs, S + 1))
    for p in range(pairs if share_prompt else 0):
        ids[2 * p + 1, :prompt] = ids[2 * p, :prompt]
    mask = np.zeros((2 * pairs, S))
    mask[:, prompt - 1:] = 1.0
    return ids[:, :-1].copy(), ids[:, 1:].copy(), mask


def test_token_nll_against_logsumexp():
    rng = np.random.Generator(np.random.PCG64(12))
    z = rng.standard_normal((6, 50)) * 2
    t = rng.integers(0, 50, size=6)
    assert np.allclose(D.token_nll(z, t), logsumexp(z, axis=1) - z[np.arange(6), t], atol=1e-13)


def test_dpo_loss_closed_form_and_coefficients():
    """One pair of length 2: delta = beta*((lp_c - lr_c) - (lp_r - lr_r)) and
    L = log(1 + e^-delta); the coefficients are dL/d(masked nll sums)."""
    beta = 0.1
    nll_p = np.array([1.0, 2.0, 0.5, 3.0])
    nll_r = np.array([1.5, 1.5, 1.0, 1.0])
    mask = np.array([0.0, 1.0, 1.0, 1.0])
    lp_c, lp_r = -2.0, -3.5
    lr_c, lr_r = -1.5, -2.0
    delta = beta * ((lp_c - lr_c) - (lp_r - lr_r))
    loss, coef = D.dpo_loss(nll_p, nll_r, mask, 2, beta)
    assert abs(loss - math.log1p(math.exp(-delta))) < 1e-15
    e = 1e-7
    for s in range(2):
        bump = np.zeros(4)
        bump[2 * s + 1] = e              # a masked-in token of sequence s
        fd = (D.dpo_loss(nll_p + bump, nll_r, mask, 2, beta)[0]
              - D.dpo_loss(nll_p - bump, nll_r, mask, 2, beta)[0]) / (2 * e)
        assert abs(fd - coef[s]) < 1e-9, (s, fd, coef[s])
    # a policy that favours the chosen answer more than the reference does: loss < ln 2
    assert delta > 0 and loss < math.log(2)


def test_dpo_zero_adapters_gives_ln2_and_no_dA():
    """B = 0 makes the policy equal the reference: delta = 0, L = ln 2 exactly,
    and dA vanishes while dB does not ("Soup layer-streamed NF4 training
    measured", section 2.5: with B = 0 the A gradient is structurally zero)."""
    cfg = _cfg()
    P = _params(cfg, b_scale=0.0)
    ids, tg, mask = _pref_batch(cfg)
    loss, g, _ = D.dpo_step(P, ids, tg, mask, cfg, beta=0.1, exact=True)
    assert abs(loss - math.log(2)) < 1e-15
    for (l, p), (dA, dB) in g["lora"].items():
        assert np.all(dA == 0) and np.any(dB != 0), (l, p)


@pytest.mark.parametrize("share_prompt", [True, False])
def test_dpo_finite_differences(share_prompt):
    """With distinct prompts the masked-out prompt tokens would contribute if
    the mask were ignored (a shared prompt cancels between chosen and
    rejected), so both layouts are checked."""
    cfg = _cfg()
    P = _params(cfg)
    ids, tg, mask = _pref_batch(cfg, share_prompt=share_prompt)
    beta = 0.5
    loss, g, _ = D.dpo_step(P, ids, tg, mask, cfg, beta, exact=True)
    rng = np.random.Generator(np.random.PCG64(13))
    eps = 1e-5
    for (l, p), (dA, dB) in g["lora"].items():
        a, b = P.lora[l][p]
        for arr, grad in ((a, dA), (b, dB)):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            old = arr[idx]
            arr[idx] = old + eps
            lp_ = D.dpo_step(P, ids, tg, mask, cfg, beta, exact=True)[0]
            arr[idx] = old - eps
            lm_ = D.dpo_step(P, ids, tg, mask, cfg, beta, exact=True)[0]
            arr[idx] = old
            fd = (lp_ - lm_) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-8 + 1e-4 * abs(fd), (l, p, idx, fd, grad[idx])


def test_slot_aliasing_shows_in_gradients_only():
    """The pages' slot-aliasing bug ("Fine-Tune 8B Models on 4GB VRAM: Soup's
    Layer Streaming", failure records: forward exact, gradients silently wrong)
    planted in the oracle: with two slots, a copy that lands in a slot before
    its last reader finished hands layer l's backward the weights of layer
    l - 2 (the layer the backward sweep prefetches into that slot). The
    forward never sees it, so logits and loss are unchanged; every adapter
    gradient at or below the first aliased layer moves far beyond the bars
    the streamed == resident (0.0) and oracle (2e-2) comparisons use."""
    cfg = _cfg(layers=4)
    P = _params(cfg)
    ids, tg = _batch(cfg, B=2, S=12)
    loss, logits, cache = D.forward(P, ids, tg, cfg)
    good = D.backward(P, cache, cfg)
    W_alias = [P.W[l] if l < 2 else P.W[l - 2] for l in range(cfg.layers)]
    bad = D.backward(D.Params(**{**P.__dict__, "W": W_alias}), cache, cfg)
    loss2, logits2, _ = D.forward(P, ids, tg, cfg)
    assert loss2 == loss and np.array_equal(logits2, logits)
    for (l, p), (dA, dB) in good["lora"].items():
        bA, bB = bad["lora"][(l, p)]
        e = max(np.max(np.abs(bA - dA)) / np.max(np.abs(dA)), np.max(np.abs(bB - dB)) / np.max(np.abs(dB)))
        if l < 3:   # layers 3 and 2 read the wrong weights; the error flows down
            assert e > 5e-2, (l, p, e)
