"""Pins for the oracle's frozen-linear + LoRA forward/backward (CPU only).

Pinned against: a brute-force triple loop, fp64 central finite differences of
L = <dy, y> (exact for this bilinear map up to rounding), the structural
zeros the pages point out (gate walkthrough, section 2.5: B = 0 makes dL/dA
vanish), the s = 0 reduction to a plain product, and non-zero adapter grads in
every layer of a stack (section 2.2, check 2).
"""
import numpy as np
import pytest

import synth
from oracle import linear, nf4, stack


def _tiny(seed, m=3, k=5, n=4, r=2):
    g = np.random.Generator(np.random.PCG64(seed))
    return (g.standard_normal((m, k)), g.standard_normal((n, k)), g.standard_normal((r, k)),
            g.standard_normal((n, r)), g.standard_normal((m, n)))


def test_forward_brute_force():
    x, w, a, b, _ = _tiny(0)
    s = 2.0
    y, u = linear.forward(x, w, a, b, s)
    m, k = x.shape
    n, r = b.shape
    for i in range(m):
        for j in range(n):
            base = sum(x[i, t] * w[j, t] for t in range(k))
            lora = sum(sum(x[i, t] * a[q, t] for t in range(k)) * b[j, q] for q in range(r))
            assert abs(y[i, j] - (base + s * lora)) < 1e-12


@pytest.mark.parametrize("seed", [1, 2])
def test_backward_finite_differences(seed):
    x, w, a, b, dy = _tiny(seed)
    s = 2.0
    g = linear.backward(x, dy, w, a, b, s)
    h = 1e-6

    def fd(arr, name):
        out = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = linear.loss(x, dy, w, a, b, s)
            arr[idx] = keep - h
            lm = linear.loss(x, dy, w, a, b, s)
            arr[idx] = keep
            out[idx] = (lp - lm) / (2 * h)
        return out

    assert np.allclose(g["dx"], fd(x, "x"), atol=1e-7)
    assert np.allclose(g["dA"], fd(a, "a"), atol=1e-7)
    assert np.allclose(g["dB"], fd(b, "b"), atol=1e-7)
    # du is the gradient w.r.t. u = x A^T
    assert np.allclose(g["du"], s * dy @ b)


def test_structural_zeros_and_plain_case():
    x, w, a, b, dy = _tiny(3)
    g = linear.backward(x, dy, w, a, np.zeros_like(b), 2.0)
    assert np.all(g["dA"] == 0) and np.any(g["dB"] != 0)
    g = linear.backward(x, dy, w, np.zeros_like(a), b, 2.0)
    assert np.all(g["dB"] == 0)
    y0, _ = linear.forward(x, w)
    y1, _ = linear.forward(x, w, a, b, 0.0)
    assert np.array_equal(y0, y1)
    assert np.array_equal(linear.backward(x, dy, w)["dx"], dy @ w)


def test_rel_err_metric():
    ref = np.array([1.0, -4.0, 2.0])
    assert linear.rel_err(ref + np.array([0, 0.02, 0]), ref) == pytest.approx(0.005)


def test_adapter_grads_nonzero_in_every_layer():
    # a 4-layer stack of small projections, LoRA on q and v
    shapes = {p: (64, 64) for p in stack.PROJ}
    m = 16
    targets = ("q", "v")

    def weights_of(i):
        return {p: nf4.bf16_to_f32(nf4.dequantize_bf16(nf4.quantize(synth.weight(i, p, *shapes[p]))))
                for p in stack.PROJ}

    def inputs_of(i):
        return {p: synth.bf16_bits_to_f32(synth.activation((m, shapes[p][1]), 0, 10 * i + j))
                for j, p in enumerate(stack.PROJ)}

    def grads_of(i):
        return {p: synth.bf16_bits_to_f32(synth.activation((m, shapes[p][0]), 1, 10 * i + j))
                for j, p in enumerate(stack.PROJ)}

    def lora_of(i):
        return {p: synth.lora_pair(i, p, *shapes[p]) for p in targets}

    res = stack.stack_step(4, weights_of, inputs_of, grads_of, lora_of, targets, 2.0)
    for layer in res:
        for p in targets:
            assert np.count_nonzero(layer[p]["dA"]) == layer[p]["dA"].size
            assert np.count_nonzero(layer[p]["dB"]) == layer[p]["dB"].size
        assert "dA" not in layer["k"]
