"""The linear-stack training step, as plain per-layer math in sequence.

TEST INFRASTRUCTURE (see oracle/__init__.py).

Streaming is a schedule, not new math (gate walkthrough, section 2.2: streamed
and resident NF4 agree to 0.0 on logits and on a 25-step loss curve, and the
buffer count n=2 vs n=3 changes nothing). So the oracle of a streamed stack is
the same per-layer computation run layer by layer: a forward sweep over
layers 0..L-1 and a backward sweep over L-1..0 in which each layer is first
recomputed (gradient checkpointing is forced by streaming; English article,
"The Principle of Layer Streaming") and then differentiated.

The linear stack keeps exactly the work the pages' FLOP convention counts
(section 4.4: 2 forward + 2 recompute + 2 dL/dx per decoder-linear weight and
token): per layer, the seven frozen projections q, k, v, o, gate, up, down at
their real shapes, each fed a seeded input x and a seeded upstream gradient
dy, with LoRA on the target projections. Attention, norms and activations sit
between the projections in a full decoder and are not part of this stack.
"""
from __future__ import annotations

from . import linear, nf4

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


def layer_step(weights, inputs, grads, lora, targets, scale):
    """One layer: forward (= recompute) and backward of the seven projections.

    weights[p]: dequantised W' values [N_out, K_in]; inputs[p]: x [M, K_in];
    grads[p]: dy [M, N_out]; lora[p]: (A, B) for p in targets.
    Returns {p: {"y", "dx", "dA", "dB"}} in fp64.
    """
    out = {}
    for p in PROJ:
        a, b = lora[p] if p in targets else (None, None)
        s = scale if p in targets else 0.0
        y, _ = linear.forward(inputs[p], weights[p], a, b, s)
        g = linear.backward(inputs[p], grads[p], weights[p], a, b, s)
        g["y"] = y
        out[p] = g
    return out


def stack_step(n_layers, weights_of, inputs_of, grads_of, lora_of, targets, scale):
    """All layers; the backward order does not change any per-layer value."""
    return [layer_step(weights_of(i), inputs_of(i), grads_of(i), lora_of(i), targets, scale)
            for i in range(n_layers)]


def layer_shard_payload(shapes) -> int:
    """Streamed bytes of one layer: the sum of its seven tensors' payloads."""
    return sum(nf4.payload_bytes(*shapes[p]) for p in PROJ)
