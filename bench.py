"""Benchmark of the streamed NF4 + LoRA linear-stack training step (placeholder)."""
import synth

LM_HEAD = {"135m": (49152, 576), "8b": (128256, 4096), "32b": (152064, 5120)}


def flops_per_token(model: str, lm_head: bool) -> int:
    """6 FLOP per frozen decoder-linear parameter per token (2 forward,
    2 recompute, 2 dL/dx; no dL/dW for a frozen base) plus, with the resident
    lm_head, 4 per lm_head parameter (2 forward, 2 dL/dx); the embedding
    lookup counts 0. Convention of the gate walkthrough, section 4.4."""
    per_layer = sum(a * b for a, b in synth.SHAPES[model].values())
    f = 6 * per_layer * synth.N_LAYERS[model]
    if lm_head:
        v, h = LM_HEAD[model]
        f += 4 * v * h
    return f


def flop_shares(model: str) -> dict:
    sh = synth.SHAPES[model]
    tot = sum(a * b for a, b in sh.values())
    return {p: a * b / tot for p, (a, b) in sh.items()}
