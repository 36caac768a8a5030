"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds random-number draws and shapes only. It does none of the
method's arithmetic: no quantisation, no rounding to the method's formats, no
products. Both the CPU oracle (``oracle/``) and the HIP path consume what it
returns; neither imports the other.

Workloads (the pages' models are stand-ins built from their shapes):
  * one 576x576 linear (SmolLM2-135M q_proj shape), M = 512 tokens;
  * the 135M-class layer: hidden 576, intermediate 1536, 9 heads x 64, 3 KV heads;
  * the 8B-class layer (Llama-3.1-8B shapes): hidden 4096, intermediate 14336,
    32 heads x 128, 8 KV heads;
  * the 32B-class layer: hidden 5120, intermediate 27648, 40 heads x 128, 8 KV heads.

Distributions (all sigmas are standard deviations): frozen weights N(0, 0.02)
fp32; LoRA A and B N(0, 0.01) fp32 (B deliberately non-zero: with B = 0 the
gradient of A is identically zero and the adapter path is not exercised);
activations x and upstream gradients dy N(0, 1), handed over as bf16 bit
patterns obtained by dropping the low 16 bits of the fp32 draw.

Seeds follow the pages' YAML seed 1234: per-tensor seed
1234 + 1000*layer + index (q,k,v,o,gate,up,down,A,B -> 0..8 per projection),
activations 1234 + 10**6 + 10*step + slot.
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 1234
PROJ = ("q", "k", "v", "o", "gate", "up", "down")
LORA_R = 16
LORA_ALPHA = 32


def _shapes(hidden, inter, heads, head_dim, kv_heads):
    kv = kv_heads * head_dim
    qd = heads * head_dim
    return {
        "q": (qd, hidden),
        "k": (kv, hidden),
        "v": (kv, hidden),
        "o": (hidden, qd),
        "gate": (inter, hidden),
        "up": (inter, hidden),
        "down": (hidden, inter),
    }


# (N_out, K_in) of each projection, PyTorch nn.Linear layout W[N_out, K_in].
SHAPES = {
    "135m": _shapes(576, 1536, 9, 64, 3),
    "8b": _shapes(4096, 14336, 32, 128, 8),
    "32b": _shapes(5120, 27648, 40, 128, 8),
}
N_LAYERS = {"135m": 30, "8b": 32, "32b": 64}
VOCAB = {"135m": 49152, "8b": 128256, "32b": 152064}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def weight_seed(layer: int, proj: str) -> int:
    return BASE_SEED + 1000 * layer + PROJ.index(proj)


def weight(layer: int, proj: str, n_out: int, k_in: int, sigma: float = 0.02) -> np.ndarray:
    """Frozen base weight W[n_out, k_in] ~ N(0, sigma) as float32."""
    g = _rng(weight_seed(layer, proj))
    return g.standard_normal((n_out, k_in), dtype=np.float32) * np.float32(sigma)


def lora_pair(layer: int, proj: str, n_out: int, k_in: int, r: int = LORA_R,
              sigma: float = 0.01) -> tuple[np.ndarray, np.ndarray]:
    """LoRA A[r, k_in] and B[n_out, r] ~ N(0, sigma) float32 (B non-zero)."""
    base = BASE_SEED + 1000 * layer + 10 * (PROJ.index(proj) + 1)
    a = _rng(base + 7).standard_normal((r, k_in), dtype=np.float32) * np.float32(sigma)
    b = _rng(base + 8).standard_normal((n_out, r), dtype=np.float32) * np.float32(sigma)
    return a, b


def bf16_bits_from_normal(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma) draws handed over as bf16 bit patterns (uint16), truncated."""
    f = _rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def activation(shape, step: int = 0, slot: int = 0) -> np.ndarray:
    """Activation x or upstream gradient dy as bf16 bits, N(0, 1)."""
    return bf16_bits_from_normal(shape, BASE_SEED + 10**6 + 10 * step + slot)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Reinterpret bf16 bit patterns as float32 values (exact widening)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def token_ids(n: int, vocab: int, step: int = 0) -> np.ndarray:
    return _rng(BASE_SEED + 2 * 10**6 + step).integers(0, vocab, size=n, dtype=np.int64)


# Decoder hyper-parameters of the stand-in models (shapes and constants only).
# 135m: SmolLM2-135M (llama architecture, tied embeddings); 8b: Llama-3.1-8B;
# tiny: a 2-layer model small enough for the fp64 oracle and finite differences.
DECODER = {
    "tiny": dict(hidden=128, inter=256, heads=4, kv_heads=2, head_dim=32, vocab=256, layers=2,
                 rope_theta=10000.0, eps=1e-5, tied=True),
    "135m": dict(hidden=576, inter=1536, heads=9, kv_heads=3, head_dim=64, vocab=49152, layers=30,
                 rope_theta=100000.0, eps=1e-5, tied=True),
    "8b": dict(hidden=4096, inter=14336, heads=32, kv_heads=8, head_dim=128, vocab=128256, layers=32,
               rope_theta=500000.0, eps=1e-5, tied=False),
    # 32B class (the shapes of the 32B layers above; llama definitions, no
    # projection biases)
    "32b": dict(hidden=5120, inter=27648, heads=40, kv_heads=8, head_dim=128, vocab=152064, layers=64,
                rope_theta=1000000.0, eps=1e-6, tied=False),
}
SHAPES["tiny"] = _shapes(128, 256, 4, 32, 2)
N_LAYERS["tiny"] = 2
VOCAB["tiny"] = 256


def embedding(model: str, which: str = "embed", sigma: float = 0.02) -> np.ndarray:
    """Embedding (or untied lm_head) [vocab, hidden] ~ N(0, sigma) float32."""
    c = DECODER[model]
    seed = BASE_SEED + 500_000 + (0 if which == "embed" else 1)
    return _rng(seed).standard_normal((c["vocab"], c["hidden"]), dtype=np.float32) * np.float32(sigma)


def embedding_bits(model: str, which: str = "embed", sigma: float = 0.02) -> np.ndarray:
    """The same table handed over as bf16 bit patterns (uint16, truncated):
    embeddings and lm_head are stored in bf16."""
    f = embedding(model, which, sigma)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def norm_weight(model: str, layer: int, which: str, sigma: float = 0.02) -> np.ndarray:
    """RMSNorm weight [hidden] ~ N(1, sigma) float32 (which: attn, mlp, final)."""
    c = DECODER[model]
    seed = BASE_SEED + 600_000 + 10 * layer + ("attn", "mlp", "final").index(which)
    return (1.0 + _rng(seed).standard_normal(c["hidden"], dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def token_batch(model: str, batch: int, seq: int, step: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Token ids and next-token targets [batch, seq], uniform in [0, vocab)."""
    g = _rng(BASE_SEED + 700_000 + step)
    v = DECODER[model]["vocab"]
    ids = g.integers(0, v, size=(batch, seq + 1), dtype=np.int64)
    return ids[:, :-1].copy(), ids[:, 1:].copy()


def preference_batch(model: str, pairs: int, seq: int, prompt: int, step: int = 0):
    """Chosen/rejected sequences for a preference step: 2 * pairs rows of seq
    tokens ordered chosen, rejected per pair; the two rows of a pair share
    their first `prompt` tokens and draw their responses independently.
    Returns ids, next-token targets [2 * pairs, seq] and the response mask
    (fp32: 1 where the target is a response token)."""
    g = _rng(BASE_SEED + 800_000 + step)
    v = DECODER[model]["vocab"]
    full = g.integers(0, v, size=(2 * pairs, seq + 1), dtype=np.int64)
    full[1::2, :prompt] = full[0::2, :prompt]
    mask = np.zeros((2 * pairs, seq), dtype=np.float32)
    mask[:, max(prompt - 1, 0):] = 1.0
    return full[:, :-1].copy(), full[:, 1:].copy(), mask
