"""Pins for the shapes and the FLOP convention the measurement uses (CPU only).

The gate walkthrough (section 4.4) fixes the numerator: 6 FLOP per frozen
decoder-linear parameter and token (2 forward + 2 recompute + 2 dL/dx), 4 per
lm_head parameter, 0 for the embedding lookup, and prints 43.98 GFLOP/token
for the 8B run with per-projection FLOP shares; section 5 prints the true
SmolLM2-135M parameter count. Reproducing those numbers from our shapes pins
both the shapes and the accounting.
"""
import bench
import synth


def test_135m_parameter_count(golden):
    hidden, vocab, layers = 576, synth.VOCAB["135m"], synth.N_LAYERS["135m"]
    linear = sum(a * b for a, b in synth.SHAPES["135m"].values())
    assert linear == 3_538_944
    # tied embedding + per layer (linears + two RMSNorm weights) + final norm
    total = vocab * hidden + layers * (linear + 2 * hidden) + hidden
    assert total == golden["params_135m_true"]["value"]


def test_8b_flops_per_token(golden):
    f = bench.flops_per_token("8b", lm_head=True)
    assert round(f / 1e9, 2) == golden["gflop_per_token_8b"]["value"]
    shares = bench.flop_shares("8b")
    g = golden["flop_shares_8b_pct"]
    assert round(100 * (shares["q"] + shares["o"]), 1) == g["q_o"]
    assert round(100 * (shares["k"] + shares["v"]), 1) == g["k_v"]
    assert round(100 * (shares["gate"] + shares["up"]), 1) == g["gate_up"]
    assert round(100 * shares["down"], 1) == g["down"]
    for tok_s, tflops in golden["tflops_from_tok_s_8b"]["cases"]:
        assert round(tok_s * f / 1e12, 2) == tflops


def test_linear_stack_flops():
    # without the resident lm_head: 6 x decoder-linear params
    f = bench.flops_per_token("8b", lm_head=False)
    assert f == 6 * 32 * 218_103_808
