"""CPU oracle for the layer-streamed NF4 + LoRA hot path.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously-correct
definition that the HIP library is checked against. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path (``layer_streamed_nf4_amd``) never imports,
links or executes anything here, and this package never imports the product:
the two share no code, tables or constants. Inputs come from ``synth``.

Sources. The pages are five web articles on the Soup fine-tuning tool's
``stream_layers`` feature. Citations name the page and the section:
  * "Soup layer-streamed NF4 training measured" (m.mzlw.cn gate walkthrough),
    sections 1.3, 2.1-2.5, 4.1-4.4, 5 -- the technical source;
  * "Fine-Tune 8B Models on 4GB VRAM: Soup's Layer Streaming"
    (tools.cooconsbit.com, English), "The Principle of Layer Streaming";
  * "Soup v0.72.4 technical analysis" (kwkr.cn), sections 2.2 and 3.1-3.3.
Where the pages are silent the published definitions they rely on are named
(QLoRA, Dettmers et al. 2023, section 3; 8-bit Optimizers via Block-wise
Quantization, Dettmers et al. 2022, section 2).

Modules:
  tables  -- the 16-entry NF4 table and the 256-entry nested (dynamic) table
  nf4     -- blockwise quantisation with double-quantised absmax, dequantisation,
             byte accounting
  linear  -- frozen-linear forward/backward with the LoRA adapter and its grads
  stack   -- the linear-stack step (per-layer math in sequence)
"""
