"""Benchmark: streamed NF4 + LoRA training step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3] [--gpus 1]

Workload (default, 8B-shaped, batch 1 x seq 512): the training step of a
llama decoder of Llama-3.1-8B shape (32 layers, hidden 4096, 32 heads over 8
KV heads, vocab 128256) whose seven projections per layer (q 4096x4096, k/v
1024x4096, o 4096x4096, gate/up 14336x4096, down 4096x14336) are NF4
double-quant shards in pinned host memory, streamed through a 2-slot device
pool by a side copy stream; embedding and lm_head resident in bf16; LoRA r16
alpha32 on q and v; AdamW on the adapters. One step = embedding, a forward
sweep over the 32 layers (prefetching i+1) keeping only each layer's input,
lm_head and cross-entropy, a backward sweep (prefetching i-1) that recomputes
each layer and differentiates it, and the optimiser update. The linear stack
alone (the seven projections per layer with seeded inputs and upstream
gradients, no attention/norms/head) is timed beside it. Inputs are seeded
synthetic tensors: W ~ N(0,0.02), embeddings N(0,0.02) bf16, norm weights
N(1,0.02), token ids uniform, A, B ~ N(0,0.01); the pages' real checkpoints
and data are not available and these shapes stand in for them.

Prints one JSON line. value = streamed tokens/s of the decoder step (B*S per
step time); extra fields carry the resident run, the step's achieved TFLOP/s
against the bf16 MFMA peak (the pages' convention: 6 FLOP per frozen linear
weight and token -- 2 forward, 2 recompute, 2 dL/dx -- plus 4 per lm_head
weight; attention and LoRA FLOPs not counted), the H2D rate against the host
link, the roofline of the dominant kernel (the forward fused dequant GEMM)
timed live with HIP events inside the decoder step, the linear stack, and
the CPU oracle timed on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import synth

LM_HEAD = {"135m": (49152, 576), "8b": (128256, 4096), "32b": (152064, 5120)}
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
HOST_LINK_GBS = 63.0          # PCIe Gen5 x16, one direction, theoretical

CONFIGS = {
    # id: (model, batch, seq, lora targets, slots, reference pass)
    2: ("135m", 1, 512, ("q", "v"), 2, None),
    3: ("8b", 1, 512, ("q", "v"), 2, None),
    4: ("8b", 4, 512, ("q", "k", "v", "o", "gate", "up", "down"), 4, None),
    # preference step: 2 chosen/rejected pairs x seq 512 through 32B-class layers
    # (251.5 MB each), a reference pass with the adapters off plus the policy step
    5: ("32b", 4, 512, ("q", "v"), 2, "separate"),
}


def flops_per_token(model: str, lm_head: bool, reference: bool = False) -> int:
    """6 FLOP per frozen decoder-linear parameter per token (2 forward,
    2 recompute, 2 dL/dx; no dL/dW for a frozen base) plus, with the resident
    lm_head, 4 per lm_head parameter (2 forward, 2 dL/dx); the embedding
    lookup counts 0. Convention of the gate walkthrough, section 4.4. A
    preference step adds the reference forward: 8 per decoder-linear and 6 per
    lm_head parameter."""
    per_layer = sum(a * b for a, b in synth.SHAPES[model].values())
    f = (8 if reference else 6) * per_layer * synth.N_LAYERS[model]
    if lm_head:
        v, h = LM_HEAD[model]
        f += (6 if reference else 4) * v * h
    return f


def executed_flops_per_token(model: str, decoder: bool, reference: bool = False) -> int:
    """The frozen-linear and lm_head FLOPs the step actually executes (same
    counting rules as flops_per_token). The decoder's recompute skips the down
    and o products (their outputs h_{i+1} and the mid-layer residual are kept
    from the forward and the backward reads nothing else of them) and the
    whole last layer (its body is kept from the forward); the linear stack
    recomputes every projection of every layer."""
    if not decoder:
        return flops_per_token(model, False, reference)
    sh = synth.SHAPES[model]
    n_layers = synth.N_LAYERS[model]
    p_lin = sum(a * b for a, b in sh.values())
    p_skip = sh["down"][0] * sh["down"][1] + sh["o"][0] * sh["o"][1]
    v, h = LM_HEAD[model]
    f = 2 * p_lin * n_layers + 2 * (p_lin - p_skip) * (n_layers - 1) + 2 * p_lin * n_layers + 4 * v * h
    if reference:
        f += 2 * p_lin * n_layers + 2 * v * h
    return f


def flop_shares(model: str) -> dict:
    sh = synth.SHAPES[model]
    tot = sum(a * b for a, b in sh.values())
    return {p: a * b / tot for p, (a, b) in sh.items()}


def lora_flops_per_token(model: str, targets) -> int:
    """LoRA forward + recompute + backward per token, reported apart from the
    frozen-base numerator: u = xA^T and y += s u B^T (2 r (k+n)) twice, du, dB,
    dA and the du.A term of dx (4 r (k+n))."""
    sh = synth.SHAPES[model]
    r = synth.LORA_R
    return synth.N_LAYERS[model] * sum(8 * r * (sh[p][0] + sh[p][1]) for p in targets)


def gemm_source_hash() -> str:
    """Hash of the fused-GEMM source: counters taken on another build do not apply."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "layer_streamed_nf4_amd", "csrc", "gemm.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel_src_hash: str, spec: str):
    """HBM bytes per launch of the dominant kernel from the committed PMC summary,
    if it was taken on this exact GEMM source and this shape (`fwd:N:K:M`, or `fwd:N1+N2:K:M` for a grouped launch);
    else None."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", "gemm_fwd_gate_up_8b_m512_pmc.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("<!--") and "=" in line:
            k, v = line.strip("<!-> \n").split("=", 1)
            fields[k.strip()] = v.strip()
    if fields.get("gemm_src_sha256_16") != kernel_src_hash or fields.get("spec") != spec:
        return None
    try:
        return int(float(fields["fetch_bytes"]) + float(fields["write_bytes"]))
    except (KeyError, ValueError):
        return None


def profile_gemm(spec: str, reps: int) -> None:
    """Run one fused GEMM shape `fwd:N:K:M` or `bwd:N:K:M` (resident weight)
    `reps` times, then a 64 MiB device copy whose FETCH/WRITE counters give the
    scale of the memory counters. `fwd:N1+N2:K:M` runs the grouped forward of
    weights of N1 and N2 outputs reading one input; `bwd:N1+N2:K:M` the
    grouped backward (one contraction over both weights, each with its own dy).
    Used under rocprofv3."""
    import torch
    import layer_streamed_nf4_amd as L
    direction, ns, k, M = spec.split(":")
    ns = [int(x) for x in ns.split("+")]
    k, M = int(k), int(M)
    dev = "cuda"
    s = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device=dev)
    g.manual_seed(synth.BASE_SEED)
    descs, end = [], 0
    for n in ns:
        descs.append(L.nf4s_tensor_layout(n, k, end))
        end = descs[-1].end
    shard = torch.zeros(end, dtype=torch.uint8, device=dev)
    for n, d in zip(ns, descs):
        w = torch.randn((n, k), generator=g, device=dev) * 0.02
        wq = torch.empty(max(256, L.nf4s_workspace_bytes(L.OP_QUANTIZE, 0, n, k)), dtype=torch.uint8,
                         device=dev)
        L.nf4_quantize_shard(w.data_ptr(), L.DTYPE_F32, n, k, shard.data_ptr(), d, None,
                             wq.data_ptr(), wq.numel(), s)
    bwd = direction == "bwd"
    n = ns[0]
    outs = [torch.empty((M, k if bwd else n_), dtype=torch.bfloat16, device=dev) for n_ in ns]
    if len(ns) > 1:
        ws_bytes = (L.grouped_bwd_workspace_bytes(ns, k, M) if bwd
                    else L.grouped_workspace_bytes(ns, k, M))
    else:
        op = L.OP_LINEAR_BWD_PACKED if bwd else L.OP_LINEAR_FWD_PACKED
        ws_bytes = L.nf4s_workspace_bytes(op, M, n, k)
    ws = torch.zeros(max(256, ws_bytes), dtype=torch.uint8, device=dev)
    # one packed input per weight of a grouped backward (its own dy), else one
    aps = []
    for n_ in (ns if bwd else ns[:1]):
        K = n_ if bwd else k
        a = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        ap = torch.empty(L.nf4s_packed_activation_bytes(M, K), dtype=torch.uint8, device=dev)
        L.nf4s_pack_activation(a.data_ptr(), M, K, ap.data_ptr(), ap.numel(), s)
        aps.append(ap)
    ap = aps[0]
    for _ in range(reps):
        if bwd and len(ns) > 1:
            L.streamed_linear_bwd_grouped(shard.data_ptr(), descs, [x.data_ptr() for x in aps], M,
                                          outs[0].data_ptr(), [None] * len(ns), [None] * len(ns), 0,
                                          ws.data_ptr(), ws.numel(), s)
        elif bwd:
            L.streamed_linear_bwd_packed(shard.data_ptr(), descs[0], ap.data_ptr(), M,
                                         outs[0].data_ptr(), None, None, 0, ws.data_ptr(),
                                         ws.numel(), s)
        elif len(ns) > 1:
            L.streamed_linear_fwd_grouped(shard.data_ptr(), descs, ap.data_ptr(), M,
                                          [o.data_ptr() for o in outs], None, None, 0, 0.0,
                                          ws.data_ptr(), ws.numel(), s)
        else:
            L.streamed_linear_fwd_packed(shard.data_ptr(), descs[0], ap.data_ptr(), M,
                                         outs[0].data_ptr(), None, None, 0, 0.0, ws.data_ptr(),
                                         ws.numel(), s)
    torch.cuda.synchronize()
    src = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"profiled {spec} x{reps}; gemm source {gemm_source_hash()}", flush=True)


def _cpu_threads() -> int:
    """Threads for the oracle's BLAS: the CPUs this process may run on, capped
    by OMP_NUM_THREADS where the environment sets the machine's share."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, n)


def _cpu_baseline(model: str, M: int, targets) -> dict:
    """The oracle, as it stands, on one full layer of the step (dequantise the
    seven tensors, then forward and backward of the seven projections with the
    adapter), scaled to tokens/s of the whole stack. Quantisation is offline
    and not timed."""
    import numpy as np

    from oracle import nf4 as onf4, stack as ostack
    cores = _cpu_threads()
    sh = synth.SHAPES[model]
    q = {p: onf4.quantize(synth.weight(0, p, *sh[p])) for p in ostack.PROJ}
    lora = {p: synth.lora_pair(0, p, *sh[p]) for p in targets}
    xs = {p: onf4.bf16_to_f32(synth.activation((M, sh[p][1]), 0, j)) for j, p in enumerate(ostack.PROJ)}
    dys = {p: onf4.bf16_to_f32(synth.activation((M, sh[p][0]), 0, 50 + j))
           for j, p in enumerate(ostack.PROJ)}
    t0 = time.perf_counter()
    w = {p: onf4.bf16_to_f32(onf4.dequantize_bf16(q[p])) for p in ostack.PROJ}
    ostack.layer_step(w, xs, dys, lora, targets, synth.LORA_ALPHA / synth.LORA_R)
    dt = time.perf_counter() - t0
    n_layers = synth.N_LAYERS[model]
    return {"value": M / (dt * n_layers), "unit": "tok/s", "cores": int(cores), "kind": "oracle",
            "sample": f"one {model} layer (7 projections, M={M}, LoRA on {'/'.join(targets)}): "
                      f"dequantise + fp64 forward/backward in {dt:.2f} s, scaled x{n_layers} layers"}


def _cpu_baseline_decoder(model: str, batch: int, seq: int, targets, preference=None) -> dict:
    """The decoder oracle, as it stands, on a bounded sample of the same step:
    the fp64 forward and backward of the head alone (embedding, final norm,
    lm_head, cross-entropy; no layer) and of one full layer plus the head,
    both timed, and the dequantisation of the layer's q tensor, timed and
    scaled to the layer's parameters. The step is the head plus L layers.
    A preference step (oracle.decoder.dpo_step: reference forward, policy
    forward and backward) is sampled on one pair of 128-token sequences and
    scaled to the step's tokens (the sample's work is linear in tokens but
    for the attention, which is small at these lengths).
    The oracle caches activations
    instead of recomputing; weight values do not change its time, so the
    sample uses the seeded fp32 weights and one table for embedding and
    lm_head."""
    import numpy as np

    from oracle import decoder as odec, nf4 as onf4
    cores = _cpu_threads()
    c = dict(synth.DECODER[model])
    c.pop("tied")
    n_layers = c["layers"]
    sh = synth.SHAPES[model]
    qq = onf4.quantize(synth.weight(0, "q", *sh["q"]))
    t0 = time.perf_counter()
    onf4.dequantize_bf16(qq)
    p_layer = sum(a * b for a, b in sh.values())
    t_deq = (time.perf_counter() - t0) * p_layer / (sh["q"][0] * sh["q"][1])
    W = [{p: synth.weight(0, p, *sh[p]).astype(np.float64) for p in odec.PROJ}]
    E = synth.bf16_bits_to_f32(synth.embedding_bits(model)).astype(np.float64)
    lora = [{p: tuple(a.astype(np.float64) for a in synth.lora_pair(0, p, *sh[p])) for p in targets}]
    norm = lambda w: synth.norm_weight(model, 0, w).astype(np.float64)  # noqa: E731
    if preference:
        s_seq = min(seq, 128)
        ids, tg, mask = synth.preference_batch(model, 1, s_seq, s_seq // 4)
        scale_tokens = (batch * seq) / ids.size
    else:
        ids, tg = synth.token_batch(model, batch, seq)
        scale_tokens = 1.0

    def timed(layers):
        cfg = odec.Config(**{**c, "layers": layers}, targets=tuple(targets))
        P = odec.Params(embed=E, lm_head=E, w_attn=[norm("attn")] * layers,
                        w_mlp=[norm("mlp")] * layers, w_final=norm("final"), W=W[:layers],
                        lora=lora[:layers])
        t0 = time.perf_counter()
        if preference:
            odec.dpo_step(P, ids, tg, mask, cfg, 0.1)
        else:
            _, _, cache = odec.forward(P, ids, tg, cfg)
            odec.backward(P, cache, cfg)
        return (time.perf_counter() - t0) * scale_tokens

    t_head = timed(0)
    t_one = timed(1)
    t_layer = t_one - t_head + t_deq
    t_step = t_head + n_layers * t_layer
    M = batch * seq
    what = (f"DPO step sampled on 1 pair x {ids.shape[1]} tokens, scaled x{scale_tokens:g} to "
            f"B{batch} S{seq}" if preference else f"B{batch} S{seq}")
    return {"value": M / t_step, "unit": "tok/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"{model} decoder, {what} (LoRA {'/'.join(targets)}), fp64 "
                      f"forward + backward: head alone {t_head:.2f} s, one layer + head "
                      f"{t_one:.2f} s; layer dequantisation {t_deq:.2f} s (scaled from q); "
                      f"step = head + {n_layers} x layer = {t_step:.1f} s"}


def _time_sharder(L, torch, sh) -> dict:
    """nf4_quantize_shard on one gate-shaped tensor (the largest of the layer),
    HIP events over 5 calls after one warm-up. Algorithmic bytes: the fp32
    weight read once (4 B/param) and the payload written (0.516 B/param);
    HBM-bound, offline (gate walkthrough, section 2.1)."""
    n, k = sh["gate"]
    dev = "cuda"
    s = torch.cuda.current_stream().cuda_stream
    w = torch.randn((n, k), device=dev) * 0.02
    d = L.nf4s_tensor_layout(n, k)
    out = torch.empty(d.end, dtype=torch.uint8, device=dev)
    ws = torch.empty(L.nf4s_workspace_bytes(L.OP_QUANTIZE, 0, n, k), dtype=torch.uint8, device=dev)
    call = lambda: L.nf4_quantize_shard(w.data_ptr(), L.DTYPE_F32, n, k, out.data_ptr(), d, None,  # noqa: E731
                                        ws.data_ptr(), ws.numel(), s)
    call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 5 * 1e3
    nbytes = 4 * n * k + L.nf4_shard_bytes(n, k)
    return {"tensor": f"{n}x{k} fp32", "us": round(us, 1), "bytes": nbytes,
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 3)}


def _cpu_model() -> str | None:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _gpu_clock_and_temp() -> dict:
    """SCLK and edge/junction temperature read through rocm-smi right after
    the timed region (None where the tool or a field is unavailable)."""
    import subprocess
    out = {"sclk_mhz": None, "temperature_c": None}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showtemp", "--json"], capture_output=True,
                           text=True, timeout=30)
        data = json.loads(r.stdout[r.stdout.index("{"):])
        card = next(iter(v for k, v in data.items() if k.startswith("card")))
        for k, v in card.items():
            if k.startswith("sclk") and "speed" in k and out["sclk_mhz"] is None:
                out["sclk_mhz"] = float(str(v).strip("()Mhz").split("Mhz")[0])
            if "junction" in k.lower() and "temperature" in k.lower():
                out["temperature_c"] = float(v)
    except Exception:  # noqa: BLE001 -- reporting only
        pass
    return out


def sweep(args) -> None:
    """Where the copies hide: the 8B linear stack streamed and resident at
    batch x 512 tokens for batch 1..16 (n = 2 slots, LoRA q/v), and at batch 4
    for n = 2, 4, 8 slots. Per point: step times, copies and bytes per step,
    and the overlap efficiency (t_copy + t_compute - t_step) / min(t_copy,
    t_compute), where t_copy is the step's bytes at the same-session pinned
    H2D rate and t_compute the resident step time (the copy hides once
    t_compute >= t_copy). Batch 4 also runs with n = 3..8 slots. One JSON
    line per point."""
    import torch

    import layer_streamed_nf4_amd as L
    from layer_streamed_nf4_amd.stack import PROJ, LinearStack, ShardSet

    L.lib()
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    model = "8b"
    sh = synth.SHAPES[model]
    n_layers = synth.N_LAYERS[model]
    dev = "cuda"
    gen = torch.Generator(device=dev)

    def weight_fn(i, p):
        gen.manual_seed(synth.weight_seed(i, p))
        return torch.randn(sh[p], generator=gen, device=dev, dtype=torch.float32) * 0.02

    shards = ShardSet(sh, n_layers, weight_fn)
    host = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    devb = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    cs = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cs):
        devb.copy_(host, non_blocking=True)
        e0.record(cs)
        for _ in range(5):
            devb.copy_(host, non_blocking=True)
        e1.record(cs)
    cs.synchronize()
    h2d_peak = 5 * (256 << 20) / (e0.elapsed_time(e1) * 1e-3)
    del host, devb
    role = {"q": "attn", "k": "attn", "v": "attn", "o": "o", "gate": "mlp", "up": "mlp", "down": "down"}

    def point(batch, slots, targets):
        M = batch * 512
        gen.manual_seed(synth.BASE_SEED + 10**6 + batch)
        xs_role = {}
        for p in PROJ:
            if role[p] not in xs_role:
                xs_role[role[p]] = torch.randn((M, sh[p][1]), generator=gen, device=dev).to(torch.bfloat16)
        dys = {p: torch.randn((M, sh[p][0]), generator=gen, device=dev).to(torch.bfloat16) for p in PROJ}
        lora = []
        for i in range(n_layers):
            d = {}
            for p in targets:
                gen.manual_seed(synth.BASE_SEED + 1000 * i + 10 * (PROJ.index(p) + 1) + 7)
                d[p] = (torch.randn((synth.LORA_R, sh[p][1]), generator=gen, device=dev) * 0.01,
                        torch.randn((sh[p][0], synth.LORA_R), generator=gen, device=dev) * 0.01)
            lora.append(d)
        inputs = lambda i, p: xs_role[role[p]]
        grads = lambda i, p: dys[p]
        out = {"kind": "sweep", "model": model, "batch": batch, "seq": 512, "tokens": M,
               "slots": slots, "lora_targets": list(targets)}
        for mode in ("streamed", "resident"):
            st = LinearStack(shards, M, targets, lora, n_slots=slots, mode=mode, keep_outputs=False)
            for _ in range(max(1, args.warmup)):
                st.step(inputs, grads)
            torch.cuda.synchronize()
            c0, b0 = st.stats()
            t = time.perf_counter()
            for _ in range(args.steps):
                st.step(inputs, grads)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t) / args.steps
            c1, b1 = st.stats()
            st.close()
            out[f"{mode}_ms"] = round(dt * 1e3, 2)
            out[f"{mode}_tok_s"] = round(M / dt, 1)
            if mode == "streamed":
                out["copies_per_step"] = (c1 - c0) / args.steps
                out["h2d_bytes_per_step"] = int((b1 - b0) / args.steps)
        t_copy = out["h2d_bytes_per_step"] / h2d_peak * 1e3
        t_comp, t_step = out["resident_ms"], out["streamed_ms"]
        out["t_copy_ms_at_pinned_peak"] = round(t_copy, 2)
        out["overlap_efficiency"] = round((t_copy + t_comp - t_step) / min(t_copy, t_comp), 3)
        out["copy_hidden"] = t_comp >= t_copy
        out["pinned_peak_gbs"] = round(h2d_peak / 1e9, 2)
        print(json.dumps(out), flush=True)
        del xs_role, dys, lora
        torch.cuda.empty_cache()

    for batch in (1, 2, 4, 8, 16):
        point(batch, 2, ("q", "v"))
    for slots in (3, 4, 5, 6, 7, 8):
        point(4, slots, ("q", "v"))
    point(4, 4, PROJ)  # the pages' config 4: B4, LoRA on all seven projections, n = 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=3, choices=sorted(CONFIGS))
    ap.add_argument("--slots", type=int, default=None)
    ap.add_argument("--no-resident", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decoder", action="store_true",
                    help="time the linear stack only (no attention, norms, lm_head, optimizer)")
    ap.add_argument("--no-linear", action="store_true",
                    help="skip the linear-stack legs (decoder configurations only)")
    ap.add_argument("--profile-gemm", default=None,
                    help="only run one fused GEMM shape, e.g. fwd:14336:4096:512 (for rocprofv3)")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--sweep", action="store_true",
                    help="batch x seq and slot sweep at the 8B shapes: one JSON line per point")
    args = ap.parse_args()
    if args.profile_gemm:
        profile_gemm(args.profile_gemm, args.reps)
        return
    if args.sweep:
        sweep(args)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported (sharding across GPUs is described, not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import layer_streamed_nf4_amd as L
    from layer_streamed_nf4_amd.stack import PROJ, LinearStack, ShardSet

    L.lib()
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    model, batch, seq, targets, slots, reference = CONFIGS[args.config]
    if args.slots:
        slots = args.slots
    M = batch * seq
    sh = synth.SHAPES[model]
    n_layers = synth.N_LAYERS[model]
    dev = "cuda"
    print(f"[bench] config {args.config}: {model} x{n_layers} layers, M={M}, LoRA {targets}, "
          f"n={slots}", file=sys.stderr, flush=True)

    gen = torch.Generator(device=dev)

    def weight_fn(i, p):
        gen.manual_seed(synth.weight_seed(i, p))
        return torch.randn(sh[p], generator=gen, device=dev, dtype=torch.float32) * 0.02

    t0 = time.perf_counter()
    shards = ShardSet(sh, n_layers, weight_fn)
    print(f"[bench] sharded {n_layers} layers ({shards.layout.nbytes / 1e6:.1f} MB each) in "
          f"{time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    def lora_init(i, p):
        gen.manual_seed(synth.BASE_SEED + 1000 * i + 10 * (PROJ.index(p) + 1) + 7)
        a = torch.randn((synth.LORA_R, sh[p][1]), generator=gen, device=dev) * 0.01
        b = torch.randn((sh[p][0], synth.LORA_R), generator=gen, device=dev) * 0.01
        return a, b

    lora = [{p: lora_init(i, p) for p in targets} for i in range(n_layers)]
    gen.manual_seed(synth.BASE_SEED + 10**6)
    # the layer's dataflow: q, k, v read the normed hidden state, o the
    # attention output, gate and up the normed hidden state of the MLP, down
    # the gated product; each upstream gradient is its own tensor
    role = {"q": "attn", "k": "attn", "v": "attn", "o": "o", "gate": "mlp", "up": "mlp", "down": "down"}
    xs_role = {}
    for p in PROJ:
        if role[p] not in xs_role:
            xs_role[role[p]] = torch.randn((M, sh[p][1]), generator=gen, device=dev).to(torch.bfloat16)
    xs = {p: xs_role[role[p]] for p in PROJ}
    dys = {p: torch.randn((M, sh[p][0]), generator=gen, device=dev).to(torch.bfloat16) for p in PROJ}
    inputs = lambda i, p: xs[p]
    grads = lambda i, p: dys[p]

    # dominant kernel: the forward fused GEMM on shapes that need no split
    # (gate/up at 8B): one call = one k_gemm_fwd launch
    def plain_fwd(direction, n, k):
        return direction == "fwd" and L.nf4s_workspace_bytes(L.OP_LINEAR_FWD_PACKED, M, n, k) == 0

    def run(mode, n_slots, timed):
        st = LinearStack(shards, M, targets, lora, n_slots=n_slots, mode=mode, keep_outputs=False,
                         time_calls=plain_fwd if timed else None)
        for _ in range(args.warmup):
            st.step(inputs, grads, reference=reference)
        torch.cuda.synchronize()
        st.timed.clear()
        c0, b0 = st.stats()
        t = time.perf_counter()
        for _ in range(args.steps):
            st.step(inputs, grads, reference=reference)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t) / args.steps
        c1, b1 = st.stats()
        durs = [(n, k, s.elapsed_time(e)) for (_, n, k, s, e) in st.timed]
        st.close()
        return dt, (b1 - b0) / args.steps, (c1 - c0) / args.steps, durs

    use_decoder = model in synth.DECODER and not args.no_decoder
    # the linear stack: the streamed projections alone
    lin_s = lin_r = None
    lin_copies, lin_durs = 0, []
    if not (use_decoder and args.no_linear):
        lin_s, lin_h2d, lin_copies, lin_durs = run("streamed", slots,
                                                   not use_decoder and args.no_resident)
        print(f"[bench] linear stack streamed: {lin_s * 1e3:.1f} ms/step, {lin_copies:.0f} "
              f"copies/step", file=sys.stderr, flush=True)
        if not args.no_resident:
            lin_r, _, _, r_durs = run("resident", slots, not use_decoder)
            if not use_decoder:
                lin_durs = r_durs
            print(f"[bench] linear stack resident: {lin_r * 1e3:.1f} ms/step", file=sys.stderr,
                  flush=True)

    dec = None
    if use_decoder:
        from layer_streamed_nf4_amd.decoder import Decoder

        c = synth.DECODER[model]
        V, H = c["vocab"], c["hidden"]
        gen.manual_seed(synth.BASE_SEED + 500_000)
        embed = (torch.randn((V, H), generator=gen, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)
        if c["tied"]:
            head = embed
        else:
            gen.manual_seed(synth.BASE_SEED + 500_001)
            head = (torch.randn((V, H), generator=gen, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)
        norms = {w: [torch.from_numpy(synth.norm_weight(model, i, w)).to(dev) for i in range(n_layers)]
                 for w in ("attn", "mlp")}
        norms["final"] = torch.from_numpy(synth.norm_weight(model, 0, "final")).to(dev)
        lora_map = {(i, p): lora[i][p] for i in range(n_layers) for p in targets}
        if reference:
            # preference pairs: 2 pairs x (chosen, rejected), a shared 128-token prompt
            ids_np, tg_np, mask_np = synth.preference_batch(model, batch // 2, seq, 128)
            mask = torch.from_numpy(mask_np.reshape(-1)).to(dev)
        else:
            ids_np, tg_np = synth.token_batch(model, batch, seq)
        ids = torch.from_numpy(ids_np.reshape(-1)).to(dev)
        tgs = torch.from_numpy(tg_np.reshape(-1)).to(dev)

        def one_step(d):
            if reference:
                d.preference_step(ids, tgs, mask, beta=0.1, schedule=reference)
            else:
                d.step(ids, tgs)

        def run_dec(mode, n_slots, timed):
            d = Decoder(c, shards, embed, head, norms, lora_map, batch, seq, targets=targets,
                        n_slots=n_slots, mode=mode, time_calls=plain_fwd if timed else None)
            first = None
            for w_ in range(args.warmup):
                one_step(d)
                if w_ == 0:
                    first = d.loss.clone()   # before any optimiser update
            torch.cuda.synchronize()
            d.timed.clear()
            c0, b0 = d.stats()
            t = time.perf_counter()
            for k_ in range(args.steps):
                one_step(d)
                if first is None:            # no warm-up: the first timed step's loss
                    first = d.loss.clone()
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t) / args.steps
            c1, b1 = d.stats()
            durs = [(n, k, s_.elapsed_time(e_) / cnt) for (_, n, k, s_, e_, cnt) in d.timed
                    for _ in range(cnt)]
            loss = (float(first.item()), float(d.loss.item()))
            d.close()
            return dt, (b1 - b0) / args.steps, (c1 - c0) / args.steps, durs, loss

        # the dominant kernel is timed live in the resident run (the same
        # launches on the same shapes), so the streamed step -- the reported
        # value -- carries no timing events; without a resident run, in the
        # streamed one
        dt_s, h2d_bytes, copies, durs, loss_s = run_dec("streamed", slots, args.no_resident)
        print(f"[bench] decoder streamed: {dt_s * 1e3:.1f} ms/step, {copies:.0f} copies/step, "
              f"loss first/last step {loss_s[0]:.6f} / {loss_s[1]:.6f}", file=sys.stderr, flush=True)
        dt_r, loss_r = None, None
        if not args.no_resident:
            dt_r, _, _, durs, loss_r = run_dec("resident", slots, True)
            print(f"[bench] decoder resident: {dt_r * 1e3:.1f} ms/step, loss first/last step "
                  f"{loss_r[0]:.6f} / {loss_r[1]:.6f}", file=sys.stderr, flush=True)
        dec = dict(loss_first_step=loss_s[0], loss_last_step_streamed=loss_s[1],
                   loss_last_step_resident=None if loss_r is None else loss_r[1],
                   losses_identical=None if loss_r is None else loss_s == loss_r,
                   steps_taken=args.warmup + args.steps)
    else:
        dt_s, h2d_bytes, copies, durs, dt_r = lin_s, lin_h2d, lin_copies, lin_durs, lin_r

    peak_mem = torch.cuda.max_memory_allocated()
    gpu_state = _gpu_clock_and_temp()

    # same-session ceilings: hipBLASLt bf16 GEMM at the dominant shape, pinned H2D
    n_d, k_d = sh["gate"]
    # the decoder runs gate and up as one grouped launch over both weights:
    # the dominant launch (and its dense same-shape ceiling) has 2 x n_out
    if use_decoder:
        n_d = 2 * n_d
    a = torch.randn((M, k_d), device=dev, dtype=torch.bfloat16)
    w = torch.randn((n_d, k_d), device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, w.t())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        torch.matmul(a, w.t())
    e1.record()
    torch.cuda.synchronize()
    blas_tflops = 2 * M * n_d * k_d / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e12
    host = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    devb = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    cs = torch.cuda.Stream()
    for _ in range(2):
        with torch.cuda.stream(cs):
            devb.copy_(host, non_blocking=True)
    cs.synchronize()
    e0.record(cs)
    for _ in range(5):
        with torch.cuda.stream(cs):
            devb.copy_(host, non_blocking=True)
    e1.record(cs)
    cs.synchronize()
    h2d_peak = 5 * (256 << 20) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del host, devb
    sharder = _time_sharder(L, torch, sh)

    tokens = M
    f_tok = flops_per_token(model, lm_head=use_decoder, reference=reference is not None)
    f_lin = flops_per_token(model, lm_head=False, reference=reference is not None)
    value = tokens / dt_s
    step_tflops = f_tok * tokens / dt_s / 1e12
    f_exec = executed_flops_per_token(model, use_decoder, reference is not None)
    dom_ms = [d for (_, _, d) in durs]
    dom_flops = [2 * M * n * k for (n, k, _) in durs]
    roofline = None
    n_g, k_g = sh["gate"]
    dom_spec = f"fwd:{n_g}+{n_g}:{k_g}:{M}" if use_decoder else f"fwd:{n_g}:{k_g}:{M}"
    if dom_ms:
        avg_ms = sum(dom_ms) / len(dom_ms)
        avg_flop = sum(dom_flops) / len(dom_flops)
        ach = avg_flop / (avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic_from_profile(gemm_source_hash(), dom_spec),
                    "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                    "kernel": "k_gemm_fwd (fused NF4 dequant + bf16 MFMA, x.W'^T, 512x128 tiles, "
                              "no split)" + ("; one grouped launch = gate and up" if use_decoder else ""),
                    "spec": dom_spec,
                    "launches": len(dom_ms), "avg_us": round(avg_ms * 1e3, 2),
                    "flop_per_launch": int(avg_flop)}
    if use_decoder:
        workload = (f"decoder training step: llama {model} ({n_layers} layers, hidden {H}, "
                    f"{c['heads']} heads / {c['kv_heads']} KV heads, vocab {V}); the seven "
                    f"projections per layer streamed from pinned host as NF4 shards, embedding "
                    f"and lm_head resident bf16, checkpointed layers recomputed in the backward, "
                    f"AdamW on the adapters"
                    + (f"; DPO preference step on {batch // 2} chosen/rejected pairs, reference "
                       f"model = the same shards with adapters off ({reference} sweep)"
                       if reference else ""))
    else:
        workload = (f"linear stack: {n_layers} layers of {model} projection shapes "
                    f"(q,k,v,o,gate,up,down), streamed from pinned host, recompute in backward"
                    + (f", preference step (reference pass with adapters off, {reference})"
                       if reference else ""))
    out = {
        "metric": "streamed NF4+LoRA train tok/s, 8B layer shape seq512; % of bf16 MFMA peak",
        "value": round(value, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt_s * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights in NF4 double-quant, N(0,0.02) bf16 "
                "embeddings, N(1,0.02) norm weights, uniform token ids, N(0,0.01) LoRA A/B; "
                "shapes stand in for the pages' checkpoints and data)",
        "config": {"workload": workload,
                   "global_batch": batch, "seq_len": seq, "tokens_per_step": tokens,
                   "lora": {"r": synth.LORA_R, "alpha": synth.LORA_ALPHA, "targets": list(targets)},
                   "slots": slots, "parallelism": "single GPU"},
        "step_tflops": round(step_tflops, 2),
        "step_frac_of_mfma_peak": round(step_tflops / PEAK_BF16_TFLOPS, 4),
        "flop_per_token": f_tok,
        "executed_flop_per_token": f_exec,
        "executed_tflops": round(f_exec * tokens / dt_s / 1e12, 2),
        "lora_flop_per_token": lora_flops_per_token(model, targets),
        "resident": None if dt_r is None else {
            "tok_s": round(tokens / dt_r, 1), "ms_per_step": round(dt_r * 1e3, 3),
            "tflops": round(f_tok * tokens / dt_r / 1e12, 2),
            "executed_tflops": round(f_exec * tokens / dt_r / 1e12, 2),
            "frac_of_mfma_peak": round(f_tok * tokens / dt_r / 1e12 / PEAK_BF16_TFLOPS, 4),
            "streamed_over_resident_time": round(dt_s / dt_r, 3)},
        "h2d": {"bytes_per_step": int(h2d_bytes), "copies_per_step": copies,
                "effective_gbs": round(h2d_bytes / dt_s / 1e9, 2),
                "pinned_peak_gbs_same_session": round(h2d_peak, 2),
                "host_link_theoretical_gbs": HOST_LINK_GBS,
                # the step's bytes at the same-session pinned rate over the step time:
                # the share of the step the host link alone needs
                "host_link_frac": round(h2d_bytes / (h2d_peak * 1e9) / dt_s, 4),
                # (t_copy + t_compute - t_step) / min(t_copy, t_compute), with t_copy the
                # step's bytes at the same-session pinned rate, t_compute the resident step
                "overlap_efficiency": None if dt_r is None else round(
                    (h2d_bytes / (h2d_peak * 1e9) + dt_r - dt_s)
                    / min(h2d_bytes / (h2d_peak * 1e9), dt_r), 3)},
        "device": {"peak_memory_allocated_gb": round(peak_mem / 1e9, 3),
                   "sclk_mhz_after_timed_region": gpu_state["sclk_mhz"],
                   "junction_temperature_c_after_timed_region": gpu_state["temperature_c"]},
        "roofline": roofline,
        "sharder": sharder,
        "hipblaslt_bf16_same_shape_tflops": round(blas_tflops, 1),
        "context": "pages (NVIDIA, full model incl. attention/lm_head/optimizer): 119.6 tok/s at "
                   "3.32 GB on an RTX 3050 Laptop 4 GB, 113 tok/s on an H100 -- context only",
    }
    if use_decoder:
        out["decoder"] = dec
        out["linear_stack"] = None if lin_s is None else {
            "streamed_tok_s": round(tokens / lin_s, 1), "streamed_ms_per_step": round(lin_s * 1e3, 3),
            "resident_tok_s": None if lin_r is None else round(tokens / lin_r, 1),
            "resident_ms_per_step": None if lin_r is None else round(lin_r * 1e3, 3),
            "flop_per_token": f_lin, "copies_per_step": lin_copies}
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=_cpu_threads()):
            out["cpu_baseline"] = (_cpu_baseline_decoder(model, batch, seq, targets, reference)
                                   if use_decoder else _cpu_baseline(model, M, targets))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
