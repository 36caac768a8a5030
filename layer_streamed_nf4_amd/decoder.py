"""The streamed NF4 QLoRA decoder training step over the C ABI.

Orchestration only: every operation runs in libnf4stream's kernels (the
streamed NF4 linears, the adapters, the resident bf16 lm_head, RMSNorm, rotary
embedding, grouped causal attention, SwiGLU, cross-entropy, AdamW), and the
slot bookkeeping lives in its native pool. torch provides device memory,
pinned host memory and streams.

The model is the llama decoder the pages train ("Soup layer-streamed NF4
training measured", sections 2.1-2.2 and 4.3: SmolLM2-135M and
Llama-3.1-8B-Instruct): pre-norm layers whose seven projections are NF4 shards
streamed through a slot pool, LoRA on the target projections, embedding and
lm_head resident in bf16, the body of every layer checkpointed. A step is

  forward:  h_0 = E[ids]; for each layer i: h_{i+1} = layer_i(h_i), keeping
            h_i only (streaming layer i+1 in while i computes);
            logits = norm(h_L) . lm_head^T; loss = mean cross-entropy;
  backward: dlogits -> dh_L; for i = L-1 .. 0: recompute layer_i from h_i
            (its second read of the shard, streaming layer i-1 in), then
            differentiate it; LoRA gradients are produced on the way;
  update:   AdamW on every adapter parameter (one flat fp32 buffer).

(English article "Fine-Tune 8B Models on 4GB VRAM", "The Principle of Layer
Streaming": forward prefetches i+1, backward i-1, every layer read twice.)
"""
from __future__ import annotations

import torch

from . import (OP_ATTENTION_BWD, OP_CROSS_ENTROPY, OP_DENSE_BWD_PACKED, OP_DENSE_FWD_PACKED,
               OP_LINEAR_BWD_PACKED, OP_LINEAR_FWD_PACKED,
               dense_linear_bwd_packed, dense_linear_fwd_packed, lora_bwd_grouped, lora_fwd_grouped,
               lora_grouped_workspace_bytes, nf4s_adamw,
               nf4s_attention_bwd, nf4s_attention_fwd, nf4s_cross_entropy, nf4s_dpo_loss,
               nf4s_embed, nf4s_logit_grad, nf4s_token_nll,
               nf4s_pack_activation, nf4s_packed_activation_bytes, nf4s_pool_acquire,
               nf4s_pool_create, nf4s_pool_destroy, nf4s_pool_release, nf4s_pool_set_debug,
               nf4s_pool_set_layer, POOL_POISON_ON_RELEASE, nf4s_pool_stats, nf4s_rmsnorm_bwd,
               nf4s_rmsnorm_fwd, nf4s_rope_pair, nf4s_swiglu_bwd, nf4s_swiglu_fwd,
               nf4s_workspace_bytes, streamed_linear_bwd_packed, streamed_linear_fwd_packed,
               streamed_linear_fwd_grouped, grouped_workspace_bytes, grouped_bwd_workspace_bytes,
               streamed_linear_bwd_grouped, streamed_linear_fwd_residual, streamed_linear_fwd_swiglu,
               nf4s_swiglu_fused_supported)
from .stack import ALIGN, PROJ, ShardSet, _prefetch_ahead, _round_up

# projections that read the same input: q, k, v the normed h; gate, up the
# normed h_mid; o and down each their own
GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))

BF16 = torch.int16  # bf16 tensors travel as their bit patterns


class Decoder:
    """One training step of the decoder, streamed (slot pool) or resident.

    cfg: hidden, inter, heads, kv_heads, head_dim, vocab, layers, rope_theta,
         eps (the llama hyper-parameters of the model).
    shards: the layers' NF4 shards (ShardSet with cfg's shapes).
    embed, lm_head: bf16-bit device tensors [vocab, hidden] (the same tensor
         when the embeddings are tied).
    norms: {"attn": [L fp32 [hidden]], "mlp": [...], "final": fp32 [hidden]}.
    lora: {(layer, proj): (A fp32 [r, k_in], B fp32 [n_out, r])} initial
         adapter values (any device); copied into one flat parameter buffer.
    """

    def __init__(self, cfg, shards: ShardSet, embed, lm_head, norms, lora, batch, seq,
                 targets=("q", "v"), r=16, alpha=32, n_slots=2, mode="streamed", lr=1e-4,
                 betas=(0.9, 0.999), adam_eps=1e-8, weight_decay=0.0, time_calls=None, poison=False,
                 trace=False):
        """time_calls: optional predicate (direction, n_out, k_in) -> bool; the
        streamed linear forward calls it accepts are bracketed by timing
        events on the compute stream, collected in self.timed as
        (direction, n_out, k_in, start, end, launches); a grouped launch
        (q, k, v; gate, up) is one entry whose n_out is the group's total."""
        assert mode in ("streamed", "resident")
        self.time_calls = time_calls
        # trace=True: after each backward, trace[i] holds dL/dh_i (fp32 [M,
        # hidden]) for i = 0..L, copied on the compute stream (for tests)
        self.trace = {} if trace else None
        self.timed = []
        self._kept_last = False  # the last layer's body is still in the buffers
        dev = "cuda"
        self.cfg = cfg
        self.sh = shards
        self.L = shards.n_layers
        self.B, self.S = batch, seq
        self.M = M = batch * seq
        self.targets = tuple(targets)
        self.r = r
        self.scale = alpha / r
        self.mode = mode
        self.lr, self.betas, self.adam_eps, self.wd = lr, betas, adam_eps, weight_decay
        self.t = 0
        H, I, V = cfg["hidden"], cfg["inter"], cfg["vocab"]
        nh, nkv, hd = cfg["heads"], cfg["kv_heads"], cfg["head_dim"]
        self.H, self.I, self.V = H, I, V
        self.qd, self.kvd = nh * hd, nkv * hd
        shapes = shards.shapes
        assert shapes["q"] == (self.qd, H) and shapes["k"] == (self.kvd, H)
        assert shapes["gate"] == (I, H) and shapes["down"] == (H, I)
        self.embed, self.lm_head, self.norms = embed, lm_head, norms
        self.compute = torch.cuda.Stream()
        self.copy = torch.cuda.Stream()

        # adapters: one flat fp32 buffer of every A and B (16-byte aligned
        # views), with gradients and AdamW moments laid out the same way
        n = 0
        self._lora_off = {}
        for i in range(self.L):
            for p in self.targets:
                no, ki = shapes[p]
                self._lora_off[(i, p)] = (n, n + r * ki)
                n += r * ki + no * r
        self.n_params = n
        self.params = torch.zeros(n, dtype=torch.float32, device=dev)
        self.grads = torch.zeros(n, dtype=torch.float32, device=dev)
        self.m = torch.zeros(n, dtype=torch.float32, device=dev)
        self.v = torch.zeros(n, dtype=torch.float32, device=dev)
        self.lora = {}
        self.lora_grads = {}
        for (i, p), (oa, ob) in self._lora_off.items():
            no, ki = shapes[p]
            A = self.params[oa:oa + r * ki].view(r, ki)
            Bm = self.params[ob:ob + no * r].view(no, r)
            a0, b0 = lora[(i, p)]
            A.copy_(torch.as_tensor(a0, dtype=torch.float32))
            Bm.copy_(torch.as_tensor(b0, dtype=torch.float32))
            self.lora[(i, p)] = (A, Bm)
            self.lora_grads[(i, p)] = (self.grads[oa:oa + r * ki].view(r, ki),
                                       self.grads[ob:ob + no * r].view(no, r))

        def f32(*shape):
            return torch.empty(shape, dtype=torch.float32, device=dev)

        def bf(*shape):
            return torch.empty(shape, dtype=BF16, device=dev)

        # residual stream checkpoints h_0 .. h_L (the layer inputs), and each
        # layer's mid-layer residual h + o(attention), the one output of the o
        # projection the backward reads: kept from the forward, so that the
        # recompute skips that product
        self.h = [f32(M, H) for _ in range(self.L + 1)]
        self.h_mids = [f32(M, H) for _ in range(self.L)]
        # one layer's recomputable body
        self.n1, self.rstd1 = bf(M, H), f32(M)
        self.q, self.k, self.vv = bf(M, self.qd), bf(M, self.kvd), bf(M, self.kvd)
        self.o, self.o32, self.lse = bf(M, self.qd), f32(M, self.qd), f32(batch, nh, seq)
        self.ao, self.h_mid = bf(M, H), f32(M, H)  # h_mid: the reference model's (adapters off)
        self.n2, self.rstd2 = bf(M, H), f32(M)
        self.g, self.u_, self.sw, self.dn = bf(M, I), bf(M, I), bf(M, I), bf(M, H)
        # head
        self.hn, self.rstd_f = bf(M, H), f32(M)
        self.logits, self.dlogits = bf(M, V), bf(M, V)
        self.loss = f32(1)
        # backward
        self.dh, self.dd = f32(M, H), bf(M, H)
        self.dsw, self.dg, self.du_ = bf(M, I), bf(M, I), bf(M, I)
        self.dnx = [bf(M, H) for _ in range(3)]
        self.do, self.dq, self.dk, self.dv = bf(M, self.qd), bf(M, self.qd), bf(M, self.kvd), bf(M, self.kvd)
        self.dhn = bf(M, H)
        # adapter intermediates: u = x . A^T per target (from the latest
        # forward of the layer), du for the backward
        self.u = {p: f32(M, r) for p in self.targets}
        self.du = {p: f32(M, r) for p in self.targets}

        ws = max(nf4s_workspace_bytes(OP_ATTENTION_BWD, M, nh, hd),
                 nf4s_workspace_bytes(OP_CROSS_ENTROPY, M, 0, 0),
                 nf4s_workspace_bytes(OP_DENSE_FWD_PACKED, M, V, H),
                 nf4s_workspace_bytes(OP_DENSE_BWD_PACKED, M, V, H))
        pk_layer = nf4s_packed_activation_bytes(M, H)
        for p in PROJ:
            no, ki = shapes[p]
            ws = max(ws, nf4s_workspace_bytes(OP_LINEAR_FWD_PACKED, M, no, ki),
                     nf4s_workspace_bytes(OP_LINEAR_BWD_PACKED, M, no, ki))
            pk_layer = max(pk_layer, nf4s_packed_activation_bytes(M, ki),
                           nf4s_packed_activation_bytes(M, no))
        pk = max(pk_layer, nf4s_packed_activation_bytes(M, V))
        for grp in (("q", "k", "v"), ("gate", "up")):
            ws = max(ws, grouped_workspace_bytes([shapes[p][0] for p in grp], shapes[grp[0]][1], M))
        # the backward of q, k, v (and of gate, up) as one contraction when
        # every member would split its contraction alone (small M): one
        # launch and one sum instead of one of each per projection
        # the first forward's gate + up with SwiGLU fused into the launch's
        # epilogue, where its shapes allow (same bits, half the output)
        self._fuse_swiglu = nf4s_swiglu_fused_supported(M, I, H) and I % 64 == 0
        self._group_bwd = {}
        for grp in (("q", "k", "v"), ("gate", "up")):
            n_outs, ki = [shapes[p][0] for p in grp], shapes[grp[0]][1]
            self._group_bwd[grp] = all(n % 64 == 0 for n in n_outs) and all(
                nf4s_workspace_bytes(OP_LINEAR_BWD_PACKED, M, n, ki) > 0 for n in n_outs)
            if self._group_bwd[grp]:
                ws = max(ws, grouped_bwd_workspace_bytes(n_outs, ki, M))
        for grp in GROUPS:
            tg = [p for p in grp if p in self.targets]
            if tg:
                n_outs, ki = [shapes[p][0] for p in tg], shapes[tg[0]][1]
                ws = max(ws, lora_grouped_workspace_bytes(n_outs, ki, M, False),
                         lora_grouped_workspace_bytes(n_outs, ki, M, True))
        self.ws = torch.empty(_round_up(max(ws, ALIGN)), dtype=torch.uint8, device=dev)
        # packed (MFMA fragment order) GEMM inputs: two buffers, so that the
        # two outputs of the SwiGLU backward can both be produced packed, and a
        # third for the third dy of a grouped q, k, v backward
        self.packed = torch.empty(_round_up(pk), dtype=torch.uint8, device=dev)
        self.packed_b = torch.empty(_round_up(pk_layer), dtype=torch.uint8, device=dev)
        self.packed_c = torch.empty(_round_up(pk_layer), dtype=torch.uint8, device=dev)
        self._packed_key = None
        self._packed_key_b = None
        self._packed_key_c = None

        self.pool = None
        if mode == "streamed":
            nb = shards.layout.nbytes
            self.slots = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(n_slots)]
            self.pool = nf4s_pool_create([s.data_ptr() for s in self.slots], nb,
                                         self.copy.cuda_stream, self.compute.cuda_stream)
            for i, hst in enumerate(shards.host):
                nf4s_pool_set_layer(self.pool, i, hst.data_ptr(), nb)
            if poison:  # every released slot is overwritten with NaN block scales
                nf4s_pool_set_debug(self.pool, POOL_POISON_ON_RELEASE)
        else:
            self.resident = shards.to_device()

    def close(self):
        if self.pool is not None:
            torch.cuda.synchronize()
            nf4s_pool_destroy(self.pool)
            self.pool = None

    def stats(self):
        return nf4s_pool_stats(self.pool) if self.pool is not None else (0, 0)

    # -- helpers ---------------------------------------------------------------------
    @property
    def _s(self):
        return self.compute.cuda_stream

    def _ws(self):
        return self.ws.data_ptr(), self.ws.numel()

    def _pack(self, a, K):
        """The packed form of a (bf16 [M, K]) for the matrix cores: the one
        its producer wrote (see _produced), else packed now into the main
        buffer unless it was the last input packed there."""
        key = (a.data_ptr(), K)
        if key == self._packed_key_b:
            return self.packed_b.data_ptr()
        if key == self._packed_key_c:
            return self.packed_c.data_ptr()
        if key != self._packed_key:
            nf4s_pack_activation(a.data_ptr(), self.M, K, self.packed.data_ptr(), self.packed.numel(),
                                 self._s)
            self._packed_key = key
        return self.packed.data_ptr()

    def _produced(self, a, K, second=False, third=False):
        """Mark a (bf16 [M, K]) as written packed by its producer into the main
        (or second, or third) buffer; returns that buffer's pointer for the
        producer."""
        if third:
            self._packed_key_c = (a.data_ptr(), K)
            return self.packed_c.data_ptr()
        if second:
            self._packed_key_b = (a.data_ptr(), K)
            return self.packed_b.data_ptr()
        self._packed_key = (a.data_ptr(), K)
        return self.packed.data_ptr()

    def _fwd(self, base, i, ps, x, ys, adapters=True, res=None):
        """Forward of the projections ps, all reading x (q, k, v or gate, up,
        or a single one), as one GEMM launch writing ys; each launch the
        time_calls predicate accepts is one timed entry with n_out the sum."""
        ki = self.sh.shapes[ps[0]][1]
        xp = self._pack(x, ki)
        tg = self._lora_u(i, ps, x, adapters)
        us = [self.u[p].data_ptr() if p in tg else None for p in ps]
        Bs = [self.lora[(i, p)][1].data_ptr() if p in tg else None for p in ps]
        r = self.r if any(us) else 0
        scale = self.scale if any(us) else 0.0
        ev = self._tick("fwd", sum(self.sh.shapes[p][0] for p in ps), ki)
        if res is not None:  # a single projection into the residual stream: res = (h_in, h_out)
            assert len(ps) == 1
            streamed_linear_fwd_residual(base, self.sh.layout.descs[ps[0]], xp, self.M, ys[0].data_ptr(),
                                         us[0], Bs[0], r, scale, res[0].data_ptr(), res[1].data_ptr(),
                                         *self._ws(), self._s)
        elif len(ps) == 1:
            streamed_linear_fwd_packed(base, self.sh.layout.descs[ps[0]], xp, self.M, ys[0].data_ptr(),
                                       us[0], Bs[0], r, scale, *self._ws(), self._s)
        else:
            streamed_linear_fwd_grouped(base, [self.sh.layout.descs[p] for p in ps], xp, self.M,
                                        [y.data_ptr() for y in ys], us, Bs, r, scale, *self._ws(),
                                        self._s)
        self._tock(ev)

    def _fwd_swiglu(self, base, i, adapters):
        """gate and up of layer i with the SwiGLU epilogue: self.sw row-major
        and, in the second packed buffer (the first holds n2, which the launch
        reads), in fragment order for the down projection."""
        H, I = self.H, self.I
        xp = self._pack(self.n2, H)
        tg = self._lora_u(i, ("gate", "up"), self.n2, adapters)
        us = [self.u[p].data_ptr() if p in tg else None for p in ("gate", "up")]
        Bs = [self.lora[(i, p)][1].data_ptr() if p in tg else None for p in ("gate", "up")]
        r, scale = (self.r, self.scale) if tg else (0, 0.0)
        ev = self._tick("fwd", 2 * I, H)
        streamed_linear_fwd_swiglu(base, self.sh.layout.descs["gate"], self.sh.layout.descs["up"], xp,
                                   self.M, self.sw.data_ptr(), self._produced(self.sw, I, second=True),
                                   self.packed_b.numel(), us, Bs, r, scale, self._s)
        self._tock(ev)

    def _lora_u(self, i, ps, x, adapters=True):
        """u = x . A^T of every adapter among ps (all reading x), one launch
        per kernel; returns those projections."""
        tg = [p for p in ps if adapters and p in self.targets]
        if tg:
            ki = self.sh.shapes[ps[0]][1]
            lora_fwd_grouped(x.data_ptr(), self.M, ki, [self.lora[(i, p)][0].data_ptr() for p in tg],
                             self.r, [self.u[p].data_ptr() for p in tg], *self._ws(), self._s)
        return tg

    def _tick(self, direction, n, k):
        if self.time_calls is None or not self.time_calls(direction, n, k):
            return None
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(self.compute)
        return (direction, n, k, start, end)

    def _tock(self, ev, launches=1):
        if ev is not None:
            ev[4].record(self.compute)
            self.timed.append(ev + (launches,))

    def _pack_group(self, dys, nos):
        """Packed pointers of the dys, one buffer each: those their producer
        wrote packed, the others packed now into the buffers left free."""
        bufs = [(self.packed, "_packed_key"), (self.packed_b, "_packed_key_b"), (self.packed_c, "_packed_key_c")]
        keys = [(dy.data_ptr(), no) for dy, no in zip(dys, nos)]
        out, used = [None] * len(dys), set()
        for j, key in enumerate(keys):
            for bi, (buf, attr) in enumerate(bufs):
                if bi not in used and getattr(self, attr) == key:
                    out[j] = buf.data_ptr()
                    used.add(bi)
                    break
        for j, key in enumerate(keys):
            if out[j] is None:
                bi = next(b for b in range(len(bufs)) if b not in used)
                buf, attr = bufs[bi]
                nf4s_pack_activation(dys[j].data_ptr(), self.M, nos[j], buf.data_ptr(), buf.numel(),
                                     self._s)
                setattr(self, attr, key)
                used.add(bi)
                out[j] = buf.data_ptr()
        return out

    def _bwd(self, base, i, ps, x, dys, dxs, dy_packed=None):
        """Backward of the projections ps, all reading x: the adapter
        gradients of the targets among them (one launch per kernel), then
        dx with each adapter's du . A added: one sum in dxs[0] when the group
        runs as one contraction, else one dx per projection. Returns the dx
        tensors that hold the result. dy_packed: the packed dy of a single
        projection, when its producer wrote it."""
        assert dy_packed is None or len(ps) == 1
        ki = self.sh.shapes[ps[0]][1]
        tg = [p for p in ps if p in self.targets]
        if tg:
            dy_of = dict(zip(ps, dys))
            lora_bwd_grouped(x.data_ptr(), [dy_of[p].data_ptr() for p in tg],
                             [self.u[p].data_ptr() for p in tg], self.M, ki,
                             [self.sh.shapes[p][0] for p in tg],
                             [self.lora[(i, p)][1].data_ptr() for p in tg], self.r, self.scale,
                             [self.lora_grads[(i, p)][0].data_ptr() for p in tg],
                             [self.lora_grads[(i, p)][1].data_ptr() for p in tg],
                             [self.du[p].data_ptr() for p in tg], 0, *self._ws(), self._s)
        if len(ps) > 1 and self._group_bwd.get(tuple(ps)):
            nos = [self.sh.shapes[p][0] for p in ps]
            streamed_linear_bwd_grouped(
                base, [self.sh.layout.descs[p] for p in ps], self._pack_group(dys, nos), self.M,
                dxs[0].data_ptr(), [self.du[p].data_ptr() if p in tg else None for p in ps],
                [self.lora[(i, p)][0].data_ptr() if p in tg else None for p in ps],
                self.r if tg else 0, *self._ws(), self._s)
            return dxs[:1]
        for p, dy, dx in zip(ps, dys, dxs):
            no = self.sh.shapes[p][0]
            dyp = self._pack(dy, no) if dy_packed is None else dy_packed
            if p in tg:
                streamed_linear_bwd_packed(base, self.sh.layout.descs[p], dyp, self.M, dx.data_ptr(),
                                           self.du[p].data_ptr(), self.lora[(i, p)][0].data_ptr(),
                                           self.r, *self._ws(), self._s)
            else:
                streamed_linear_bwd_packed(base, self.sh.layout.descs[p], dyp, self.M, dx.data_ptr(),
                                           None, None, 0, *self._ws(), self._s)
        return list(dxs)

    # -- one layer ---------------------------------------------------------------------
    def _layer_fwd(self, i, base, recompute, adapters=True, hin=None, hout=None, keep=False):
        """Layer i's body from h_i. The recompute keeps the fp32 attention
        output for the backward and skips h_{i+1} and the mid-layer residual
        h_mid, which are already stored (and with them the down and o
        projections' products, which nothing else reads; only their adapters'
        u are recomputed); keep=True keeps the fp32 attention output in a
        first forward too (the last layer, whose backward follows the head
        with the body buffers intact).
        adapters=False runs the frozen base alone (the reference model, whose
        h_mid goes to a scratch buffer); hin/hout default to the checkpoints
        h_i, h_{i+1}."""
        c, s, M = self.cfg, self._s, self.M
        H = self.H
        self._packed_key = self._packed_key_b = self._packed_key_c = None
        own = adapters and hin is None  # the policy's own sweep: h_mid is a checkpoint
        h_mid = self.h_mids[i] if own else self.h_mid
        assert own or not recompute
        hin = self.h[i] if hin is None else hin
        hout = self.h[i + 1] if hout is None else hout
        a = adapters
        nf4s_rmsnorm_fwd(hin.data_ptr(), self.norms["attn"][i].data_ptr(), M, H, c["eps"],
                         self.n1.data_ptr(), self.rstd1.data_ptr(), s, packed=self._produced(self.n1, H))
        self._fwd(base, i, ("q", "k", "v"), self.n1, (self.q, self.k, self.vv), a)
        nf4s_rope_pair(self.q.data_ptr(), c["heads"], self.k.data_ptr(), c["kv_heads"], M, self.S,
                       c["head_dim"], c["rope_theta"], 0, s)
        nf4s_attention_fwd(self.q.data_ptr(), self.k.data_ptr(), self.vv.data_ptr(), self.B, self.S,
                           c["heads"], c["kv_heads"], c["head_dim"], self.o.data_ptr(),
                           self.o32.data_ptr() if recompute or keep else None, self.lse.data_ptr(), s,
                           packed=self._produced(self.o, c["heads"] * c["head_dim"]))
        if recompute:
            self._lora_u(i, ("o",), self.o, a)
        else:
            self._fwd(base, i, ("o",), self.o, (self.ao,), a, res=(hin, h_mid))
        nf4s_rmsnorm_fwd(h_mid.data_ptr(), self.norms["mlp"][i].data_ptr(), M, H, c["eps"],
                         self.n2.data_ptr(), self.rstd2.data_ptr(), s, packed=self._produced(self.n2, H))
        fuse = self._fuse_swiglu and not recompute and not keep
        if fuse:
            self._fwd_swiglu(base, i, a)
        else:
            self._fwd(base, i, ("gate", "up"), self.n2, (self.g, self.u_), a)
        if recompute:
            # h_{i+1} is stored and the backward reads no output of the down
            # projection: only its adapter's u is recomputed, from the SwiGLU
            # output, which nothing else in the backward reads
            if a and "down" in self.targets:
                nf4s_swiglu_fwd(self.g.data_ptr(), self.u_.data_ptr(), M, self.I, self.sw.data_ptr(), s)
                self._lora_u(i, ("down",), self.sw, a)
        else:
            if not fuse:
                nf4s_swiglu_fwd(self.g.data_ptr(), self.u_.data_ptr(), M, self.I, self.sw.data_ptr(), s,
                                packed=self._produced(self.sw, self.I))
            self._fwd(base, i, ("down",), self.sw, (self.dn,), a, res=(h_mid, hout))

    def _layer_bwd(self, i, base):
        """dh holds dL/dh_{i+1} on entry (and dd its bf16 form, packed in
        packed_c) and dL/dh_i on exit (likewise, for i > 0); the layer's body
        was just recomputed (with the fp32 attention output kept)."""
        c, s, M, H = self.cfg, self._s, self.M, self.H
        self._packed_key = self._packed_key_b = self._packed_key_c = None
        self._bwd(base, i, ("down",), self.sw, (self.dd,), (self.dsw,),
                  dy_packed=self.packed_c.data_ptr())
        # the row-major dg, du feed only the gate/up adapters' gradients; the
        # GEMM reads the packed copies
        rows = "gate" in self.targets or "up" in self.targets
        nf4s_swiglu_bwd(self.dsw.data_ptr(), self.g.data_ptr(), self.u_.data_ptr(), M, self.I,
                        self.dg.data_ptr() if rows else None, self.du_.data_ptr() if rows else None, s,
                        dg_packed=self._produced(self.dg, self.I),
                        du_packed=self._produced(self.du_, self.I, second=True))
        dn = self._bwd(base, i, ("gate", "up"), self.n2, (self.dg, self.du_), self.dnx[:2])
        self._packed_key_b = None
        # the norm's backward also leaves dh as the o projection's bf16 input
        nf4s_rmsnorm_bwd([x.data_ptr() for x in dn], self.h_mids[i].data_ptr(),
                         self.norms["mlp"][i].data_ptr(), self.rstd2.data_ptr(), M, H, 1,
                         self.dh.data_ptr(), s, y=self.dd.data_ptr(), packed=self._produced(self.dd, H))
        self._bwd(base, i, ("o",), self.o, (self.dd,), (self.do,))
        nf4s_attention_bwd(self.q.data_ptr(), self.k.data_ptr(), self.vv.data_ptr(),
                           self.o32.data_ptr(), self.do.data_ptr(), self.lse.data_ptr(), self.B,
                           self.S, c["heads"], c["kv_heads"], c["head_dim"], self.dq.data_ptr(),
                           self.dk.data_ptr(), self.dv.data_ptr(), *self._ws(), s,
                           dv_packed=self._produced(self.dv, c["kv_heads"] * c["head_dim"], third=True))
        # the inverse rotation also leaves dq and dk packed for the q / k backward
        nf4s_rope_pair(self.dq.data_ptr(), c["heads"], self.dk.data_ptr(), c["kv_heads"], M, self.S,
                       c["head_dim"], c["rope_theta"], 1, s,
                       q_packed=self._produced(self.dq, c["heads"] * c["head_dim"]),
                       k_packed=self._produced(self.dk, c["kv_heads"] * c["head_dim"], second=True))
        dn = self._bwd(base, i, ("q", "k", "v"), self.n1, (self.dq, self.dk, self.dv), self.dnx)
        self._packed_key_c = None  # packed_c now receives dL/dh_i for the next layer's down projection
        nf4s_rmsnorm_bwd([x.data_ptr() for x in dn], self.h[i].data_ptr(),
                         self.norms["attn"][i].data_ptr(), self.rstd1.data_ptr(), M, H, 1,
                         self.dh.data_ptr(), s, y=self.dd.data_ptr() if i > 0 else None,
                         packed=self.packed_c.data_ptr() if i > 0 else None)

    # -- the step ----------------------------------------------------------------------
    def _check_ids(self, ids, targets):
        assert ids.numel() == self.M and targets.numel() == self.M
        assert ids.dtype == torch.int64 and targets.dtype == torch.int64

    def _head_fwd(self, h_last):
        """Final norm and the resident lm_head: self.logits from h_L."""
        c, M, H, V, s = self.cfg, self.M, self.H, self.V, self._s
        self._packed_key = self._packed_key_b = self._packed_key_c = None
        nf4s_rmsnorm_fwd(h_last.data_ptr(), self.norms["final"].data_ptr(), M, H, c["eps"],
                         self.hn.data_ptr(), self.rstd_f.data_ptr(), s, packed=self._produced(self.hn, H))
        dense_linear_fwd_packed(self.lm_head.data_ptr(), V, H, self._pack(self.hn, H), M,
                                self.logits.data_ptr(), *self._ws(), s)

    def _forward_sweep(self, adapters, then=()):
        """Layers 0..L-1 from h_0; `then` is the order in which layers are read
        after this sweep (what the pool prefetches beyond its end). With
        the adapters on, the last layer's body stays in the buffers for the
        backward, which then skips its recompute (same kernels, same inputs:
        the same bits)."""
        L = self.L
        for i in range(L):
            base = self._acquire(i, list(range(i + 1, L)) + list(then))
            keep = adapters and i == L - 1
            self._layer_fwd(i, base, recompute=False, adapters=adapters, keep=keep)
            self._release(i)
        self._kept_last = adapters

    def _backward(self):
        """From self.dlogits: lm_head and final norm backward, then the
        backward sweep that recomputes each layer and differentiates it."""
        M, H, V, s, L = self.M, self.H, self.V, self._s, self.L
        self._packed_key = self._packed_key_b = self._packed_key_c = None
        dense_linear_bwd_packed(self.lm_head.data_ptr(), V, H, self._pack(self.dlogits, V), M,
                                self.dhn.data_ptr(), *self._ws(), s)
        # (every norm backward of the sweep also leaves dh as bf16 dd, packed
        # in packed_c: the input of the next layer's down-projection backward)
        nf4s_rmsnorm_bwd([self.dhn.data_ptr()], self.h[L].data_ptr(), self.norms["final"].data_ptr(),
                         self.rstd_f.data_ptr(), M, H, 0, self.dh.data_ptr(), s, y=self.dd.data_ptr(),
                         packed=self.packed_c.data_ptr())
        for i in range(L - 1, -1, -1):
            base = self._acquire(i, range(i - 1, -1, -1))
            if not (i == L - 1 and self._kept_last):
                self._layer_fwd(i, base, recompute=True)
            if self.trace is not None:  # dL/dh_{i+1}, the gradient layer i starts from
                with torch.cuda.stream(self.compute):
                    self.trace[i + 1] = self.dh.clone()
            self._layer_bwd(i, base)
            self._release(i)
        self._kept_last = False
        if self.trace is not None:
            with torch.cuda.stream(self.compute):
                self.trace[0] = self.dh.clone()

    def forward_backward(self, ids, targets):
        """Queue the forward and backward sweeps for token ids / next-token
        targets (device int64 [batch*seq]); returns at once. The loss lands in
        self.loss, the logits in self.logits, adapter gradients in self.grads."""
        M, H, V = self.M, self.H, self.V
        self._check_ids(ids, targets)
        self.compute.wait_stream(torch.cuda.current_stream())
        s = self._s
        nf4s_embed(self.embed.data_ptr(), V, H, ids.data_ptr(), M, self.h[0].data_ptr(), s)
        self._forward_sweep(adapters=True, then=range(self.L - 1, -1, -1))
        self._head_fwd(self.h[self.L])
        nf4s_cross_entropy(self.logits.data_ptr(), targets.data_ptr(), M, V, self.loss.data_ptr(),
                           self.dlogits.data_ptr(), *self._ws(), s)
        self._backward()
        torch.cuda.current_stream().wait_stream(self.compute)

    def preference_forward_backward(self, ids, targets, mask, beta=0.1, schedule="separate"):
        """DPO step ("Soup v0.72.4 technical analysis", sections 3.1-3.3): the
        reference model is the same streamed base with the adapters off, the
        policy the base with them on; no second model. Rows are 2 * pairs
        sequences of S tokens ordered chosen, rejected per pair; mask (fp32
        [batch*seq]) weights the response tokens.

        schedule "separate": a reference forward sweep, then the policy's
        forward and backward sweeps (three reads of a layer per step, the
        pages' ~1.5x of the plain step); "fused": the reference forward of a
        layer runs while the policy's forward holds it (two reads). Both give
        identical results. Loss in self.loss, policy logits in self.logits,
        reference log-probabilities in self.nll_ref, gradients in self.grads."""
        assert schedule in ("separate", "fused")
        assert self.B % 2 == 0, "sequences come in chosen/rejected pairs"
        M, H, V, S, L = self.M, self.H, self.V, self.S, self.L
        self._check_ids(ids, targets)
        assert mask.numel() == M and mask.dtype == torch.float32
        self._ensure_preference_buffers(schedule)
        self.compute.wait_stream(torch.cuda.current_stream())
        s = self._s
        nf4s_embed(self.embed.data_ptr(), V, H, ids.data_ptr(), M, self.h[0].data_ptr(), s)
        if schedule == "separate":
            # the reference sweep prefetches the policy's first layers
            self._forward_sweep(adapters=False, then=range(L))
            self._head_fwd(self.h[L])
            nf4s_token_nll(self.logits.data_ptr(), targets.data_ptr(), M, V, self.nll_ref.data_ptr(), s)
            self._forward_sweep(adapters=True, then=range(L - 1, -1, -1))
        else:
            href = self.href
            for i in range(L):
                base = self._acquire(i, list(range(i + 1, L)) + list(range(L - 1, -1, -1)))
                self._layer_fwd(i, base, recompute=False, adapters=False,
                                hin=self.h[0] if i == 0 else href[i % 2], hout=href[(i + 1) % 2])
                self._layer_fwd(i, base, recompute=False, keep=i == L - 1)
                self._release(i)
            self._kept_last = True
            self._head_fwd(href[L % 2])
            nf4s_token_nll(self.logits.data_ptr(), targets.data_ptr(), M, V, self.nll_ref.data_ptr(), s)
        self._head_fwd(self.h[L])
        nf4s_token_nll(self.logits.data_ptr(), targets.data_ptr(), M, V, self.nll_pol.data_ptr(), s)
        nf4s_dpo_loss(self.nll_pol.data_ptr(), self.nll_ref.data_ptr(), mask.data_ptr(), self.B // 2, S,
                      beta, self.loss.data_ptr(), self.seq_coef.data_ptr(), s)
        nf4s_logit_grad(self.logits.data_ptr(), targets.data_ptr(), self.seq_coef.data_ptr(),
                        mask.data_ptr(), M, S, V, self.dlogits.data_ptr(), s)
        self._backward()
        torch.cuda.current_stream().wait_stream(self.compute)

    def _ensure_preference_buffers(self, schedule):
        dev = "cuda"
        if not hasattr(self, "nll_ref"):
            self.nll_ref = torch.empty(self.M, dtype=torch.float32, device=dev)
            self.nll_pol = torch.empty(self.M, dtype=torch.float32, device=dev)
            self.seq_coef = torch.empty(self.B, dtype=torch.float32, device=dev)
        if schedule == "fused" and not hasattr(self, "href"):
            # the reference model's residual stream (current and next layer)
            self.href = [torch.empty((self.M, self.H), dtype=torch.float32, device=dev)
                         for _ in range(2)]

    def preference_step(self, ids, targets, mask, beta=0.1, schedule="separate"):
        self.preference_forward_backward(ids, targets, mask, beta, schedule)
        self.optimizer_step()

    def optimizer_step(self):
        """AdamW on every adapter parameter (one launch over the flat buffer)."""
        self.t += 1
        self.compute.wait_stream(torch.cuda.current_stream())
        nf4s_adamw(self.params.data_ptr(), self.grads.data_ptr(), self.m.data_ptr(), self.v.data_ptr(),
                   self.n_params, self.lr, self.betas[0], self.betas[1], self.adam_eps, self.wd,
                   self.t, self._s)
        torch.cuda.current_stream().wait_stream(self.compute)

    def step(self, ids, targets):
        self.forward_backward(ids, targets)
        self.optimizer_step()

    def _acquire(self, i, ahead):
        """Layer i's slot; then prefetch the next n - 1 distinct layers of
        `ahead` (the rest of the step's reading order)."""
        if self.pool is None:
            return self.resident[i].data_ptr()
        base = nf4s_pool_acquire(self.pool, i)
        _prefetch_ahead(self.pool, i, ahead, len(self.slots) - 1)
        return base

    def _release(self, i):
        if self.pool is not None:
            nf4s_pool_release(self.pool, i)
