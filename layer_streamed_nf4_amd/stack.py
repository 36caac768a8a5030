"""The streamed linear-stack training step over the C ABI.

Orchestration only: every byte of arithmetic runs in libnf4stream's kernels and
the slot bookkeeping lives in its native pool; this module decides the order of
calls. torch provides device memory, pinned host memory and streams.

A layer is the seven frozen projections q, k, v, o, gate, up, down of a
llama-style decoder at their real shapes (gate walkthrough "Soup layer-streamed
NF4 training measured", section 4.4 counts exactly their 2 forward + 2
recompute + 2 dL/dx FLOPs per weight and token). A step is a forward sweep over
layers 0..L-1 and a backward sweep over L-1..0 that recomputes each layer before
differentiating it (English article "Fine-Tune 8B Models on 4GB VRAM",
"The Principle of Layer Streaming": streaming forces checkpointing, so every
layer is read twice per step; the forward prefetches i+1 and the backward
i-1 on a dedicated stream while layer i computes).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import (DTYPE_F32, OP_LINEAR_BWD_PACKED, OP_LINEAR_FWD_PACKED, OP_LORA_BWD, OP_LORA_FWD,
               OP_QUANTIZE, lora_bwd, lora_fwd, nf4_quantize_shard, nf4s_pack_activation,
               nf4s_packed_activation_bytes, nf4s_pool_acquire, nf4s_pool_create,
               nf4s_pool_destroy, nf4s_pool_prefetch, nf4s_pool_release, nf4s_pool_set_layer,
               nf4s_pool_set_debug, POOL_POISON_ON_RELEASE,
               nf4s_pool_stats, nf4s_tensor_layout, nf4s_workspace_bytes,
               streamed_linear_bwd_packed, streamed_linear_fwd_packed)

PROJ = ("q", "k", "v", "o", "gate", "up", "down")
ALIGN = 256


def _round_up(x, a=ALIGN):
    return (x + a - 1) // a * a


def stream_handle(s: torch.cuda.Stream) -> int:
    return s.cuda_stream


@dataclass
class LayerLayout:
    """Byte layout of one layer shard: the seven tensors back to back."""
    shapes: dict
    descs: dict = field(default_factory=dict)
    nbytes: int = 0

    def __post_init__(self):
        base = 0
        for p in PROJ:
            d = nf4s_tensor_layout(*self.shapes[p], base)
            self.descs[p] = d
            base = d.end
        self.nbytes = _round_up(base)


class ShardSet:
    """Layer shards quantised on the device and parked in pinned host memory.

    weight_fn(layer, proj) returns the fp32 weight [n_out, k_in] on the device.
    The quantiser runs once per tensor, offline (gate walkthrough, section 2.1).
    """

    def __init__(self, shapes, n_layers, weight_fn, device="cuda", pinned=True, keep_device=False):
        self.layout = LayerLayout(shapes)
        self.n_layers = n_layers
        self.shapes = shapes
        nb = self.layout.nbytes
        ws_bytes = max(nf4s_workspace_bytes(OP_QUANTIZE, 0, *shapes[p]) for p in PROJ)
        ws = torch.empty(_round_up(ws_bytes), dtype=torch.uint8, device=device)
        status = torch.zeros(1, dtype=torch.int32, device=device)
        stage = torch.empty(nb, dtype=torch.uint8, device=device)
        s = torch.cuda.current_stream().cuda_stream
        self.host = []
        self.device = []
        for i in range(n_layers):
            for p in PROJ:
                w = weight_fn(i, p).contiguous()
                assert w.dtype == torch.float32 and tuple(w.shape) == tuple(shapes[p])
                nf4_quantize_shard(w.data_ptr(), DTYPE_F32, *shapes[p], stage.data_ptr(),
                                   self.layout.descs[p], status.data_ptr(), ws.data_ptr(),
                                   ws.numel(), s)
                del w
            if pinned:
                h = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
                h.copy_(stage)
                self.host.append(h)
            if keep_device:
                self.device.append(stage.clone())
        torch.cuda.synchronize()
        if int(status.item()) != 0:
            raise ValueError("non-finite weight in a quantised tensor")

    @classmethod
    def from_host(cls, shapes, n_layers, host):
        """A shard set over existing host copies of the layer shards (for
        example read back from a shard cache); nothing is quantised."""
        self = cls.__new__(cls)
        self.layout = LayerLayout(shapes)
        self.n_layers = n_layers
        self.shapes = shapes
        assert len(host) == n_layers and all(h.numel() == self.layout.nbytes for h in host)
        self.host = list(host)
        self.device = []
        return self

    def to_device(self):
        """Resident copies of every layer shard (the resident-NF4 reference)."""
        if not self.device:
            self.device = [h.to("cuda") for h in self.host]
        return self.device


def _prefetch_ahead(pool, cur, ahead, depth):
    """Prefetch the first `depth` distinct layers of `ahead` other than cur, in
    order ("Fine-Tune 8B Models on 4GB VRAM: Soup's Layer Streaming", "The
    Principle of Layer Streaming": the next layer is fetched on the side
    stream while the current one computes; with n slots, n - 1 can be in
    flight or waiting). The pool never evicts a prefetched layer for a later
    prefetch, so the nearest layers keep their slots."""
    seen = []
    for j in ahead:
        if len(seen) >= depth:
            break
        if j != cur and j not in seen:
            seen.append(j)
            nf4s_pool_prefetch(pool, j)


class LinearStack:
    """Runs the linear-stack step streamed (slot pool) or resident.

    lora[i][p] = (A fp32 [r, k_in], B fp32 [n_out, r]) device tensors for the
    target projections. inputs(i, p) / grads(i, p) return bf16-bit tensors
    (int16 storage) x [M, k_in] and dy [M, n_out].
    """

    def __init__(self, shards: ShardSet, M, targets, lora, r=16, alpha=32, n_slots=2,
                 mode="streamed", keep_outputs=True, time_calls=None, poison=False):
        """time_calls: optional predicate (direction, n_out, k_in) -> bool; the
        linear calls it accepts are bracketed by timing events on the compute
        stream and collected in self.timed as (direction, n_out, k_in, start, end).
        poison: the pool overwrites every released slot with NaN block scales
        (ordered after its last reader), so a read after release would show."""
        assert mode in ("streamed", "resident")
        self.sh = shards
        self.M = M
        self.targets = tuple(targets)
        self.lora = lora
        self.r = r
        self.scale = alpha / r
        self.mode = mode
        self.keep = keep_outputs
        dev = "cuda"
        shapes = shards.shapes
        self.compute = torch.cuda.Stream()
        self.copy = torch.cuda.Stream()
        ws = 0
        pk = 0
        for p in PROJ:
            n, k = shapes[p]
            ws = max(ws, nf4s_workspace_bytes(OP_LINEAR_FWD_PACKED, M, n, k),
                     nf4s_workspace_bytes(OP_LINEAR_BWD_PACKED, M, n, k),
                     nf4s_workspace_bytes(OP_LORA_FWD, M, n, k),
                     nf4s_workspace_bytes(OP_LORA_BWD, M, n, k))
            pk = max(pk, nf4s_packed_activation_bytes(M, k), nf4s_packed_activation_bytes(M, n))
        self.ws = torch.empty(_round_up(max(ws, ALIGN)), dtype=torch.uint8, device=dev)
        # the activation of the current projection in the matrix cores' fragment
        # order; projections that read the same input (q, k, v; gate, up) share it
        self.packed = torch.empty(_round_up(pk), dtype=torch.uint8, device=dev)
        self._packed_key = None
        # u = x . A^T per target, produced by the (re)computed forward of a layer
        # and consumed by that layer's backward
        self.u = {p: torch.empty((M, r), dtype=torch.float32, device=dev) for p in self.targets}
        self.du = torch.empty((M, r), dtype=torch.float32, device=dev)
        self.pool = None
        if mode == "streamed":
            nb = shards.layout.nbytes
            self.slots = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(n_slots)]
            self.pool = nf4s_pool_create([s.data_ptr() for s in self.slots], nb,
                                         self.copy.cuda_stream, self.compute.cuda_stream)
            for i, h in enumerate(shards.host):
                nf4s_pool_set_layer(self.pool, i, h.data_ptr(), nb)
            if poison:
                nf4s_pool_set_debug(self.pool, POOL_POISON_ON_RELEASE)
        else:
            self.resident = shards.to_device()
        self.y = {}
        self.dx = {}
        self.grads = {}
        self.time_calls = time_calls
        self.timed = []

    def close(self):
        if self.pool is not None:
            torch.cuda.synchronize()
            nf4s_pool_destroy(self.pool)
            self.pool = None

    def stats(self):
        return nf4s_pool_stats(self.pool) if self.pool is not None else (0, 0)

    # -- one layer -----------------------------------------------------------------
    def _out(self, store, key, shape, dtype):
        t = store.get(key)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device="cuda")
            store[key] = t
        return t

    def _pack(self, a, K):
        """Pack a (bf16 [M, K]) unless it is the input packed last; kernels run
        in order on the compute stream, so one buffer serves all projections."""
        key = (a.data_ptr(), K)
        if key != self._packed_key:
            nf4s_pack_activation(a.data_ptr(), self.M, K, self.packed.data_ptr(), self.packed.numel(),
                                 self.compute.cuda_stream)
            self._packed_key = key
        return self.packed.data_ptr()

    def _layer_fwd(self, i, base, inputs, store_key, adapters=True):
        s = self.compute.cuda_stream
        shapes = self.sh.shapes
        self._packed_key = None  # inputs may differ from layer to layer
        for p in PROJ:
            n, k = shapes[p]
            x = inputs(i, p)
            xp = self._pack(x, k)
            y = self._out(self.y, (store_key(i), p), (self.M, n), torch.int16)
            if adapters and p in self.targets:
                A, B = self.lora[i][p]
                u = self.u[p]
                lora_fwd(x.data_ptr(), self.M, k, A.data_ptr(), self.r, u.data_ptr(),
                         self.ws.data_ptr(), self.ws.numel(), s)
                ev = self._tick("fwd", n, k)
                streamed_linear_fwd_packed(base, self.sh.layout.descs[p], xp, self.M, y.data_ptr(),
                                           u.data_ptr(), B.data_ptr(), self.r, self.scale,
                                           self.ws.data_ptr(), self.ws.numel(), s)
                self._tock(ev)
            else:
                ev = self._tick("fwd", n, k)
                streamed_linear_fwd_packed(base, self.sh.layout.descs[p], xp, self.M, y.data_ptr(),
                                           None, None, 0, 0.0, self.ws.data_ptr(), self.ws.numel(), s)
                self._tock(ev)

    def _layer_bwd(self, i, base, inputs, grads):
        s = self.compute.cuda_stream
        shapes = self.sh.shapes
        key = i if self.keep else 0
        self._packed_key = None
        for p in PROJ:
            n, k = shapes[p]
            x = inputs(i, p)
            dy = grads(i, p)
            dx = self._out(self.dx, (key, p), (self.M, k), torch.int16)
            if p in self.targets:
                A, B = self.lora[i][p]
                dA = self._out(self.grads, (i, p, "dA"), (self.r, k), torch.float32)
                dB = self._out(self.grads, (i, p, "dB"), (n, self.r), torch.float32)
                # u = x . A^T from this layer's recompute
                lora_bwd(x.data_ptr(), dy.data_ptr(), self.u[p].data_ptr(), self.M, k, n, B.data_ptr(),
                         self.r, self.scale, dA.data_ptr(), dB.data_ptr(), self.du.data_ptr(), 0,
                         self.ws.data_ptr(), self.ws.numel(), s)
                dyp = self._pack(dy, n)
                ev = self._tick("bwd", n, k)
                streamed_linear_bwd_packed(base, self.sh.layout.descs[p], dyp, self.M, dx.data_ptr(),
                                           self.du.data_ptr(), A.data_ptr(), self.r,
                                           self.ws.data_ptr(), self.ws.numel(), s)
                self._tock(ev)
            else:
                dyp = self._pack(dy, n)
                ev = self._tick("bwd", n, k)
                streamed_linear_bwd_packed(base, self.sh.layout.descs[p], dyp, self.M, dx.data_ptr(),
                                           None, None, 0, self.ws.data_ptr(), self.ws.numel(), s)
                self._tock(ev)

    def _tick(self, direction, n, k):
        if self.time_calls is None or not self.time_calls(direction, n, k):
            return None
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(self.compute)
        return (direction, n, k, start, end)

    def _tock(self, ev):
        if ev is not None:
            ev[4].record(self.compute)
            self.timed.append(ev)

    # -- the step ------------------------------------------------------------------
    def step(self, inputs, grads, reference=None):
        """Forward sweep then backward sweep with recompute. Kernels are queued
        on the compute stream, copies on the copy stream; returns at once.

        reference: None for a plain adapter step; "separate" or "fused" for a
        preference step, which also runs the reference model -- the same frozen
        shards with the adapters switched off, no second model (kwkr.cn
        "Soup v0.72.4 technical analysis", sections 3.1-3.3). "separate" gives
        the reference its own forward sweep before the policy's (three reads
        of every layer per step, the pages' ~1.5x); "fused" runs the reference
        forward on each layer while the policy's forward holds it (two reads).
        Reference outputs land in self.y with keys ("ref", i) (or
        ("ref", 0) when outputs are not kept)."""
        assert reference in (None, "separate", "fused")
        L = self.sh.n_layers
        fkey = (lambda i: ("f", i)) if self.keep else (lambda i: ("f", 0))
        rkey = (lambda i: ("r", i)) if self.keep else (lambda i: ("f", 0))
        refkey = (lambda i: ("ref", i)) if self.keep else (lambda i: ("ref", 0))
        self.compute.wait_stream(torch.cuda.current_stream())
        fwd, bwd = list(range(L)), list(range(L - 1, -1, -1))
        # the order in which the step reads the layers: the pool prefetches
        # along it (the last reference layer prefetches the policy's first)
        order = (fwd if reference == "separate" else []) + fwd + bwd
        t = 0
        if reference == "separate":
            for i in fwd:
                base = self._acquire(i, order[t + 1:])
                self._layer_fwd(i, base, inputs, refkey, adapters=False)
                self._release(i)
                t += 1
        for i in fwd:
            base = self._acquire(i, order[t + 1:])
            if reference == "fused":
                self._layer_fwd(i, base, inputs, refkey, adapters=False)
            self._layer_fwd(i, base, inputs, fkey)
            self._release(i)
            t += 1
        for i in bwd:
            base = self._acquire(i, order[t + 1:])
            self._layer_fwd(i, base, inputs, rkey)      # recompute
            self._layer_bwd(i, base, inputs, grads)
            self._release(i)
            t += 1
        torch.cuda.current_stream().wait_stream(self.compute)

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
