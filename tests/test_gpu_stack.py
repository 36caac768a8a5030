"""Streamed linear stack on the GPU: streamed == resident (0.0), invariance to
the pool size, recompute == forward, non-zero adapter grads in every layer, and
per-layer agreement with the oracle.

Gate walkthrough ("Soup layer-streamed NF4 training measured"), section 2.2:
streamed vs resident NF4 logits max abs diff 0.0, 25-step losses identical,
same seed twice 0.0, buffer count n=2 vs n=3 0.0, LoRA grads non-zero in 30/30
layers, on the 135M model (30 layers, hidden 576, B1 S512, LoRA r16 on q/v).
Stand-in here: the 30 layers' seven projections at those shapes with seeded
weights and seeded activations/upstream gradients per layer.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import layer_streamed_nf4_amd as L
import synth
from layer_streamed_nf4_amd.stack import PROJ, LinearStack, ShardSet
from oracle import linear, nf4, stack as ostack
from tests import stack32b
from tests.gpu_helpers import bits_to_f32, dev_bf16bits, dev_f32, host_u16, require_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

MODEL = "135m"
SHAPES = synth.SHAPES[MODEL]
N_LAYERS = synth.N_LAYERS[MODEL]
M = 512
TARGETS = ("q", "v")


@pytest.fixture(scope="module")
def world():
    require_gpu()
    shards = ShardSet(SHAPES, N_LAYERS, lambda i, p: dev_f32(synth.weight(i, p, *SHAPES[p])))
    lora = [{p: (dev_f32(a), dev_f32(b)) for p in TARGETS
             for a, b in [synth.lora_pair(i, p, *SHAPES[p])]} for i in range(N_LAYERS)]
    xs = {}
    dys = {}
    for i in range(N_LAYERS):
        for j, p in enumerate(PROJ):
            n, k = SHAPES[p]
            xs[i, p] = synth.activation((M, k), 0, 100 * i + j)
            dys[i, p] = synth.activation((M, n), 0, 100 * i + 50 + j)
    xd = {key: dev_bf16bits(v) for key, v in xs.items()}
    dyd = {key: dev_bf16bits(v) for key, v in dys.items()}
    return dict(shards=shards, lora=lora, xs=xs, dys=dys, xd=xd, dyd=dyd)


def _run(world, mode, n_slots=2):
    st = LinearStack(world["shards"], M, TARGETS, world["lora"], n_slots=n_slots, mode=mode)
    st.step(lambda i, p: world["xd"][i, p], lambda i, p: world["dyd"][i, p])
    torch.cuda.synchronize()
    out = {}
    for key, t in st.y.items():
        out[("y",) + key] = t.cpu().numpy().copy()
    for key, t in st.dx.items():
        out[("dx",) + key] = t.cpu().numpy().copy()
    for key, t in st.grads.items():
        out[("g",) + key] = t.cpu().numpy().copy()
    stats = st.stats()
    st.close()
    return out, stats


@pytest.fixture(scope="module")
def resident(world):
    return _run(world, "resident")[0]


def _same(a, b):
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


@pytest.mark.parametrize("n_slots", [2, 3, 8])
def test_streamed_equals_resident(world, resident, n_slots):
    print(f"stack streamed n={n_slots}", flush=True)
    got, (copies, nbytes) = _run(world, "streamed", n_slots)
    _same(got, resident)
    # each layer is read in the forward and again in the backward, except the
    # ones still resident in a slot when the backward sweep starts
    assert copies == 2 * N_LAYERS - n_slots
    assert nbytes == copies * world["shards"].layout.nbytes


def test_same_seed_twice(world, resident):
    again, _ = _run(world, "streamed", 2)
    _same(again, resident)


def test_recompute_equals_forward_and_grads_nonzero(resident):
    for i in range(N_LAYERS):
        for p in PROJ:
            assert np.array_equal(resident[("y", ("f", i), p)], resident[("y", ("r", i), p)])
        for p in TARGETS:
            dA = resident[("g", i, p, "dA")]
            dB = resident[("g", i, p, "dB")]
            assert np.count_nonzero(dA) == dA.size and np.count_nonzero(dB) == dB.size


@pytest.mark.parametrize("layer", [0, 17, N_LAYERS - 1])
def test_layers_match_oracle(world, resident, layer):
    weights = {p: bits_to_f32(nf4.dequantize_bf16(nf4.quantize(synth.weight(layer, p, *SHAPES[p]))))
               for p in PROJ}
    inputs = {p: bits_to_f32(world["xs"][layer, p]) for p in PROJ}
    grads = {p: bits_to_f32(world["dys"][layer, p]) for p in PROJ}
    lora = {p: synth.lora_pair(layer, p, *SHAPES[p]) for p in TARGETS}
    ref = ostack.layer_step(weights, inputs, grads, lora, TARGETS, 2.0)
    for p in PROJ:
        y = bits_to_f32(resident[("y", ("f", layer), p)].view(np.uint16))
        dx = bits_to_f32(resident[("dx", layer, p)].view(np.uint16))
        assert linear.rel_err(y, ref[p]["y"]) <= 5e-3, p
        assert linear.rel_err(dx, ref[p]["dx"]) <= 5e-3, p
        if p in TARGETS:
            assert linear.rel_err(resident[("g", layer, p, "dA")], ref[p]["dA"]) <= 5e-3
            assert linear.rel_err(resident[("g", layer, p, "dB")], ref[p]["dB"]) <= 5e-3


def test_prefetch_copies_bytes_and_orders_events():
    require_gpu()
    nbytes = 3 * 1024 * 1024 + 256
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8).pin_memory()
    slot = torch.zeros(nbytes + 4096, dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    free_ev = L.nf4s_event_create()
    ready = L.nf4s_event_create()
    L.nf4s_event_record(free_ev, torch.cuda.current_stream().cuda_stream)
    L.layer_prefetch(slot.data_ptr(), slot.numel(), src.data_ptr(), nbytes, cs.cuda_stream, free_ev, ready)
    L.nf4s_stream_wait_event(torch.cuda.current_stream().cuda_stream, ready)
    assert torch.equal(slot[:nbytes].cpu(), src)
    L.nf4s_event_destroy(free_ev)
    L.nf4s_event_destroy(ready)


def test_pool_slots_evict_and_reregister():
    """Two slots, three layers: least recently used eviction, a held slot is
    never a victim, and a layer registered again is copied afresh."""
    require_gpu()
    nbytes = 1024 * 1024
    srcs = [torch.full((nbytes,), 11 * (i + 1), dtype=torch.uint8).pin_memory() for i in range(4)]
    slots = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    cs = torch.cuda.Stream()
    comp = torch.cuda.current_stream().cuda_stream
    pool = L.nf4s_pool_create([t.data_ptr() for t in slots], nbytes, cs.cuda_stream, comp)
    try:
        for i in range(3):
            L.nf4s_pool_set_layer(pool, i, srcs[i].data_ptr(), nbytes)

        def read(layer):
            ptr = L.nf4s_pool_acquire(pool, layer)
            slot = next(t for t in slots if t.data_ptr() == ptr)
            val = slot.cpu()
            L.nf4s_pool_release(pool, layer)
            return val

        assert torch.equal(read(0), srcs[0]) and torch.equal(read(1), srcs[1])
        assert L.nf4s_pool_stats(pool) == (2, 2 * nbytes)
        assert torch.equal(read(0), srcs[0])                  # resident: no copy
        assert L.nf4s_pool_stats(pool)[0] == 2
        assert torch.equal(read(2), srcs[2])                  # evicts layer 1
        assert torch.equal(read(0), srcs[0])
        assert L.nf4s_pool_stats(pool)[0] == 3
        # a held slot is no victim: with both held, a prefetch is refused
        L.nf4s_pool_acquire(pool, 0)
        L.nf4s_pool_acquire(pool, 2)
        with pytest.raises(L.Nf4sError) as e:
            L.nf4s_pool_prefetch(pool, 1)
        assert e.value.code == L.ESLOT
        with pytest.raises(L.Nf4sError) as e:               # held: not replaced
            L.nf4s_pool_set_layer(pool, 0, srcs[3].data_ptr(), nbytes)
        assert e.value.code == L.ESLOT
        L.nf4s_pool_release(pool, 0)
        L.nf4s_pool_release(pool, 2)
        L.nf4s_pool_set_layer(pool, 0, srcs[3].data_ptr(), nbytes)
        assert torch.equal(read(0), srcs[3])                  # copied afresh
        assert L.nf4s_pool_stats(pool)[0] == 4
    finally:
        torch.cuda.synchronize()
        L.nf4s_pool_destroy(pool)


def test_pool_refuses_unregistered_layers_and_keeps_reservations():
    """Layer indices that were never registered (-1 included: it also marks an
    empty slot) are ESLOT for prefetch, acquire and release, also after a
    re-registration emptied a slot. A prefetch never evicts a layer an earlier
    prefetch reserved; an empty slot is filled before a resident layer is
    evicted; an acquire may take a reserved slot when nothing else is left."""
    require_gpu()
    nbytes = 256 * 1024
    srcs = [torch.full((nbytes,), 7 * (i + 1), dtype=torch.uint8).pin_memory() for i in range(6)]
    slots = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(3)]
    cs = torch.cuda.Stream()
    comp = torch.cuda.current_stream().cuda_stream
    pool = L.nf4s_pool_create([t.data_ptr() for t in slots], nbytes, cs.cuda_stream, comp)
    try:
        for i in range(5):
            L.nf4s_pool_set_layer(pool, i, srcs[i].data_ptr(), nbytes)
        for bad in (-1, 5, 100):
            for call in (lambda: L.nf4s_pool_prefetch(pool, bad), lambda: L.nf4s_pool_acquire(pool, bad),
                         lambda: L.nf4s_pool_release(pool, bad)):
                with pytest.raises(L.Nf4sError) as e:
                    call()
                assert e.value.code == L.ESLOT, bad

        def held_value(layer):
            ptr = L.nf4s_pool_acquire(pool, layer)
            return next(t for t in slots if t.data_ptr() == ptr).cpu()

        assert torch.equal(held_value(0), srcs[0])
        L.nf4s_pool_prefetch(pool, 1)
        L.nf4s_pool_prefetch(pool, 2)                         # pool: 0 held, 1 and 2 reserved
        assert L.nf4s_pool_stats(pool)[0] == 3
        L.nf4s_pool_prefetch(pool, 3)                         # no slot to take: nothing copied
        assert L.nf4s_pool_stats(pool)[0] == 3
        L.nf4s_pool_release(pool, 0)
        L.nf4s_pool_prefetch(pool, 3)                         # evicts 0, not a reserved layer
        assert L.nf4s_pool_stats(pool)[0] == 4
        for j in (1, 2, 3):
            assert torch.equal(held_value(j), srcs[j])
            L.nf4s_pool_release(pool, j)
        assert L.nf4s_pool_stats(pool)[0] == 4                # all three were resident
        # re-registering layer 2 empties its slot; the next copy goes there
        L.nf4s_pool_set_layer(pool, 2, srcs[5].data_ptr(), nbytes)
        with pytest.raises(L.Nf4sError) as e:
            L.nf4s_pool_acquire(pool, -1)
        assert e.value.code == L.ESLOT
        assert torch.equal(held_value(4), srcs[4])
        L.nf4s_pool_release(pool, 4)
        assert torch.equal(held_value(1), srcs[1])            # 1 survived: the empty slot took 4
        assert torch.equal(held_value(3), srcs[3])
        assert L.nf4s_pool_stats(pool)[0] == 5
        # 1 and 3 held, the third slot holds 4: an acquire takes it even when
        # it is reserved
        L.nf4s_pool_prefetch(pool, 4)
        assert torch.equal(held_value(2), srcs[5])
        assert L.nf4s_pool_stats(pool)[0] == 6
        for j in (1, 3, 2):
            L.nf4s_pool_release(pool, j)
    finally:
        torch.cuda.synchronize()
        L.nf4s_pool_destroy(pool)


def test_pool_copy_waits_for_the_release_on_the_device():
    """A copy into a released slot is issued only once the compute stream has
    passed the release: a reader queued behind ≈ms of compute before the
    release still sees the old layer, and the next acquire sees the new one."""
    require_gpu()
    nbytes = 8 << 20
    srcs = [torch.full((nbytes,), 5 * (i + 1), dtype=torch.uint8).pin_memory() for i in range(3)]
    slots = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    cs = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    pool = L.nf4s_pool_create([t.data_ptr() for t in slots], nbytes, cs.cuda_stream, comp.cuda_stream)
    a = torch.randn((4096, 4096), device="cuda", dtype=torch.bfloat16)
    try:
        for i in range(3):
            L.nf4s_pool_set_layer(pool, i, srcs[i].data_ptr(), nbytes)
        ptr0 = L.nf4s_pool_acquire(pool, 0)
        slot0 = next(t for t in slots if t.data_ptr() == ptr0)
        for _ in range(20):                                  # keep the compute stream busy
            a = (a @ a) * (1.0 / 64)
        seen = slot0.clone()                                 # queued behind the matmuls
        L.nf4s_pool_release(pool, 0)
        ptr1 = L.nf4s_pool_acquire(pool, 1)                  # the other slot
        L.nf4s_pool_release(pool, 1)
        L.nf4s_pool_prefetch(pool, 2)                        # evicts layer 0 (least recently used)
        ptr2 = L.nf4s_pool_acquire(pool, 2)
        assert ptr2 == ptr0 and ptr1 != ptr0
        after = slot0.clone()
        L.nf4s_pool_release(pool, 2)
        torch.cuda.synchronize()
        assert torch.equal(seen.cpu(), srcs[0])
        assert torch.equal(after.cpu(), srcs[2])
    finally:
        torch.cuda.synchronize()
        L.nf4s_pool_destroy(pool)


def test_pool_destroy_issues_pending_copies():
    """Copies asked for and never acquired are still enqueued before the pool
    is destroyed (its issuer drains its requests, then stops)."""
    require_gpu()
    nbytes = 4 << 20
    srcs = [torch.full((nbytes,), 3 * (i + 1), dtype=torch.uint8).pin_memory() for i in range(2)]
    slots = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    cs = torch.cuda.Stream()
    pool = L.nf4s_pool_create([t.data_ptr() for t in slots], nbytes, cs.cuda_stream,
                              torch.cuda.current_stream().cuda_stream)
    for i in range(2):
        L.nf4s_pool_set_layer(pool, i, srcs[i].data_ptr(), nbytes)
        L.nf4s_pool_prefetch(pool, i)
    L.nf4s_pool_destroy(pool)
    cs.synchronize()
    got = sorted(int(t[0].item()) for t in slots)
    assert got == [3, 6] and all(torch.equal(t.cpu(), srcs[(int(t[0].item()) // 3) - 1]) for t in slots)


def test_poisoned_release_is_never_read():
    """With the pool's poison mode on, every released slot is overwritten with
    NaN block scales on the copy stream, ordered after its free event exactly
    as the next copy would be. The streamed step still equals the resident one
    bit for bit (no kernel reads a slot after its release) and every layer is
    copied twice (a poisoned slot holds no layer)."""
    require_gpu()
    nbytes = 4096
    src = torch.full((nbytes,), 3, dtype=torch.uint8).pin_memory()
    slots = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    cs = torch.cuda.Stream()
    comp = torch.cuda.current_stream().cuda_stream
    pool = L.nf4s_pool_create([t.data_ptr() for t in slots], nbytes, cs.cuda_stream, comp)
    try:
        L.nf4s_pool_set_debug(pool, L.POOL_POISON_ON_RELEASE)
        with pytest.raises(L.Nf4sError) as e:
            L.nf4s_pool_set_debug(pool, 2)
        assert e.value.code == L.EINVAL
        L.nf4s_pool_set_layer(pool, 0, src.data_ptr(), nbytes)
        ptr = L.nf4s_pool_acquire(pool, 0)
        slot = next(t for t in slots if t.data_ptr() == ptr)
        assert torch.equal(slot.cpu(), src)
        L.nf4s_pool_release(pool, 0)
        torch.cuda.synchronize()
        assert bool((slot.cpu() == 255).all())
        assert L.nf4s_pool_acquire(pool, 0) is not None and L.nf4s_pool_stats(pool)[0] == 2
        L.nf4s_pool_release(pool, 0)
    finally:
        torch.cuda.synchronize()
        L.nf4s_pool_destroy(pool)


@pytest.mark.parametrize("n_slots", [2, 3])
def test_streamed_with_poisoned_releases_equals_resident(world, resident, n_slots):
    st = LinearStack(world["shards"], M, TARGETS, world["lora"], n_slots=n_slots, mode="streamed",
                     poison=True)
    st.step(lambda i, p: world["xd"][i, p], lambda i, p: world["dyd"][i, p])
    torch.cuda.synchronize()
    got = {("y",) + k: t.cpu().numpy().copy() for k, t in st.y.items()}
    got.update({("dx",) + k: t.cpu().numpy().copy() for k, t in st.dx.items()})
    got.update({("g",) + k: t.cpu().numpy().copy() for k, t in st.grads.items()})
    copies, _ = st.stats()
    st.close()
    _same(got, resident)
    assert copies == 2 * N_LAYERS


def test_pageable_source_is_refused():
    require_gpu()
    src = torch.zeros(4096, dtype=torch.uint8)           # pageable
    slot = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.Nf4sError) as e:
        L.layer_prefetch(slot.data_ptr(), 4096, src.data_ptr(), 4096, torch.cuda.Stream().cuda_stream)
    assert e.value.code == L.ENOTPINNED


def test_shard_cache_roundtrip_streams_identically(world, resident, tmp_path):
    """Shards quantised on the GPU, saved, loaded back into pinned memory and
    streamed give the resident result bit for bit (gate walkthrough section 5:
    a cached shard set is reused as is)."""
    from layer_streamed_nf4_amd import shardcache
    fp = shardcache.fingerprint_recipe({"model": MODEL, "weights": "synth.weight", "layers": N_LAYERS})
    path = str(tmp_path / "shards")
    shardcache.save(world["shards"], path, fp)
    back = shardcache.load(path, SHAPES, N_LAYERS, fp)
    for a, b in zip(world["shards"].host, back.host):
        assert torch.equal(a, b)
    w2 = dict(world)
    w2["shards"] = back
    got, _ = _run(w2, "streamed", 2)
    _same(got, resident)


@pytest.mark.parametrize("reference", ["separate", "fused"])
def test_preference_step_streamed_equals_resident(world, resident, reference):
    """Preference step: a reference pass with the adapters off over the same
    streamed shards, then the policy step (kwkr.cn "Soup v0.72.4 technical
    analysis", sections 3.1-3.3). Streamed == resident bit for bit; the policy
    part equals the plain step; reference outputs equal the adapter-free
    product; copies in one step from an empty pool: 3L - n (separate) or
    2L - n (fused), against 2L - n for the plain step."""
    print(f"preference {reference}", flush=True)

    def run(mode):
        st = LinearStack(world["shards"], M, TARGETS, world["lora"], n_slots=2, mode=mode)
        st.step(lambda i, p: world["xd"][i, p], lambda i, p: world["dyd"][i, p], reference=reference)
        torch.cuda.synchronize()
        out = {("y",) + k: t.cpu().numpy().copy() for k, t in st.y.items()}
        out.update({("dx",) + k: t.cpu().numpy().copy() for k, t in st.dx.items()})
        out.update({("g",) + k: t.cpu().numpy().copy() for k, t in st.grads.items()})
        stats = st.stats()
        st.close()
        return out, stats

    streamed, (copies, _) = run("streamed")
    res, _ = run("resident")
    _same(streamed, res)
    policy = {k: v for k, v in streamed.items() if not (k[0] == "y" and k[1][0] == "ref")}
    _same(policy, resident)
    assert copies == (3 if reference == "separate" else 2) * N_LAYERS - 2
    # the reference outputs are the adapter-free products: equal to the policy
    # output for non-adapted projections, different for the adapted ones
    for i in (0, N_LAYERS - 1):
        for p in PROJ:
            ref = streamed[("y", ("ref", i), p)]
            pol = streamed[("y", ("f", i), p)]
            if p in TARGETS:
                assert not np.array_equal(ref, pol), (i, p)
            else:
                assert np.array_equal(ref, pol), (i, p)


def test_32b_layers_preference_streamed_equals_resident():
    """Layers larger than 165 MiB (32B-class shapes: 251.5 MB per layer shard)
    streamed through a 2-slot pool give the resident results bit for bit,
    gradients included, in a preference step -- the size at which the pages'
    streamed gradients went silently wrong (gate walkthrough section 2.5,
    "Fine-Tune 8B Models on 4GB VRAM", "Boundary Conditions List"). Also with
    every released slot poisoned (NaN block scales written after its free
    event): no kernel reads a slot after its release."""
    require_gpu()
    world32 = stack32b.setup()
    assert world32["shards"].layout.nbytes > 165 * 2**20
    a, b = stack32b.run(world32, "streamed"), stack32b.run(world32, "resident")
    _same(a, b)
    c = stack32b.run(world32, "streamed", poison=True)
    _same(c, b)
    for i in range(stack32b.N_LAYERS):
        for p in TARGETS:
            assert np.count_nonzero(a[("g", i, p, "dA")]) > 0
            assert np.count_nonzero(a[("g", i, p, "dB")]) > 0


def test_32b_layers_serialized_equals_async(tmp_path):
    """The same streamed 32B-class preference step in a child process with
    every kernel and copy serialised (AMD_SERIALIZE_KERNEL=3,
    AMD_SERIALIZE_COPY=3: no overlap of copy and compute at all) gives the
    asynchronous run's bits: the overlap changes no value."""
    require_gpu()
    out = str(tmp_path / "serial.npz")
    env = dict(os.environ, AMD_SERIALIZE_KERNEL="3", AMD_SERIALIZE_COPY="3")
    print("serialised child process", flush=True)
    r = subprocess.run([sys.executable, "-m", "tests.stack32b", out], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    serial = dict(np.load(out))
    got = stack32b.run(stack32b.setup(), "streamed")
    assert set(serial) == {stack32b.key_str(k) for k in got}
    for k, v in got.items():
        assert np.array_equal(v.view(np.uint8), serial[stack32b.key_str(k)].view(np.uint8)), k
