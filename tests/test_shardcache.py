"""Shard cache (host logic, no GPU): a saved shard set loads back byte for
byte, and every key field, a damaged layer or a missing file is refused.

Gate walkthrough ("Soup layer-streamed NF4 training measured"), sections 2.1
and 2.4: the sharder and the reader must agree on method, block parameters and
the shared tables; section 5: a cached shard set is reused as is.
"""
import json
import os

import numpy as np
import pytest
import torch

import layer_streamed_nf4_amd as L
import synth
from layer_streamed_nf4_amd import shardcache
from layer_streamed_nf4_amd.stack import LayerLayout, ShardSet

SHAPES = synth.SHAPES["135m"]
N = 2
FP = shardcache.fingerprint_recipe({"weights": "N(0,0.02)", "seed": 1234, "model": "135m"})


def _fake_set(seed=0):
    nb = LayerLayout(SHAPES).nbytes
    rng = np.random.Generator(np.random.PCG64(seed))
    host = [torch.from_numpy(rng.integers(0, 256, size=nb, dtype=np.uint8)) for _ in range(N)]
    return ShardSet.from_host(SHAPES, N, host)


def test_roundtrip(tmp_path):
    s = _fake_set()
    path = str(tmp_path / "cache")
    shardcache.save(s, path, FP)
    back = shardcache.load(path, SHAPES, N, FP, pinned=False)
    for a, b in zip(s.host, back.host):
        assert torch.equal(a, b)
    assert back.layout.nbytes == s.layout.nbytes


def test_key_contents():
    k = shardcache.cache_key(SHAPES, N, FP)
    assert (k["method"], k["blocksize"], k["nested_block"], k["double_quant"]) == ("nf4", 64, 256, 1)
    assert k["table_hash"] == f"{L.nf4s_table_hash():016x}"
    assert k["layer_bytes"] == LayerLayout(SHAPES).nbytes
    assert k["source"] == FP


def test_fingerprints_differ_per_recipe():
    a = shardcache.fingerprint_recipe({"seed": 1})
    assert a == shardcache.fingerprint_recipe({"seed": 1})
    assert a != shardcache.fingerprint_recipe({"seed": 2})


@pytest.mark.parametrize("field,value", [("table_hash", "0" * 16), ("blocksize", 32), ("double_quant", 0),
                                         ("method", "fp4"), ("format", "other/1"), ("layer_bytes", 1)])
def test_edited_key_is_refused(tmp_path, field, value):
    path = str(tmp_path / "cache")
    shardcache.save(_fake_set(), path, FP)
    mp = os.path.join(path, shardcache.MANIFEST)
    m = json.load(open(mp))
    m["key"][field] = value
    json.dump(m, open(mp, "w"))
    with pytest.raises(shardcache.ShardCacheMismatch, match=field):
        shardcache.load(path, SHAPES, N, FP, pinned=False)


def test_other_source_shapes_or_depth_are_refused(tmp_path):
    path = str(tmp_path / "cache")
    shardcache.save(_fake_set(), path, FP)
    with pytest.raises(shardcache.ShardCacheMismatch, match="source"):
        shardcache.load(path, SHAPES, N, shardcache.fingerprint_recipe({"seed": 9}), pinned=False)
    with pytest.raises(shardcache.ShardCacheMismatch, match="n_layers"):
        shardcache.load(path, SHAPES, N + 1, FP, pinned=False)
    other = dict(SHAPES)
    other["q"] = (576, 512)
    with pytest.raises(shardcache.ShardCacheMismatch, match="shapes"):
        shardcache.load(path, other, N, FP, pinned=False)


def test_damaged_or_missing_layer_is_refused(tmp_path):
    path = str(tmp_path / "cache")
    shardcache.save(_fake_set(), path, FP)
    f1 = os.path.join(path, "layer_00001.bin")
    b = bytearray(open(f1, "rb").read())
    b[12345] ^= 1
    open(f1, "wb").write(bytes(b))
    with pytest.raises(shardcache.ShardCacheMismatch, match="damaged"):
        shardcache.load(path, SHAPES, N, FP, pinned=False)
    os.remove(f1)
    with pytest.raises(shardcache.ShardCacheMismatch, match="missing"):
        shardcache.load(path, SHAPES, N, FP, pinned=False)
    with pytest.raises(shardcache.ShardCacheMismatch, match="no shard cache"):
        shardcache.load(str(tmp_path / "nowhere"), SHAPES, N, FP, pinned=False)


def test_save_replaces_existing_cache(tmp_path):
    path = str(tmp_path / "cache")
    shardcache.save(_fake_set(0), path, FP)
    new = _fake_set(1)
    shardcache.save(new, path, FP)
    back = shardcache.load(path, SHAPES, N, FP, pinned=False)
    assert all(torch.equal(a, b) for a, b in zip(new.host, back.host))
    assert not [d for d in os.listdir(tmp_path) if d.startswith(".shards-")]
