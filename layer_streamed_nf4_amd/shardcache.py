"""Shard cache: a quantised shard set on disk, keyed by method and source.

The quantiser runs once per tensor and its bytes are reused ("shards ready"
when nothing has to be re-quantised: gate walkthrough "Soup layer-streamed NF4
training measured", section 5), and a shard set is only valid for the method,
block parameters, code tables and source weights it was made from (same page,
sections 2.1 and 2.4: the sharder and the reader must agree on the
quantisation keys; a mismatch is refused rather than silently degraded). A
cached set is therefore keyed by

  format, method (nf4), blocksize, nested block, double quant, the library's
  table hash, the per-projection shapes, the number of layers, the byte layout
  of a layer, and a caller-supplied fingerprint of the source weights,

and `load` raises `ShardCacheMismatch` naming the first field that differs,
or a corrupted / missing layer. Layout on disk: `manifest.json` plus one raw
file per layer (`layer_00000.bin` ...), each with its SHA-256 in the manifest.
Writes go to a temporary directory renamed into place, so a crash never leaves
a half-written cache that looks valid.
"""
from __future__ import annotations

import hashlib
import json
import os
import shutil
import tempfile

import numpy as np
import torch

from . import nf4s_table_hash
from .stack import PROJ, LayerLayout, ShardSet

FORMAT = "nf4stream-shards/1"
MANIFEST = "manifest.json"


class ShardCacheMismatch(RuntimeError):
    """The cache on disk was made for something else, or is damaged."""


def fingerprint_recipe(recipe: dict) -> str:
    """Fingerprint of weights that a recipe fully determines (seeded synthetic
    weights): SHA-256 of the recipe's canonical JSON."""
    return "recipe:" + hashlib.sha256(json.dumps(recipe, sort_keys=True).encode()).hexdigest()


def fingerprint_weights(weight_fn, shapes: dict, n_layers: int) -> str:
    """Fingerprint of the source weights themselves: SHA-256 over every fp32
    tensor in layer/projection order (reads each tensor back to the host)."""
    h = hashlib.sha256()
    for i in range(n_layers):
        for p in PROJ:
            w = weight_fn(i, p)
            assert tuple(w.shape) == tuple(shapes[p])
            h.update(w.detach().to("cpu", torch.float32).contiguous().numpy().tobytes())
    return "weights:" + h.hexdigest()


def cache_key(shapes: dict, n_layers: int, source_fingerprint: str) -> dict:
    lay = LayerLayout(shapes)
    return {
        "format": FORMAT,
        "method": "nf4",
        "blocksize": 64,
        "nested_block": 256,
        "double_quant": 1,
        "table_hash": f"{nf4s_table_hash():016x}",
        "shapes": {p: [int(shapes[p][0]), int(shapes[p][1])] for p in PROJ},
        "n_layers": int(n_layers),
        "layer_bytes": int(lay.nbytes),
        "layout": {p: [int(d.off_packed), int(d.off_q8), int(d.off_nested), int(d.off_offset), int(d.end)]
                   for p, d in lay.descs.items()},
        "source": source_fingerprint,
    }


def _layer_file(i: int) -> str:
    return f"layer_{i:05d}.bin"


def save(shards: ShardSet, path: str, source_fingerprint: str) -> None:
    """Write the shard set's host copies and the manifest under `path`
    (replacing an existing cache there)."""
    key = cache_key(shards.shapes, shards.n_layers, source_fingerprint)
    parent = os.path.dirname(os.path.abspath(path)) or "."
    os.makedirs(parent, exist_ok=True)
    tmp = tempfile.mkdtemp(prefix=".shards-", dir=parent)
    try:
        sums = []
        for i, h in enumerate(shards.host):
            b = h.cpu().numpy().tobytes()
            assert len(b) == key["layer_bytes"]
            with open(os.path.join(tmp, _layer_file(i)), "wb") as f:
                f.write(b)
            sums.append(hashlib.sha256(b).hexdigest())
        with open(os.path.join(tmp, MANIFEST), "w") as f:
            json.dump({"key": key, "layers_sha256": sums}, f, indent=1, sort_keys=True)
        if os.path.isdir(path):
            shutil.rmtree(path)
        os.replace(tmp, path)
    except BaseException:
        shutil.rmtree(tmp, ignore_errors=True)
        raise


def load(path: str, shapes: dict, n_layers: int, source_fingerprint: str,
         pinned: bool = True) -> ShardSet:
    """Load a cached shard set, refusing any mismatch of the key or damage to
    a layer file. pinned=True puts the layers in page-locked host memory, as
    the slot pool requires."""
    mpath = os.path.join(path, MANIFEST)
    if not os.path.isfile(mpath):
        raise ShardCacheMismatch(f"no shard cache at {path}")
    with open(mpath) as f:
        manifest = json.load(f)
    want = cache_key(shapes, n_layers, source_fingerprint)
    have = manifest.get("key", {})
    for field in want:
        if have.get(field) != want[field]:
            raise ShardCacheMismatch(f"cache key field {field!r} differs: cached {have.get(field)!r}, "
                                     f"expected {want[field]!r}")
    sums = manifest.get("layers_sha256", [])
    if len(sums) != n_layers:
        raise ShardCacheMismatch(f"manifest lists {len(sums)} layers, expected {n_layers}")
    host = []
    for i in range(n_layers):
        fp = os.path.join(path, _layer_file(i))
        if not os.path.isfile(fp):
            raise ShardCacheMismatch(f"layer file {fp} is missing")
        b = np.fromfile(fp, dtype=np.uint8)
        if b.size != want["layer_bytes"] or hashlib.sha256(b.tobytes()).hexdigest() != sums[i]:
            raise ShardCacheMismatch(f"layer {i} is damaged (size or checksum differs)")
        t = torch.from_numpy(b)
        host.append(t.pin_memory() if pinned else t)
    return ShardSet.from_host(shapes, n_layers, host)
