"""A three-layer stack of 32B-class shapes (251.5 MB per layer shard, above the
165 MiB at which the pages' streamed gradients went wrong: "Fine-Tune 8B Models
on 4GB VRAM: Soup's Layer Streaming", failure records) in a preference step,
with seeded device inputs. Shared by the GPU stack tests and, run as

    python -m tests.stack32b OUT.npz

by the child process that repeats the streamed step with serialised kernels
and copies. No arithmetic of the method lives here.
"""
import sys

import numpy as np
import torch

import synth
from layer_streamed_nf4_amd.stack import PROJ, LinearStack, ShardSet

N_LAYERS, M = 3, 64
TARGETS = ("q", "v")


def setup():
    shapes = synth.SHAPES["32b"]
    g = torch.Generator(device="cuda")

    def weight_fn(i, p):
        g.manual_seed(synth.weight_seed(i, p))
        return torch.randn(shapes[p], generator=g, device="cuda") * 0.02

    shards = ShardSet(shapes, N_LAYERS, weight_fn)
    lora = []
    for i in range(N_LAYERS):
        d = {}
        for p in TARGETS:
            n, k = shapes[p]
            g.manual_seed(10_000 + 10 * i + PROJ.index(p))
            d[p] = (torch.randn((16, k), generator=g, device="cuda") * 0.01,
                    torch.randn((n, 16), generator=g, device="cuda") * 0.01)
        lora.append(d)
    g.manual_seed(77)
    xs = {p: torch.randn((M, shapes[p][1]), generator=g, device="cuda").to(torch.bfloat16) for p in PROJ}
    dys = {p: torch.randn((M, shapes[p][0]), generator=g, device="cuda").to(torch.bfloat16) for p in PROJ}
    return dict(shards=shards, lora=lora, xs=xs, dys=dys)


def run(world, mode, poison=False):
    st = LinearStack(world["shards"], M, TARGETS, world["lora"], n_slots=2, mode=mode, poison=poison)
    st.step(lambda i, p: world["xs"][p], lambda i, p: world["dys"][p], reference="separate")
    torch.cuda.synchronize()
    out = {("y",) + k: t.cpu().numpy().copy() for k, t in st.y.items()}
    out.update({("dx",) + k: t.cpu().numpy().copy() for k, t in st.dx.items()})
    out.update({("g",) + k: t.cpu().numpy().copy() for k, t in st.grads.items()})
    st.close()
    return out


def key_str(k):
    return "|".join(str(x) for x in k)


if __name__ == "__main__":
    res = run(setup(), "streamed")
    np.savez(sys.argv[1], **{key_str(k): v for k, v in res.items()})
    print("saved", len(res), "arrays", flush=True)
