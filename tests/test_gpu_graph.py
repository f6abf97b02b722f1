"""The verify call captured into a HIP graph (through torch.cuda.CUDAGraph)
and replayed: the library launches kernels only (no allocation, no memset, no
host synchronisation), so every replay must give the eager result bitwise.
Inputs change between replays (copied into the captured buffers), with eager
work and synchronisations in between."""
from __future__ import annotations

import pytest
import torch

from mla_tree_verify_amd import _lib, api, gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("prefix,nsplit,merge", [(16384, 0, 0), (256, 0, 0), (150, 0, 1), (300, 1, 0)])
def test_graph_replays_match_eager(prefix, nsplit, merge):
    """merge = 1 at prefix 150: the split kernel merges its 3 splits (tickets
    in the workspace, reset by the last workgroup, same epoch on every replay)."""
    cases = [gen.make_case(9, prefix, tree="random", seed=500 + k) for k in range(3)]
    bufs = {k: getattr(cases[0], k).to(DEV) for k in ("q_nope", "q_rope", "kv_latent", "k_rope", "tree_parent")}
    n = prefix + 9
    ws = torch.zeros(max(16, _lib.workspace_size(9, 64, 1, n, n, nsplit=nsplit, merge=merge)), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty(9, 64, 512, dtype=torch.float32, device=DEV)
    lse = torch.empty(9, 64, dtype=torch.float32, device=DEV)

    def call():
        api.mla_verify(bufs["q_nope"], bufs["q_rope"], bufs["kv_latent"], bufs["k_rope"], bufs["tree_parent"],
                       prefix, cases[0].scale, out=out, lse=lse, workspace=ws, nsplit=nsplit, merge=merge)

    # eager references
    refs = []
    for c in cases:
        for k in bufs:
            bufs[k].copy_(getattr(c, k).to(DEV))
        call()
        torch.cuda.synchronize()
        refs.append((out.clone(), lse.clone()))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(6):
        k = rep % 3
        for name in bufs:
            bufs[name].copy_(getattr(cases[k], name).to(DEV))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, refs[k][0]) and torch.equal(lse, refs[k][1]), f"replay {rep} differs from eager"
        # eager work between replays
        torch.randn(1000, device=DEV).sum().item()


def test_graph_replays_match_eager_ragged_batch():
    """A ragged batch (the chunk list built from the offsets on the device):
    three batches with the same shapes but different offsets and data, one
    captured call replayed on each."""
    lens = [[300, 2500, 41, 1200], [1500, 900, 1300, 341], [41, 41, 3900, 59]]
    cases = [gen.make_batched_case(4, 9, prefix_lens=[n - 9 for n in ls], tree="random", seed=510 + k)
             for k, ls in enumerate(lens)]
    total = sum(lens[0])
    assert all(sum(ls) == total for ls in lens)
    max_kv = max(max(ls) for ls in lens)
    bufs = {k: getattr(cases[0], k).to(DEV)
            for k in ("q_nope", "q_rope", "kv_latent", "k_rope", "tree_parent", "kv_offsets")}
    ws = torch.zeros(max(16, _lib.workspace_size(9, 64, 4, total, max_kv)), dtype=torch.uint8, device=DEV)
    out = torch.empty(4, 9, 64, 512, dtype=torch.float32, device=DEV)
    lse = torch.empty(4, 9, 64, dtype=torch.float32, device=DEV)

    def call():
        api.mla_verify_batched(bufs["q_nope"], bufs["q_rope"], bufs["kv_latent"], bufs["k_rope"],
                               bufs["tree_parent"], bufs["kv_offsets"], cases[0].scale, max_kv=max_kv, out=out,
                               lse=lse, workspace=ws)

    refs = []
    for c in cases:
        for k in bufs:
            bufs[k].copy_(getattr(c, k).to(DEV))
        call()
        torch.cuda.synchronize()
        refs.append((out.clone(), lse.clone()))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(6):
        k = (2 * rep + 1) % 3
        for name in bufs:
            bufs[name].copy_(getattr(cases[k], name).to(DEV))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, refs[k][0]) and torch.equal(lse, refs[k][1]), f"replay {rep} differs from eager"
        torch.randn(1000, device=DEV).sum().item()
