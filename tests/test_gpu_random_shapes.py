"""Seeded random shapes through the C ABI against the fp64 oracle: query
length, head count, batch size and lengths (including empty prefixes), tree
shape, contiguous or paged KV, split count, partial format and the merge in
the split kernel, drawn together so that combinations no hand-picked case
names are exercised. Every output element meets the parity bar."""
from __future__ import annotations

import random

import numpy as np
import pytest
import torch

import oracle.mla_verify_oracle as orc
from mla_tree_verify_amd import api, gen

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 2e-3, 1e-2, 1e-3
DEV = "cuda:0"
N_CASES = 60


def draw(i: int):
    rng = random.Random(7000 + i)
    q = rng.choice([1, 2, 3, 5, 9, 16, 33, 64])
    heads = rng.choice([1, 3, 8, 16, 64, 64, 128])
    batch = rng.choice([1, 1, 2, 3, 5, 9])
    rows = q * heads * batch
    maxp = 4000 if rows <= 2048 else 600 if rows <= 8192 else 150
    spec = dict(q=q, heads=heads, batch=batch, tree=rng.choice(["random", "chain", "star", "bounded"]),
                paged=rng.random() < 0.25, merge=int(rng.random() < 0.15), partials=int(rng.random() < 0.2),
                nsplit=rng.choice([0, 0, 0, 1, 2, 3, 5]), extra=rng.choice([0, 17, 500]))
    if batch == 1:
        spec["prefix"] = rng.choice([0, 1, 31, 32, 33, rng.randrange(0, maxp)])
    else:
        spec["prefixes"] = [rng.choice([0, 1, 40, rng.randrange(0, maxp)]) for _ in range(batch)]
    return spec


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    sp = draw(i)
    if sp["batch"] == 1:
        case = gen.make_case(sp["q"], sp["prefix"], tree=sp["tree"], seed=8000 + i, num_heads=sp["heads"])
    else:
        case = gen.make_batched_case(sp["batch"], sp["q"], prefix_lens=sp["prefixes"], tree=sp["tree"],
                                     num_heads=sp["heads"], seed=8000 + i)
    kw = dict(nsplit=sp["nsplit"], partials=sp["partials"], merge=sp["merge"])
    d = {k: getattr(case, k).to(DEV) for k in ("q_nope", "q_rope", "kv_latent", "k_rope", "tree_parent")}
    if sp["paged"]:
        pg = gen.make_paged(case, seed=9000 + i, extra_rows=sp["extra"])
        offs = case.kv_offsets.to(DEV) if case.batched else None
        out, lse = api.mla_verify_paged(d["q_nope"], d["q_rope"], pg.pool_latent.to(DEV), pg.pool_rope.to(DEV),
                                        pg.kv_index.to(DEV), d["tree_parent"], case.scale, kv_offsets=offs, **kw)
        ro, rl = orc.mla_verify_paged(case.q_nope, case.q_rope, pg.pool_latent, pg.pool_rope, pg.kv_index,
                                      case.tree_parent, case.scale,
                                      **({"kv_offsets": case.kv_offsets} if case.batched
                                         else {"prefix_len": case.prefix_len}))
    elif case.batched:
        out, lse = api.mla_verify_batched(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                                          case.kv_offsets.to(DEV), case.scale, **kw)
        ro, rl = orc.mla_verify_batched(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                                        case.kv_offsets, case.scale)
    else:
        out, lse = api.mla_verify(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                                  case.prefix_len, case.scale, **kw)
        ro, rl = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                                case.prefix_len, case.scale)
    torch.cuda.synchronize()
    o = out.cpu().double().numpy()
    l = lse.cpu().double().numpy()
    assert np.isfinite(o).all() and np.isfinite(l).all(), f"{sp}: non-finite output"
    err = np.abs(o - ro)
    tol = ATOL + RTOL * np.abs(ro)
    assert (err <= tol).all(), f"{sp}: worst err/tol {(err / tol).max():.3f}"
    assert np.abs(l - rl).max() <= LSE_TOL, f"{sp}: lse err {np.abs(l - rl).max():.2e}"
