"""GPU parity at the largest sizes the boundary accepts: a sequence of
MLAV_MAX_KV rows (the byte offsets of one sequence's latent rows reach
4.1e9 of the 32-bit range the kernels use) and paged rows at the top of a
pool of MLAV_MAX_POOL rows, against the fp64 oracle element by element."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.mla_verify_oracle as orc
from mla_tree_verify_amd import api, gen

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 2e-3, 1e-2, 1e-3
DEV = "cuda:0"
MAX_KV = 4_000_000  # MLAV_MAX_KV
MAX_POOL = 4_000_000  # MLAV_MAX_POOL


def assert_parity(out, lse, ro, rl, what):
    o = out.cpu().double().numpy()
    err = np.abs(o - ro)
    bad = err > ATOL + RTOL * np.abs(ro)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside the bar, max err {err.max():.3e}"
    lerr = np.abs(lse.cpu().double().numpy() - rl).max()
    assert lerr <= LSE_TOL, f"{what}: lse err {lerr:.3e}"


def test_longest_sequence():
    q, heads = 2, 8
    case = gen.make_case(q, MAX_KV - q, tree="chain", num_heads=heads, seed=9100)
    print(f"longest sequence: {MAX_KV} kv rows, q {q}, H {heads}", flush=True)
    pl = api.device_plan(q, 1, MAX_KV, MAX_KV, num_heads=heads)
    out, lse = api.mla_verify(case.q_nope.to(DEV), case.q_rope.to(DEV), case.kv_latent.to(DEV),
                              case.k_rope.to(DEV), case.tree_parent.to(DEV), case.prefix_len, case.scale)
    torch.cuda.synchronize()
    ro, rl = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                            case.prefix_len, case.scale)
    assert_parity(out, lse, ro, rl, f"{MAX_KV} kv rows, {pl.nsplit} splits of {pl.chunk}")


def test_paged_rows_at_the_top_of_the_largest_pool():
    q, prefix = 9, 5000
    case = gen.make_case(q, prefix, tree="random", seed=9200)
    n = prefix + q
    print(f"paged: {n} logical rows in a pool of {MAX_POOL}", flush=True)
    g = torch.Generator().manual_seed(9201)
    # logical row j -> a distinct pool row among the last 2 n rows of the pool
    kv_index = (MAX_POOL - 1 - torch.randperm(2 * n, generator=g)[:n]).to(torch.int32)
    pool_lat = torch.empty(MAX_POOL, 512, dtype=torch.bfloat16, device=DEV)
    pool_rope = torch.empty(MAX_POOL, 64, dtype=torch.bfloat16, device=DEV)
    rows = kv_index.to(DEV).long()
    pool_lat.index_copy_(0, rows, case.kv_latent.to(DEV))
    pool_rope.index_copy_(0, rows, case.k_rope.to(DEV))
    out, lse = api.mla_verify_paged(case.q_nope.to(DEV), case.q_rope.to(DEV), pool_lat, pool_rope,
                                    kv_index.to(DEV), case.tree_parent.to(DEV), case.scale)
    torch.cuda.synchronize()
    ro, rl = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                            case.prefix_len, case.scale)
    assert_parity(out, lse, ro, rl, f"paged rows at the top of a {MAX_POOL}-row pool")
