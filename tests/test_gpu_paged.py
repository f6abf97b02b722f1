"""GPU parity of the paged-KV entry point (one token per page) through the C ABI.

The page table scatters the logical KV rows over a larger pool filled with
large garbage values; the kernels must read exactly the mapped rows. Bar as
in the other parity tests: |out - ref| <= 2e-3 + 1e-2 |ref|, |lse - ref| <= 1e-3.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.mla_verify_oracle as orc
from mla_tree_verify_amd import api, gen

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 2e-3, 1e-2, 1e-3
DEV = "cuda:0"


def assert_parity(out, lse, ref_out, ref_lse, label=""):
    o = out.double().numpy()
    l = lse.double().numpy()
    assert np.isfinite(o).all() and np.isfinite(l).all(), f"{label}: non-finite output"
    err = np.abs(o - ref_out)
    tol = ATOL + RTOL * np.abs(ref_out)
    assert (err <= tol).all(), f"{label}: worst err/tol {(err / tol).max():.3f}"
    assert np.abs(l - ref_lse).max() <= LSE_TOL, f"{label}: lse err {np.abs(l - ref_lse).max():.2e}"


def run_paged(case: gen.Case, pg: gen.Paged, kv_index=None, **kw):
    idx = pg.kv_index if kv_index is None else kv_index
    offs = case.kv_offsets.to(DEV) if case.batched else None
    out, lse = api.mla_verify_paged(case.q_nope.to(DEV), case.q_rope.to(DEV), pg.pool_latent.to(DEV),
                                    pg.pool_rope.to(DEV), idx.to(DEV), case.tree_parent.to(DEV), case.scale,
                                    kv_offsets=offs, **kw)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def run_contiguous(case: gen.Case, **kw):
    d = {k: getattr(case, k).to(DEV) for k in ("q_nope", "q_rope", "kv_latent", "k_rope", "tree_parent")}
    out, lse = api.mla_verify(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                              case.prefix_len, case.scale, **kw)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def oracle_paged(case: gen.Case, pg: gen.Paged, kv_index=None):
    idx = pg.kv_index if kv_index is None else kv_index
    if case.batched:
        return orc.mla_verify_paged(case.q_nope, case.q_rope, pg.pool_latent, pg.pool_rope, idx, case.tree_parent,
                                    case.scale, kv_offsets=case.kv_offsets)
    return orc.mla_verify_paged(case.q_nope, case.q_rope, pg.pool_latent, pg.pool_rope, idx, case.tree_parent,
                                case.scale, prefix_len=case.prefix_len)


@pytest.mark.parametrize("q,p,tree,extra", [(1, 0, "random", 3), (5, 0, "star", 0), (9, 31, "random", 100),
                                            (9, 300, "random", 1000), (33, 2048, "bounded", 77),
                                            (9, 4096, "random", 4096), (64, 700, "random", 10)])
def test_paged_parity(q, p, tree, extra):
    case = gen.make_case(q, p, tree=tree, seed=2000 + q + p)
    pg = gen.make_paged(case, seed=3000 + q + p, extra_rows=extra)
    out, lse = run_paged(case, pg)
    ro, rl = oracle_paged(case, pg)
    assert_parity(out, lse, ro, rl, f"paged q{q} p{p}")


@pytest.mark.parametrize("partials", [0, 1])
def test_paged_bitwise_equals_contiguous(partials):
    """The gathered tiles are the same bytes in the same LDS places, so the
    result is bitwise the contiguous one (same plan)."""
    case = gen.make_workload("q9_p16384")
    pg = gen.make_paged(case, seed=5, extra_rows=20000)
    out, lse = run_paged(case, pg, partials=partials)
    o2, l2 = run_contiguous(case, partials=partials)
    assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_paged_batched():
    case = gen.make_batched_case(3, 9, prefix_lens=[100, 2500, 40], tree="random", seed=23)
    pg = gen.make_paged(case, seed=24, extra_rows=500)
    out, lse = run_paged(case, pg)
    ro, rl = oracle_paged(case, pg)
    assert_parity(out, lse, ro, rl, "paged batched")


def test_paged_valu_kernel():
    case = gen.make_case(9, 900, tree="random", seed=25)
    pg = gen.make_paged(case, seed=26, extra_rows=300)
    out, lse = run_paged(case, pg, kernel=1)
    ro, rl = oracle_paged(case, pg)
    assert_parity(out, lse, ro, rl, "paged valu")


def test_paged_entries_outside_the_pool_read_zero_rows():
    """Entries outside [0, pool_rows) are read as zero rows (no access out of
    bounds), in both kernels."""
    case = gen.make_case(9, 600, tree="random", seed=27)
    pg = gen.make_paged(case, seed=28, extra_rows=50)
    idx = pg.kv_index.clone()
    idx[[3, 100, 333, 599]] = torch.tensor([-1, -7, pg.pool_latent.shape[0], 2**31 - 1], dtype=torch.int32)
    ro, rl = oracle_paged(case, pg, kv_index=idx)
    for kernel in (0, 1):
        out, lse = run_paged(case, pg, kv_index=idx, kernel=kernel)
        assert_parity(out, lse, ro, rl, f"out-of-pool entries, kernel {kernel}")


@pytest.mark.parametrize("q,heads,p,tree", [(9, 8, 700, "random"), (5, 3, 300, "star"), (9, 128, 500, "random"),
                                            (33, 16, 1500, "bounded")])
def test_paged_head_counts(q, heads, p, tree):
    """Row blocks that several tokens share, or that pad past the last
    (token, head) row: the query block of each row block is read from rows
    that exist only, the padded rows read as zeros and are never stored."""
    case = gen.make_case(q, p, tree=tree, seed=4000 + q + p + heads, num_heads=heads)
    pg = gen.make_paged(case, seed=4100 + heads, extra_rows=300)
    out, lse = run_paged(case, pg)
    ro, rl = oracle_paged(case, pg)
    assert_parity(out, lse, ro, rl, f"paged H{heads} q{q} p{p}")


def test_paged_reference_max_restart():
    """The redo of a chunk after a weight overflow (a late key far above the
    first tile's max) reloads its first tiles through the page table."""
    case = gen.make_case(3, 200, tree="chain", seed=31, num_heads=64)
    case.kv_latent[150] = (case.q_nope[0, 0].float() * 0.5).to(torch.bfloat16)
    case.k_rope[150] = (case.q_rope[0, 0].float() * 0.5).to(torch.bfloat16)
    case.scale = 1.0
    pg = gen.make_paged(case, seed=33, extra_rows=100)
    for kw in ({}, {"nsplit": 3}):
        out, lse = run_paged(case, pg, **kw)
        ro, rl = oracle_paged(case, pg)
        assert_parity(out, lse, ro, rl, f"paged restart {kw}")


@pytest.mark.parametrize("batch,q,lo,hi,heads,seed", [(3, 9, 20, 2500, 64, 41), (70, 2, 4, 300, 8, 42)])
def test_paged_ragged_batch(batch, q, lo, hi, heads, seed):
    """Ragged batches through the page table: the chunk list path of the paged
    kernel, with one lane per sequence (3) and with groups of 64 (70)."""
    case = gen.make_batched_case(batch, q, prefix_lo=lo, prefix_hi=hi, tree="random", num_heads=heads, seed=seed)
    pg = gen.make_paged(case, seed=seed + 1, extra_rows=500)
    out, lse = run_paged(case, pg)
    ro, rl = oracle_paged(case, pg)
    assert_parity(out, lse, ro, rl, f"paged batch {batch}")
