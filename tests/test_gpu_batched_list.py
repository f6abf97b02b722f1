"""Batched calls through the chunk list: every (sequence, split, row block)
item runs exactly where the list puts it, for ragged and equal lengths, up to
and past 64 sequences (one lane per sequence, then groups of 64), chunks that
end exactly on a sequence end, and a sequence with inconsistent offsets.

The workspace and the outputs start as NaN, so an item that never runs leaves
NaN partials (the combine then writes non-finite rows) or unwritten NaN rows;
every output element is compared with the fp64 oracle.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle.mla_verify_oracle as orc
from mla_tree_verify_amd import _lib, api, gen

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 2e-3, 1e-2, 1e-3
DEV = "cuda:0"


def run_nan_filled(case, max_kv=None, offsets=None, **kw):
    offs = case.kv_offsets if offsets is None else offsets
    if max_kv is None:
        max_kv = int((offs[1:] - offs[:-1]).max())
    d = {k: getattr(case, k).to(DEV) for k in ("q_nope", "q_rope", "kv_latent", "k_rope", "tree_parent")}
    bsz, q, h = case.q_nope.shape[:3]
    total = int(case.kv_latent.shape[0])
    opt = _lib.options(kw.get("nsplit", 0), 0, 0, kw.get("partials", 0), merge=kw.get("merge", 0))
    need = int(_lib.load().mla_verify_workspace_size(q, h, bsz, total, max_kv, 0, ctypes.byref(opt)))
    ws = torch.full((max(need, 4) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    out = torch.full((bsz, q, h, 512), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((bsz, q, h), float("nan"), dtype=torch.float32, device=DEV)
    api.mla_verify_batched(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                           offs.to(DEV), case.scale, max_kv=max_kv, out=out, lse=lse, workspace=ws, **kw)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def check(out, lse, ref_out, ref_lse, label):
    assert np.isfinite(out).all() and np.isfinite(lse).all(), f"{label}: non-finite output (an item did not run)"
    err = np.abs(out - ref_out)
    tol = ATOL + RTOL * np.abs(ref_out)
    assert (err <= tol).all(), f"{label}: worst err/tol {(err / tol).max():.3f}"
    assert np.abs(lse - ref_lse).max() <= LSE_TOL, f"{label}: lse"


def oracle(case):
    return orc.mla_verify_batched(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                                  case.kv_offsets, case.scale)


@pytest.mark.parametrize("batch,q,lo,hi,heads,seed", [
    (2, 9, 40, 3000, 64, 1),     # two sequences, very different lengths
    (8, 5, 16, 1500, 64, 2),     # several length classes of the last chunk
    (64, 3, 8, 400, 16, 3),      # exactly one lane per sequence
    (65, 3, 8, 400, 16, 4),      # one past: the grouped search
    (150, 2, 4, 300, 8, 5),      # three groups of sequences
    (12, 33, 30, 900, 8, 6),     # several row blocks per token group
    (256, 1, 2, 60, 4, 12),      # four full groups, loaded at once
    (300, 1, 2, 120, 4, 11),     # five groups of 64 sequences, one row block each
    (1000, 2, 2, 200, 4, 21),    # sixteen groups
    (4096, 1, 1, 16, 2, 23),     # 64 groups of short sequences, several rounds of workgroups per CU
])
def test_ragged_batches(batch, q, lo, hi, heads, seed):
    case = gen.make_batched_case(batch, q, prefix_lo=lo, prefix_hi=hi, tree="random", num_heads=heads, seed=seed)
    out, lse = run_nan_filled(case)
    ro, rl = oracle(case)
    check(out, lse, ro, rl, f"B{batch} q{q}")


@pytest.mark.parametrize("nsplit", [0, 3])
def test_equal_lengths(nsplit):
    case = gen.make_batched_case(6, 9, prefix_lens=[700] * 6, tree="random", num_heads=32, seed=7)
    out, lse = run_nan_filled(case, nsplit=nsplit)
    ro, rl = oracle(case)
    check(out, lse, ro, rl, f"equal nsplit {nsplit}")


def test_chunks_ending_on_sequence_ends():
    """Forced 4 splits of the longest sequence (1024 rows): chunk 256, and the
    other lengths are whole multiples of it (no shorter last chunk) or one past."""
    q = 4
    lens = [1024, 256, 512, 257, 768, 1023]
    case = gen.make_batched_case(len(lens), q, prefix_lens=[n - q for n in lens], tree="random", num_heads=16,
                                 seed=8)
    pl = _lib.plan(q, 16, len(lens), sum(lens), max(lens), 256, nsplit=4)
    assert pl.chunk == 256
    out, lse = run_nan_filled(case, nsplit=4)
    ro, rl = oracle(case)
    check(out, lse, ro, rl, "whole chunks")


@pytest.mark.parametrize("merge", [0, 1])
def test_merge_in_split_kernel_batched(merge):
    case = gen.make_batched_case(5, 9, prefix_lens=[300, 40, 1200, 700, 90], tree="random", num_heads=64, seed=9)
    out, lse = run_nan_filled(case, nsplit=3, merge=merge)
    ro, rl = oracle(case)
    check(out, lse, ro, rl, f"merge {merge}")


def test_inconsistent_sequence_next_to_valid_ones():
    """Sequence 1's end is moved below its start: its rows are NaN, the
    others (whose bounds are consistent) stay exact."""
    case = gen.make_batched_case(4, 9, prefix_lens=[120, 300, 60, 500], tree="random", num_heads=64, seed=10)
    bad = case.kv_offsets.clone()
    bad[2] = bad[1] - 3
    out, lse = run_nan_filled(case, max_kv=600, offsets=bad)
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    ro, rl = oracle(case)
    offs = case.kv_offsets.tolist()
    for b in (0, 3):
        check(out[b], lse[b], ro[b], rl[b], f"seq {b}")
    # sequence 2 now reads rows [offs[1] - 3, offs[3]): its own query against those keys
    sub = gen.Case(q_nope=case.q_nope[2:3].contiguous(), q_rope=case.q_rope[2:3].contiguous(),
                   kv_latent=case.kv_latent, k_rope=case.k_rope, tree_parent=case.tree_parent[2:3].contiguous(),
                   prefix_len=0, scale=case.scale,
                   kv_offsets=torch.tensor([0, offs[3] - offs[1] + 3], dtype=torch.int64))
    sub.kv_latent = case.kv_latent[offs[1] - 3:offs[3]].contiguous()
    sub.k_rope = case.k_rope[offs[1] - 3:offs[3]].contiguous()
    r2o, r2l = oracle(sub)
    check(out[2], lse[2], r2o[0], r2l[0], "seq 2 (widened)")
