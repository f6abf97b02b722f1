"""Plans of 2..4 KV splits (short prefixes) merged inside the split kernel
(option merge = 1): the last workgroup of each row block to finish merges that
block's int16 partials, so the call is one launch. Checked against the fp64 oracle (bar as
in the other parity tests: |out - ref| <= 2e-3 + 1e-2 |ref|, |lse - ref| <=
1e-3), against the separate combine kernel on the same partials, on a
workspace full of garbage, and for run-to-run determinism."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.mla_verify_oracle as orc
from mla_tree_verify_amd import _lib, api, gen

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 2e-3, 1e-2, 1e-3
DEV = "cuda:0"


def cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def assert_parity(out, lse, ref_out, ref_lse, label=""):
    o = out.double().numpy()
    l = lse.double().numpy()
    assert np.isfinite(o).all() and np.isfinite(l).all(), f"{label}: non-finite output"
    err = np.abs(o - ref_out)
    tol = ATOL + RTOL * np.abs(ref_out)
    assert (err <= tol).all(), f"{label}: worst err/tol {(err / tol).max():.3f}"
    assert np.abs(l - ref_lse).max() <= LSE_TOL, f"{label}: lse err {np.abs(l - ref_lse).max():.2e}"


def dev_inputs(case: gen.Case):
    return [getattr(case, k).to(DEV) for k in ("q_nope", "q_rope", "kv_latent", "k_rope", "tree_parent")]


def run(case: gen.Case, **kw):
    qn, qr, lat, rope, par = dev_inputs(case)
    out, lse = api.mla_verify(qn, qr, lat, rope, par, case.prefix_len, case.scale, **kw)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


# (q, heads, prefix, tree): 2, 3 and 4 splits, head counts below, at and above 64
CASES = [(9, 64, 150, "random"), (9, 64, 100, "random"), (9, 64, 220, "bounded"), (1, 64, 200, "random"),
         (33, 64, 150, "random"), (64, 64, 400, "random"), (9, 8, 180, "random"), (9, 16, 240, "chain"),
         (9, 128, 120, "random"), (5, 3, 150, "star")]


@pytest.mark.parametrize("q,heads,p,tree", CASES)
def test_merged_parity(q, heads, p, tree):
    n = p + q
    pl = _lib.plan(q, heads, 1, n, n, cus(), merge=1)
    assert 2 <= pl.nsplit <= 4 and pl.combine == 2, "the case must take the merged path"
    case = gen.make_case(q, p, tree=tree, seed=7000 + q + p + heads, num_heads=heads)
    out, lse = run(case, merge=1)
    ro, rl = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                            case.prefix_len, case.scale)
    assert_parity(out, lse, ro, rl, f"merged q{q} H{heads} p{p}")


@pytest.mark.parametrize("q,heads,p,tree", CASES[:6:2] + CASES[6:8])
def test_merged_equals_combine_kernel(q, heads, p, tree):
    """Same partials, two merge codes: equal up to the order of the sums."""
    case = gen.make_case(q, p, tree=tree, seed=7100 + q + p + heads, num_heads=heads)
    o1, l1 = run(case, merge=1)
    o2, l2 = run(case)
    assert torch.allclose(o1, o2, rtol=1e-5, atol=1e-6), (o1 - o2).abs().max()
    assert torch.allclose(l1, l2, rtol=1e-6, atol=1e-6), (l1 - l2).abs().max()


def test_merged_on_garbage_workspace_and_tickets_reset():
    """The ticket words need no clearing: a workspace of random bytes gives
    the bitwise result of a zeroed one, and every ticket is 0 after the call."""
    case = gen.make_case(9, 150, tree="random", seed=7200)
    n = 159
    need = _lib.workspace_size(9, 64, 1, n, n, merge=1)
    tickets = 9 * 8  # one 8-byte word per row block, at the end of the workspace
    qn, qr, lat, rope, par = dev_inputs(case)
    ws0 = torch.zeros(need, dtype=torch.uint8, device=DEV)
    o0, l0 = api.mla_verify(qn, qr, lat, rope, par, 150, case.scale, workspace=ws0, merge=1)
    g = torch.Generator().manual_seed(1)
    for k in range(3):
        ws = torch.randint(0, 256, (need,), dtype=torch.uint8, generator=g).to(DEV)
        if k == 2:  # every word a ticket of some other epoch with a count of 1
            ws[-tickets:].view(torch.int64).fill_((12345 << 16) | 1)
        o, l = api.mla_verify(qn, qr, lat, rope, par, 150, case.scale, workspace=ws, merge=1)
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(l, l0), f"garbage workspace {k}"
        assert int(ws[-tickets:].count_nonzero()) == 0, "tickets not reset"


def test_merged_batched_mixed_split_counts():
    """Sequences of 1, 2, 3 and 4 splits in one call: one-split sequences
    write directly, the others merge in the kernel."""
    lens = [30, 80, 150, 220]
    case = gen.make_batched_case(4, 9, prefix_lens=lens, tree="random", seed=7300)
    total = int(case.kv_offsets[-1])
    pl = _lib.plan(9, 64, 4, total, max(lens) + 9, cus(), merge=1)
    assert pl.combine == 2
    d = {k: getattr(case, k).to(DEV) for k in ("q_nope", "q_rope", "kv_latent", "k_rope", "tree_parent")}
    out, lse = api.mla_verify_batched(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                                      case.kv_offsets, case.scale, merge=1)
    torch.cuda.synchronize()
    ro, rl = orc.mla_verify_batched(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                                    case.kv_offsets, case.scale)
    assert_parity(out.cpu(), lse.cpu(), ro, rl, "merged batched")


def test_merged_paged():
    case = gen.make_case(9, 180, tree="random", seed=7400)
    pg = gen.make_paged(case, seed=7401, extra_rows=500)
    out, lse = api.mla_verify_paged(case.q_nope.to(DEV), case.q_rope.to(DEV), pg.pool_latent.to(DEV),
                                    pg.pool_rope.to(DEV), pg.kv_index.to(DEV), case.tree_parent.to(DEV), case.scale,
                                    merge=1)
    torch.cuda.synchronize()
    ro, rl = orc.mla_verify_paged(case.q_nope, case.q_rope, pg.pool_latent, pg.pool_rope, pg.kv_index,
                                  case.tree_parent, case.scale, prefix_len=case.prefix_len)
    assert_parity(out.cpu(), lse.cpu(), ro, rl, "merged paged")


def test_merged_run_to_run_bitwise():
    """Whichever workgroup arrives last, the merge reads the same partials in
    the same order: repeated calls on one workspace are bitwise equal."""
    case = gen.make_case(33, 150, tree="random", seed=7500)
    qn, qr, lat, rope, par = dev_inputs(case)
    ws = torch.empty(_lib.workspace_size(33, 64, 1, 183, 183, merge=1), dtype=torch.uint8, device=DEV)
    o0, l0 = api.mla_verify(qn, qr, lat, rope, par, 150, case.scale, workspace=ws, merge=1)
    o0, l0 = o0.clone(), l0.clone()
    for _ in range(20):
        o, l = api.mla_verify(qn, qr, lat, rope, par, 150, case.scale, workspace=ws, merge=1)
        assert torch.equal(o, o0) and torch.equal(l, l0)
    torch.cuda.synchronize()
