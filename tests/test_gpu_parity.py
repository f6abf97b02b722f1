"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar, element by element: |out - ref| <= 2e-3 + 1e-2 |ref| and |lse - ref| <= 1e-3.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle.mla_verify_oracle as orc
from mla_tree_verify_amd import _lib, api, gen

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 2e-3, 1e-2, 1e-3
DEV = "cuda:0"


def dev_case(case: gen.Case):
    d = {k: getattr(case, k).to(DEV) for k in ("q_nope", "q_rope", "kv_latent", "k_rope", "tree_parent")}
    if case.batched:
        d["kv_offsets"] = case.kv_offsets.to(DEV)
    return d


def run(case: gen.Case, **kw):
    d = dev_case(case)
    if case.batched:
        out, lse = api.mla_verify_batched(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"],
                                          d["tree_parent"], d["kv_offsets"], case.scale,
                                          max_kv=int((case.kv_offsets[1:] - case.kv_offsets[:-1]).max()), **kw)
    else:
        out, lse = api.mla_verify(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                                  case.prefix_len, case.scale, **kw)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def oracle(case: gen.Case):
    if case.batched:
        return orc.mla_verify_batched(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                                      case.kv_offsets, case.scale)
    return orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                          case.prefix_len, case.scale)


def assert_parity(out, lse, ref_out, ref_lse, label=""):
    o = out.double().numpy()
    l = lse.double().numpy()
    assert np.isfinite(o).all() and np.isfinite(l).all(), f"{label}: non-finite output"
    err = np.abs(o - ref_out)
    tol = ATOL + RTOL * np.abs(ref_out)
    bad = err > tol
    assert not bad.any(), (f"{label}: {int(bad.sum())} of {bad.size} outputs off; worst err/tol "
                           f"{(err / tol).max():.3f} at {np.unravel_index((err / tol).argmax(), err.shape)}")
    lerr = np.abs(l - ref_lse).max()
    assert lerr <= LSE_TOL, f"{label}: lse max err {lerr:.2e}"


# ---------------------------------------------------------------------------
# small and edge shapes: prefix around tile (32) and chunk boundaries, q from 1 to 64
# ---------------------------------------------------------------------------
EDGE = [
    (1, 0, "random"), (1, 1, "star"), (2, 0, "chain"), (5, 0, "star"), (9, 0, "random"),
    (9, 1, "random"), (9, 22, "random"), (9, 23, "chain"), (9, 24, "random"), (9, 31, "random"),
    (9, 32, "star"), (9, 33, "random"), (9, 55, "random"), (9, 63, "chain"), (9, 64, "random"),
    (9, 65, "random"), (9, 100, "bounded"), (9, 256, "random"), (9, 1000, "random"),
    (33, 0, "bounded"), (33, 31, "bounded"), (33, 128, "random"), (33, 512, "bounded"),
    (33, 2048, "bounded"), (64, 0, "random"), (64, 7, "chain"), (64, 300, "random"), (64, 1000, "star"),
    (17, 4096, "random"), (3, 9999, "chain"),
]


@pytest.mark.parametrize("q,p,tree", EDGE)
def test_edge_shapes(q, p, tree):
    case = gen.make_case(q, p, tree=tree, seed=1000 + 7 * q + p)
    out, lse = run(case)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, f"q{q} p{p} {tree}")


@pytest.mark.parametrize("name", sorted(gen.WORKLOADS))
def test_workloads_full_size(name):
    case = gen.make_workload(name)
    out, lse = run(case)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, name)


def test_chunk_boundaries():
    """The benchmark workload's chunk (608 keys on 256 CUs) as an explicit plan, with the
    sequence ending just before, at and just after one, two and three chunk
    boundaries (mla_verify_partials splits exactly at multiples of the chunk;
    the combine kernel merges)."""
    pl = api.device_plan(9, 1, 16393, 16393)
    c = int(pl.chunk)
    for n in (c - 1, c, c + 1, 2 * c - 1, 2 * c, 2 * c + 1, 3 * c):
        case = gen.make_case(9, n - 9, tree="random", seed=n)
        d = dev_case(case)
        plan = _lib.Plan(-(-n // c), 32, c, 0, 0)
        po, pls = api.mla_verify_partials(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                                          n - 9, case.scale, plan)
        out, lse = api.combine(po, pls)
        torch.cuda.synchronize()
        ro, rl = oracle(case)
        assert_parity(out.cpu().view(9, 64, 512), lse.cpu().view(9, 64), ro, rl, f"n={n} (chunk {c})")


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_split_count_invariance():
    case = gen.make_case(9, 3000, tree="random", seed=77)
    ro, rl = oracle(case)
    outs = {}
    for ns in (1, 2, 3, 7, 0, 94):
        out, lse = run(case, nsplit=ns, partials=1)  # fp32 partials: only reassociation differs
        assert_parity(out, lse, ro, rl, f"nsplit={ns}")
        outs[ns] = (out, lse)
    base_o, base_l = outs[1]
    scale = base_o.abs().max().item()
    for ns, (o, l) in outs.items():
        assert (o - base_o).abs().max().item() <= 1e-5 * scale + 1e-6, f"nsplit {ns} differs"
        assert (l - base_l).abs().max().item() <= 1e-5


def test_masked_tree_rows_do_not_matter_bitwise():
    case = gen.make_case(9, 700, tree="random", seed=5)
    out, lse = run(case)
    anc = orc.ancestors_inclusive(case.tree_parent.tolist())
    for i in range(9):
        c2 = gen.make_case(9, 700, tree="random", seed=5)
        for u in range(9):
            if u not in anc[i]:
                c2.kv_latent[700 + u] = 1e4 if u % 2 else -1e4
                c2.k_rope[700 + u] = -1e4 if u % 2 else 1e4
        o2, l2 = run(c2)
        assert torch.equal(o2[i], out[i]) and torch.equal(l2[i], lse[i]), f"token {i} changed"


def test_head_permutation():
    case = gen.make_case(9, 500, tree="random", seed=9)
    out, lse = run(case)
    perm = torch.randperm(64, generator=torch.Generator().manual_seed(3))
    c2 = gen.make_case(9, 500, tree="random", seed=9)
    c2.q_nope = c2.q_nope[:, perm].contiguous()
    c2.q_rope = c2.q_rope[:, perm].contiguous()
    o2, l2 = run(c2)
    assert (o2 - out[:, perm]).abs().max().item() <= 1e-6
    assert (l2 - lse[:, perm]).abs().max().item() <= 1e-6


def test_run_to_run_bitwise():
    case = gen.make_workload("q9_p4096")
    o1, l1 = run(case)
    o2, l2 = run(case)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_batched_equals_per_sequence():
    case = gen.make_batched_case(4, 9, prefix_lens=[100, 3000, 33, 1500], tree="random", seed=21)
    out, lse = run(case)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, "batched")
    offs = case.kv_offsets.tolist()
    for b in range(4):
        single = gen.Case(q_nope=case.q_nope[b].contiguous(), q_rope=case.q_rope[b].contiguous(),
                          kv_latent=case.kv_latent[offs[b]:offs[b + 1]].contiguous(),
                          k_rope=case.k_rope[offs[b]:offs[b + 1]].contiguous(),
                          tree_parent=case.tree_parent[b].contiguous(), prefix_len=offs[b + 1] - offs[b] - 9,
                          scale=case.scale)
        o, l = run(single)
        assert_parity(o, l, ro[b], rl[b], f"seq {b}")


def test_bad_offsets_give_nan_not_fault():
    case = gen.make_batched_case(2, 9, prefix_lens=[100, 200], tree="random", seed=2)
    d = dev_case(case)
    bad = case.kv_offsets.clone()
    bad[1] = 5  # sequence 0 shorter than its tree
    out, lse = api.mla_verify_batched(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                                      bad.to(DEV), case.scale, max_kv=300)
    torch.cuda.synchronize()
    assert torch.isnan(out[0]).all() and torch.isnan(lse[0]).all()


# ---------------------------------------------------------------------------
# numerically special inputs
# ---------------------------------------------------------------------------
def test_reference_max_restart():
    """A late key whose score is far above the first tile's max (about 400 in
    log2 units: its weight overflows fp32) takes the redo-the-chunk path; the
    result stays exact."""
    case = gen.make_case(3, 200, tree="chain", seed=31, num_heads=64)
    case.kv_latent[150] = (case.q_nope[0, 0].float() * 0.5).to(torch.bfloat16)
    case.k_rope[150] = (case.q_rope[0, 0].float() * 0.5).to(torch.bfloat16)
    case.scale = 1.0
    ro, rl = oracle(case)
    for kw in ({}, {"nsplit": 3}, {"nsplit": 3, "merge": 1}):
        out, lse = run(case, **kw)
        assert_parity(out, lse, ro, rl, f"restart {kw}")


def test_large_weights_without_restart():
    """A late key about 100 (log2 units) above the first tile's max: its
    weight 2^100 is still finite in fp32, so the chunk runs once, and the
    result (that row is nearly one-hot on the late key) stays exact."""
    case = gen.make_case(3, 200, tree="chain", seed=32, num_heads=64)
    q0 = torch.cat([case.q_nope[0, 0].float(), case.q_rope[0, 0].float()])
    case.scale = 0.25
    c = 81.0 / (case.scale * float(q0 @ q0))  # score of row (0, 0) on key 150: about 81 natural
    case.kv_latent[150] = (case.q_nope[0, 0].float() * c).to(torch.bfloat16)
    case.k_rope[150] = (case.q_rope[0, 0].float() * c).to(torch.bfloat16)
    out, lse = run(case)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, "weights near 2^100")


@pytest.mark.parametrize("nsplit", [1, 0])
def test_large_values_do_not_overflow_the_accumulators(nsplit):
    """Values up to about 2^30 (inside the 2^31 precondition) under weights
    near 2^95: the first tile's keys score 0, every later key scores 88 (about
    127 in log2 units: below the score redo threshold), and all values are
    positive, so a chunk's fp32 sums pass 2^128 unless the kernel redoes the
    chunk with its own maximum as the reference. The exact result is the
    mean of the later keys' values."""
    case = gen.make_case(3, 2000, tree="chain", seed=33, num_heads=64)
    case.q_nope.zero_()
    case.q_rope.fill_(1.0)
    case.scale = 1.0
    case.k_rope[:32] = 0
    case.k_rope[32:] = 1.375  # 64 x 1.375 = 88
    case.kv_latent.copy_((case.kv_latent.float().abs() * 2.0 ** 28).to(torch.bfloat16))
    assert case.kv_latent.float().abs().max().item() < 2.0 ** 31
    ro, rl = oracle(case)
    out, lse = run(case, nsplit=nsplit)
    assert_parity(out, lse, ro, rl, f"values near 2^30, nsplit={nsplit}")


def test_peaky_single_key_dominates():
    case = gen.make_case(9, 777, tree="random", seed=41)
    case.scale = 4.0  # nearly one-hot softmax rows
    out, lse = run(case)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, "one-hot")


def test_single_bf16_weight_mode_on_normal_inputs():
    case = gen.make_workload("q9_p4096")
    out, lse = run(case, pv_mode=1)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, "pv_mode=1")


# ---------------------------------------------------------------------------
# the second (VALU) kernel and the combine kernel on their own
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("q,p,tree", [(9, 0, "star"), (9, 33, "random"), (33, 700, "bounded"), (9, 5000, "chain")])
def test_valu_kernel(q, p, tree):
    case = gen.make_case(q, p, tree=tree, seed=p + q)
    out, lse = run(case, kernel=1)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, f"valu q{q} p{p}")


@pytest.mark.parametrize("nsplit", [1, 2, 5, 28, 64])
def test_combine_kernel_on_synthetic_partials(nsplit):
    g = torch.Generator().manual_seed(nsplit)
    rows = 128
    part = torch.randn(nsplit, rows, 512, generator=g, dtype=torch.float32) * 3
    plse = torch.randn(nsplit, rows, generator=g, dtype=torch.float32) * 20
    if nsplit > 1:
        plse[0, :7] = -math.inf  # empty parts
        plse[:, 5] = -math.inf  # a row with nothing at all
    out, lse = api.combine(part.to(DEV), plse.to(DEV))
    torch.cuda.synchronize()
    ro, rl = orc.lse_merge(list(part.double().numpy()), list(plse.double().numpy()))
    o = out.cpu().double().numpy()
    assert np.abs(o - ro).max() <= 1e-5 * max(1.0, np.abs(ro).max())
    l = lse.cpu().double().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin)
    assert np.abs(l[fin] - rl[fin]).max() <= 1e-5 * max(1.0, np.abs(rl[fin]).max())


def test_workspace_too_small_is_rejected():
    case = gen.make_workload("q9_p16384")
    d = dev_case(case)
    with pytest.raises(_lib.MLAVError) as e:
        api.mla_verify(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                       case.prefix_len, case.scale, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == _lib.MLAV_ERR_WORKSPACE


def test_workspace_off_the_device_is_rejected():
    """A host or strided workspace never reaches the library (its pointer would
    be dereferenced on the GPU)."""
    case = gen.make_workload("q9_p4096")
    d = dev_case(case)
    args = (d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"], case.prefix_len, case.scale)
    need = _lib.workspace_size(case.q_len, 64, 1, case.prefix_len + case.q_len, case.prefix_len + case.q_len)
    assert need > 0
    with pytest.raises(ValueError, match="workspace"):
        api.mla_verify(*args, workspace=torch.empty(need, dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace"):
        api.mla_verify(*args, workspace=torch.empty(2 * need, dtype=torch.uint8, device=DEV)[::2])


def test_partials_then_combine_equals_full_call():
    case = gen.make_workload("q9_p16384")
    d = dev_case(case)
    out, lse = run(case, partials=1)
    pl = api.device_plan(case.q_len, 1, case.prefix_len + case.q_len, case.prefix_len + case.q_len)
    po, pls = api.mla_verify_partials(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                                      case.prefix_len, case.scale, pl)
    o2, l2 = api.combine(po, pls)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu().view_as(out), out) and torch.equal(l2.cpu().view_as(lse), lse)


def test_partials_merge_like_the_oracle_merge():
    """Forced 4-way split: the combine kernel and the oracle's merge formula
    give the same result from the same partials, and both match the oracle."""
    case = gen.make_case(9, 4000, tree="random", seed=88)
    ro, rl = oracle(case)
    d = dev_case(case)
    q = case.q_len
    pl = api.device_plan(q, 1, 4000 + q, 4000 + q, nsplit=4)
    po, pls = api.mla_verify_partials(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                                      4000, case.scale, pl)
    o_all, l_all = api.combine(po, pls)
    torch.cuda.synchronize()
    assert_parity(o_all.cpu().view(q, 64, 512), l_all.cpu().view(q, 64), ro, rl, "4 partials")
    m_o, m_l = orc.lse_merge(list(po.cpu().double().numpy()), list(pls.cpu().double().numpy()))
    assert np.abs(m_o - o_all.cpu().view(q, 64, 512).double().numpy()).max() <= 1e-5
    assert np.abs(m_l - l_all.cpu().view(q, 64).double().numpy()).max() <= 1e-5


@pytest.mark.parametrize("name", ["q9_p16384", "q33_p16384_peaky", "q9_p65536_chain"])
def test_compact_partials_within_bound(name):
    """int16 split partials (the default) against fp32 partials on the same
    split plan. Each stored partial is within scale/2 = (largest |value| of its
    row) / 65534 of the fp32 one; the combine takes a convex combination of the
    partials of a row and each partial row is a convex combination of value
    rows, so every output is within max|kv_latent| / 65534 of the fp32-partial
    output (plus fp32 rounding). The lse does not depend on the stored values;
    the two combine kernels add the split weights in different orders, so it
    agrees to fp32 reassociation."""
    case = gen.make_workload(name)
    oc, lc = run(case)
    of, lf = run(case, partials=1)
    bound = case.kv_latent.float().abs().max().item() / 65534.0
    diff = (oc - of).abs().max().item()
    assert diff <= bound * 1.01 + 1e-6, f"{name}: compact vs fp32 partials differ by {diff:.3e} > {bound:.3e}"
    assert (lc - lf).abs().max().item() <= 1e-6 * max(1.0, lf.abs().max().item())
    ro, rl = oracle(case) if name != "q9_p65536_chain" else (None, None)
    if ro is not None:
        assert_parity(oc, lc, ro, rl, f"{name} compact partials")


# ---------------------------------------------------------------------------
# head counts other than 64: a workgroup covers 64 consecutive (token, head)
# rows, so rows of several tokens (different tree masks) share a workgroup
# below 64 heads and a token spans several workgroups above
# ---------------------------------------------------------------------------
HEADS_CASES = [
    (8, 9, 4096, "random", 0), (8, 9, 300, "random", 0), (16, 9, 1000, "random", 0), (16, 33, 2048, "bounded", 0),
    (32, 9, 777, "chain", 0), (128, 9, 2000, "random", 0), (128, 33, 500, "bounded", 0), (1, 9, 300, "random", 0),
    (48, 5, 900, "random", 0), (8, 64, 1000, "random", 0),
    # chunks made of tree keys only: rows fix their reference max at their own first visible tile
    (8, 40, 0, "random", 0), (16, 40, 64, "random", 2), (64, 40, 64, "random", 2), (8, 64, 32, "chain", 3),
]


@pytest.mark.parametrize("heads,q,p,tree,nsplit", HEADS_CASES)
def test_head_counts(heads, q, p, tree, nsplit):
    case = gen.make_case(q, p, tree=tree, num_heads=heads, seed=4000 + heads + q + p)
    out, lse = run(case, nsplit=nsplit)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, f"H={heads} q={q} p={p}")


@pytest.mark.parametrize("q,p,nsplit", [(64, 40, 0), (9, 3000, 4)])
def test_max_head_count(q, p, nsplit):
    """MLAV_MAX_HEADS = 1024 heads: 64 x 1024 = 65 536 rows in 1024 row blocks
    (one split each), and 9 x 1024 rows over 4 forced splits (576 workgroups)."""
    case = gen.make_case(q, p, tree="random", num_heads=1024, seed=4500 + q + p)
    out, lse = run(case, nsplit=nsplit)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, f"H1024 q{q} p{p}")


@pytest.mark.parametrize("heads", [8, 128])
def test_head_counts_valu_kernel(heads):
    case = gen.make_case(9, 700, tree="random", num_heads=heads, seed=4100 + heads)
    out, lse = run(case, kernel=1)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, f"valu H={heads}")


def test_head_counts_batched():
    case = gen.make_batched_case(3, 9, prefix_lens=[100, 1500, 40], tree="random", num_heads=16, seed=4200)
    out, lse = run(case)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, "batched H=16")


def test_head_counts_partials_padded_rows():
    """q * H = 72 rows: partials come in two padded blocks of 64 rows and the
    combine of the first 72 equals the full call."""
    case = gen.make_case(9, 3000, tree="random", num_heads=8, seed=4300)
    d = dev_case(case)
    out, lse = run(case, partials=1)
    pl = api.device_plan(9, 1, 3009, 3009, num_heads=8)
    assert pl.nsplit > 1
    po, pls = api.mla_verify_partials(d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"],
                                      3000, case.scale, pl)
    assert tuple(po.shape) == (pl.nsplit, 128, 512)
    o2, l2 = api.combine(po, pls)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu()[:72].view_as(out), out) and torch.equal(l2.cpu()[:72].view_as(lse), lse)


@pytest.mark.parametrize("heads,prefix,nsplit", [(8, 6000, 0), (8, 3000, 20)])
def test_padding_rows_of_int16_partials_are_never_read(heads, prefix, nsplit):
    """q * H = 72 rows: the last row block is mostly padding, whose int16
    partial rows the split kernel does not store. A workspace of random bytes
    must give the bitwise result of a zeroed one (four-wave combine for the
    planner's split count at prefix 6000, one-wave combine for 19 splits at
    prefix 3000), which also matches the oracle."""
    case = gen.make_case(9, prefix, tree="random", num_heads=heads, seed=4600 + nsplit)
    d = dev_case(case)
    n = prefix + 9
    pl = api.device_plan(9, 1, n, n, nsplit=nsplit, num_heads=heads)
    assert (pl.nsplit > 32) == (nsplit == 0)  # four-wave combine, then the one-wave form
    need = _lib.workspace_size(9, heads, 1, n, n, nsplit=nsplit)
    assert need > 0
    args = (d["q_nope"], d["q_rope"], d["kv_latent"], d["k_rope"], d["tree_parent"], prefix, case.scale)
    o0, l0 = api.mla_verify(*args, workspace=torch.zeros(need, dtype=torch.uint8, device=DEV), nsplit=nsplit)
    g = torch.Generator().manual_seed(11)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, generator=g).to(DEV)
    o1, l1 = api.mla_verify(*args, workspace=ws, nsplit=nsplit)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    ro, rl = oracle(case)
    assert_parity(o1.cpu(), l1.cpu(), ro, rl, f"H {heads}, padded rows, nsplit {nsplit}")


@pytest.mark.parametrize("prefix,nsplit", [(4727, 74), (6391, 100), (4471, 140), (6007, 188)])
def test_wide_combine_batch_sizes(prefix, nsplit):
    """The four-wave combine at split counts whose per-wave share needs 20 and
    28 loads per lane, and past 128 splits (batches of 32 merged with a
    running max), against the oracle."""
    case = gen.make_case(9, prefix, tree="random", seed=4500 + nsplit)
    pl = api.device_plan(9, 1, prefix + 9, prefix + 9, nsplit=nsplit)
    assert pl.nsplit == nsplit
    out, lse = run(case, nsplit=nsplit)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, f"compact, {pl.nsplit} splits")


@pytest.mark.parametrize("nsplit", [5, 32, 33, 40, 100])
def test_compact_combine_split_counts(nsplit):
    """Both combine forms of the int16 partials (one wave per row up to 32
    splits, four waves per row beyond) against the oracle."""
    case = gen.make_case(9, 6000, tree="random", seed=4400 + nsplit)
    pl = api.device_plan(9, 1, 6009, 6009, nsplit=nsplit)
    out, lse = run(case, nsplit=nsplit)
    ro, rl = oracle(case)
    assert_parity(out, lse, ro, rl, f"compact, {pl.nsplit} splits")
