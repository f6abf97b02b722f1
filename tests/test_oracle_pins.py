"""Pins for the fp64 oracle: each ties it to something other than itself.

The pages print no output values for the verify kernel (they report only
error magnitudes against their own naive kernel), so the oracle is pinned by
the mathematics instead:

  pin 1  brute force of the UNABSORBED form in pure-Python loops (math.fsum)
         with random per-head up-projections: absorbing W_UK into the query
         and applying W_UV to the latent output must give the same result,
         by associativity;
  pin 2  torch's scaled_dot_product_attention and logsumexp in float64, with
         the tree mask built by boolean transitive closure;
  pin 3  closed forms: a single visible key, identical keys, equal scores
         (mean of the visible values), chain tree == causal block, and head
         permutation equivariance;
  pin 5  the LSE merge of results over disjoint key subsets equals the
         result over their union.

``test_pins_catch_planted_mistakes`` plants plausible mistakes in the oracle
(monkeypatched, CPU only) and checks that some pin fails for each.
"""
from __future__ import annotations

import math
import random

import numpy as np
import pytest
import torch

import oracle.mla_verify_oracle as orc
from mla_tree_verify_amd import gen

TOL = 1e-12


# --------------------------------------------------------------------------
# pin 1: brute force, unabsorbed form
# --------------------------------------------------------------------------
def _closure_dp(parent):
    """anc*(i) by dynamic programming over the topological order."""
    anc = []
    for i, p in enumerate(parent):
        s = {i}
        if p >= 0:
            s |= anc[p]
        anc.append(s)
    return anc


def brute_force_unabsorbed(qn_u, qr, lat, rope, w_uk, w_uv, parent, prefix_len, scale):
    """Pure-Python loops. qn_u [q][H][d_nope] is the UNabsorbed nope query;
    keys/values are up-projected per head: k = W_UK[h] L[j], v = W_UV[h] L[j]."""
    q = len(parent)
    heads = len(w_uk)
    anc = _closure_dp(parent)
    out, lse = [], []
    for i in range(q):
        keys = list(range(prefix_len)) + [prefix_len + t for t in range(q) if t in anc[i]]
        out_i, lse_i = [], []
        for h in range(heads):
            scores = []
            vals = []
            for j in keys:
                k_nope = [math.fsum(w_uk[h][d][c] * lat[j][c] for c in range(len(lat[j]))) for d in range(len(w_uk[h]))]
                v = [math.fsum(w_uv[h][e][c] * lat[j][c] for c in range(len(lat[j]))) for e in range(len(w_uv[h]))]
                terms = [qn_u[i][h][d] * k_nope[d] for d in range(len(k_nope))]
                terms += [qr[i][h][r] * rope[j][r] for r in range(len(rope[j]))]
                scores.append(scale * math.fsum(terms))
                vals.append(v)
            m = max(scores)
            e = [math.exp(s - m) for s in scores]
            l_ = math.fsum(e)
            out_i.append([math.fsum(e[k] * vals[k][c] for k in range(len(keys))) / l_ for c in range(len(vals[0]))])
            lse_i.append(m + math.log(l_))
        out.append(out_i)
        lse.append(lse_i)
    return np.array(out), np.array(lse)


def pin1_error(seed: int) -> float:
    rng = random.Random(seed)
    heads = rng.randint(1, 4)
    d_nope = rng.randint(4, 16)
    d_v = rng.randint(4, 16)
    dl = rng.randint(8, 32)
    dr = rng.randint(2, 8)
    prefix_len = rng.choice([0, 1, 3, 7])
    q = rng.randint(1, 6)
    g = torch.Generator().manual_seed(seed)
    parent = gen.random_tree(q, g)
    n = prefix_len + q
    lat = torch.randn(n, dl, generator=g, dtype=torch.float64)
    rope = torch.randn(n, dr, generator=g, dtype=torch.float64)
    qn_u = torch.randn(q, heads, d_nope, generator=g, dtype=torch.float64)
    qr = torch.randn(q, heads, dr, generator=g, dtype=torch.float64)
    w_uk, w_uv = gen.make_mla_weights(heads, d_nope, d_v, dl, seed + 1000)
    scale = float(np.float32(0.37))
    bo, bl = brute_force_unabsorbed(qn_u.tolist(), qr.tolist(), lat.tolist(), rope.tolist(),
                                    w_uk.tolist(), w_uv.tolist(), parent, prefix_len, scale)
    # absorbed: q_abs[i,h] = W_UK[h]^T q_nope[i,h]; output up-projected by W_UV afterwards
    q_abs = torch.einsum("hdc,ihd->ihc", w_uk, qn_u).numpy()
    o_lat, ol = orc.mla_verify(q_abs, qr.numpy(), lat.numpy(), rope.numpy(), parent, prefix_len, scale)
    o_v = np.einsum("hec,ihc->ihe", w_uv.numpy(), o_lat)
    return max(np.abs(o_v - bo).max(), np.abs(ol - bl).max())


@pytest.mark.parametrize("seed", range(12))
def test_pin1_bruteforce_unabsorbed(seed):
    assert pin1_error(seed) < TOL


# --------------------------------------------------------------------------
# pin 2: torch SDPA (float64, CPU) with a transitive-closure mask
# --------------------------------------------------------------------------
def closure_mask(parent, prefix_len) -> torch.Tensor:
    q = len(parent)
    a = torch.eye(q, dtype=torch.int64)
    for i, p in enumerate(parent):
        if p >= 0:
            a[i, p] = 1
    while True:  # boolean transitive closure by repeated squaring
        b = ((a + a @ a) > 0).to(torch.int64)
        if torch.equal(a, b):
            break
        a = b
    mask = torch.zeros(q, prefix_len + q, dtype=torch.bool)
    mask[:, :prefix_len] = True
    mask[:, prefix_len:] = a.bool()
    return mask


def sdpa_reference(case: gen.Case):
    qn = case.q_nope.double()
    qr = case.q_rope.double()
    lat = case.kv_latent.double()
    rope = case.k_rope.double()
    parent = case.tree_parent.tolist()
    p = case.prefix_len
    q, h, dl = qn.shape
    n = p + q
    sc = float(np.float32(case.scale))
    qq = torch.cat([qn, qr], -1).permute(1, 0, 2).contiguous()  # [H, q, 576]
    kk = torch.cat([lat, rope], -1).unsqueeze(0).expand(h, n, -1).contiguous()
    vv = lat.unsqueeze(0).expand(h, n, dl).contiguous()
    mask = closure_mask(parent, p)
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=sc)
    s = sc * torch.matmul(qq, kk.transpose(-1, -2))
    lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
    return out.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


def pin2_error(case: gen.Case) -> float:
    ro, rl = sdpa_reference(case)
    oo, ol = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope,
                            case.tree_parent, case.prefix_len, case.scale)
    return max(np.abs(oo - ro).max(), np.abs(ol - rl).max())


@pytest.mark.parametrize("q,p,tree,seed", [
    (9, 256, "random", 1),
    (9, 1024, "random", 2),
    (33, 512, "bounded", 3),
    (9, 4096, "chain", 4),
    (5, 0, "random", 5),
    (1, 17, "star", 6),
])
def test_pin2_sdpa_fp64(q, p, tree, seed):
    case = gen.make_case(q, p, tree=tree, seed=seed)
    assert pin2_error(case) < TOL


# --------------------------------------------------------------------------
# pin 3: closed forms and special cases
# --------------------------------------------------------------------------
def pin3_single_key_error() -> float:
    """P = 0 and a star tree: every token sees only itself, so out = its own
    latent row and lse = its one score."""
    case = gen.make_case(6, 0, tree="star", seed=11, num_heads=8)
    oo, ol = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope,
                            case.tree_parent, 0, case.scale)
    lat = case.kv_latent.double().numpy()
    rope = case.k_rope.double().numpy()
    qn = case.q_nope.double().numpy()
    qr = case.q_rope.double().numpy()
    sc = float(np.float32(case.scale))
    err = 0.0
    for i in range(6):
        err = max(err, np.abs(oo[i] - lat[i][None, :]).max())
        s_ii = sc * (qn[i] @ lat[i] + qr[i] @ rope[i])
        err = max(err, np.abs(ol[i] - s_ii).max())
    return err


def pin3_identical_keys_error() -> float:
    """All key rows identical: out = that row, lse = s + ln |V(i)|."""
    case = gen.make_case(7, 13, tree="random", seed=12, num_heads=4)
    n = 13 + 7
    case.kv_latent[:] = case.kv_latent[0]
    case.k_rope[:] = case.k_rope[0]
    oo, ol = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope,
                            case.tree_parent, 13, case.scale)
    lat0 = case.kv_latent[0].double().numpy()
    rope0 = case.k_rope[0].double().numpy()
    sc = float(np.float32(case.scale))
    anc = _closure_dp(case.tree_parent.tolist())
    err = np.abs(oo - lat0).max()
    for i in range(7):
        s = sc * (case.q_nope[i].double().numpy() @ lat0 + case.q_rope[i].double().numpy() @ rope0)
        err = max(err, np.abs(ol[i] - (s + math.log(13 + len(anc[i])))).max())
    assert n == case.kv_latent.shape[0]
    return err


def pin3_equal_scores_error() -> float:
    """q_nope = 0 and identical rope keys: all visible scores are equal, so
    out = mean of the visible latent rows and lse = sc*(q_pe . r) + ln |V(i)|."""
    case = gen.make_case(9, 21, tree="random", seed=13, num_heads=4)
    case.q_nope.zero_()
    case.k_rope[:] = case.k_rope[0]
    oo, ol = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope,
                            case.tree_parent, 21, case.scale)
    lat = case.kv_latent.double().numpy()
    r0 = case.k_rope[0].double().numpy()
    sc = float(np.float32(case.scale))
    anc = _closure_dp(case.tree_parent.tolist())
    err = 0.0
    for i in range(9):
        rows = list(range(21)) + [21 + t for t in sorted(anc[i])]
        mean = lat[rows].mean(axis=0)
        err = max(err, np.abs(oo[i] - mean[None, :]).max())
        expect = sc * (case.q_rope[i].double().numpy() @ r0) + math.log(len(rows))
        err = max(err, np.abs(ol[i] - expect).max())
    return err


def pin3_chain_causal_error() -> float:
    """A chain tree makes the tree block causal: SDPA with a lower-triangular block."""
    case = gen.make_case(9, 64, tree="chain", seed=14, num_heads=8)
    qn = case.q_nope.double()
    qr = case.q_rope.double()
    lat = case.kv_latent.double()
    rope = case.k_rope.double()
    sc = float(np.float32(case.scale))
    qq = torch.cat([qn, qr], -1).permute(1, 0, 2)
    kk = torch.cat([lat, rope], -1)
    mask = torch.ones(9, 64 + 9, dtype=torch.bool)
    mask[:, 64:] = torch.ones(9, 9, dtype=torch.bool).tril()
    s = sc * qq @ kk.T
    s = s.masked_fill(~mask, float("-inf"))
    ref = torch.softmax(s, -1) @ lat
    oo, _ = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope,
                           case.tree_parent, 64, case.scale)
    return np.abs(oo - ref.permute(1, 0, 2).numpy()).max()


def pin3_head_permutation_error() -> float:
    """Heads are independent and share one mask row: permuting the query heads
    permutes the outputs the same way."""
    case = gen.make_case(5, 30, tree="random", seed=15, num_heads=16)
    perm = torch.randperm(16, generator=torch.Generator().manual_seed(1))
    oo, ol = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope,
                            case.tree_parent, 30, case.scale)
    po, pl = orc.mla_verify(case.q_nope[:, perm], case.q_rope[:, perm], case.kv_latent, case.k_rope,
                            case.tree_parent, 30, case.scale)
    return max(np.abs(po - oo[:, perm.numpy()]).max(), np.abs(pl - ol[:, perm.numpy()]).max())


def test_pin3_single_visible_key():
    assert pin3_single_key_error() < TOL


def test_pin3_identical_keys():
    assert pin3_identical_keys_error() < TOL


def test_pin3_equal_scores_mean():
    assert pin3_equal_scores_error() < TOL


def test_pin3_chain_is_causal():
    assert pin3_chain_causal_error() < TOL


def test_pin3_head_permutation():
    assert pin3_head_permutation_error() < TOL


# --------------------------------------------------------------------------
# pin 5: LSE merge over disjoint key subsets == result over the union
# --------------------------------------------------------------------------
def pin5_error(nparts: int, seed: int) -> float:
    g = torch.Generator().manual_seed(seed)
    heads, dl, dr, n = 8, 32, 8, 200
    qn = torch.randn(heads, dl, generator=g, dtype=torch.float64).numpy()
    qr = torch.randn(heads, dr, generator=g, dtype=torch.float64).numpy()
    lat = torch.randn(n, dl, generator=g, dtype=torch.float64).numpy() * 2.0
    rope = torch.randn(n, dr, generator=g, dtype=torch.float64).numpy()
    scale = float(np.float32(0.3))
    cuts = sorted(torch.randperm(n - 1, generator=g)[: nparts - 1].add(1).tolist())
    bounds = [0] + cuts + [n]
    outs, lses = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        o, l = orc.attend_rows(qn, qr, lat[a:b], rope[a:b], scale)
        outs.append(o)
        lses.append(l)
    # an empty part (lse = -inf) must not change anything
    o, l = orc.attend_rows(qn, qr, lat[:0], rope[:0], scale)
    outs.append(o)
    lses.append(l)
    mo, ml = orc.lse_merge(outs, lses)
    ro, rl = orc.attend_rows(qn, qr, lat, rope, scale)
    return max(np.abs(mo - ro).max(), np.abs(ml - rl).max())


@pytest.mark.parametrize("nparts,seed", [(2, 0), (3, 1), (7, 2), (28, 3)])
def test_pin5_lse_merge(nparts, seed):
    assert pin5_error(nparts, seed) < TOL


def test_lse_merge_all_empty():
    o, l = orc.lse_merge([np.zeros((3, 4))] * 2, [np.full(3, -np.inf)] * 2)
    assert np.all(o == 0) and np.all(np.isneginf(l))


# --------------------------------------------------------------------------
# the oracle itself: tree handling
# --------------------------------------------------------------------------
def test_check_tree_rejects_bad_parents():
    for bad in ([0], [-2], [-1, 1], [-1, 0, 3]):
        with pytest.raises(ValueError):
            orc.check_tree(bad)
    orc.check_tree([-1, 0, 0, 1, -1])


def test_masked_rows_do_not_matter():
    """Overwriting tree rows invisible to token i leaves token i's output unchanged (bitwise)."""
    case = gen.make_case(9, 40, tree="random", seed=21, num_heads=8)
    oo, ol = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope,
                            case.tree_parent, 40, case.scale)
    anc = _closure_dp(case.tree_parent.tolist())
    for i in range(9):
        lat = case.kv_latent.clone()
        rope = case.k_rope.clone()
        for t in range(9):
            if t not in anc[i]:
                lat[40 + t] = 1e4
                rope[40 + t] = -1e4
        po, pl = orc.mla_verify(case.q_nope, case.q_rope, lat, rope, case.tree_parent, 40, case.scale)
        assert np.array_equal(po[i], oo[i]) and np.array_equal(pl[i], ol[i])


# --------------------------------------------------------------------------
# planted mistakes: every one must trip at least one pin
# --------------------------------------------------------------------------
def _all_pin_errors():
    errs = [pin1_error(s) for s in range(4)]
    errs.append(pin2_error(gen.make_case(9, 64, tree="random", seed=31, num_heads=8)))
    errs.append(pin2_error(gen.make_case(6, 0, tree="bounded", seed=32, num_heads=8)))
    errs += [pin3_single_key_error(), pin3_identical_keys_error(), pin3_equal_scores_error(),
             pin3_chain_causal_error(), pin3_head_permutation_error()]
    errs += [pin5_error(3, 7)]
    return errs


def _no_self(parent):
    return [[a for a in anc if a != i] for i, anc in enumerate(_orig_anc(parent))]


def _parent_only(parent):
    return [sorted({i} | ({int(parent[i])} if int(parent[i]) >= 0 else set())) for i in range(len(parent))]


_orig_anc = orc.ancestors_inclusive
_orig_attend = orc.attend_rows


def _attend_drop_rope(qn, qr, lat, rope, scale):
    return _orig_attend(qn, qr * 0.0, lat, rope, scale)


def _attend_lse_unshifted(qn, qr, lat, rope, scale):
    o, l = _orig_attend(qn, qr, lat, rope, scale)
    sc = orc.fp32_scale(scale)
    m = (sc * (qn @ lat.T + qr @ rope.T)).max(axis=1) if lat.shape[0] else 0.0
    return o, l - m


def _attend_log2_lse(qn, qr, lat, rope, scale):
    o, l = _orig_attend(qn, qr, lat, rope, scale)
    return o, l / math.log(2.0)


def _attend_wrong_sign_rope(qn, qr, lat, rope, scale):
    return _orig_attend(qn, -qr, lat, rope, scale)


def _attend_transposed_heads(qn, qr, lat, rope, scale):
    o, l = _orig_attend(qn, qr, lat, rope, scale)
    return o[::-1].copy(), l[::-1].copy()


def _tree_rows_shifted(parent):
    # node t read from row P + t - 1: plant it via the ancestor ids
    return [[max(a - 1, 0) for a in anc] for anc in _orig_anc(parent)]


PLANTED = {
    "no_self": ("ancestors_inclusive", _no_self),
    "parent_only": ("ancestors_inclusive", _parent_only),
    "tree_row_off_by_one": ("ancestors_inclusive", _tree_rows_shifted),
    "drop_rope": ("attend_rows", _attend_drop_rope),
    "rope_sign": ("attend_rows", _attend_wrong_sign_rope),
    "lse_no_max": ("attend_rows", _attend_lse_unshifted),
    "lse_log2": ("attend_rows", _attend_log2_lse),
    "heads_swapped": ("attend_rows", _attend_transposed_heads),
    "scale_sqrt576": ("fp32_scale", lambda s: float(np.float32(1.0 / math.sqrt(576.0)))),
}


def test_real_oracle_passes_all_pins():
    assert max(_all_pin_errors()) < TOL


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = PLANTED[name]
    monkeypatch.setattr(orc, attr, fn)
    try:
        errs = _all_pin_errors()
        worst = max(e for e in errs if np.isfinite(e)) if any(np.isfinite(errs)) else float("inf")
        caught = worst > 1e-6 or not all(np.isfinite(errs))
    except Exception:
        caught = True  # a crash is also a detection
    assert caught, f"planted mistake {name!r} slipped through every pin"


# ---------------------------------------------------------------------------
# paged KV: the gather through the page table
# ---------------------------------------------------------------------------
def test_paged_oracle_equals_contiguous_oracle():
    """Scattering the KV rows over a larger pool of garbage rows and reading
    them back through the page table gives exactly the contiguous result."""
    case = gen.make_case(5, 40, tree="random", seed=71, num_heads=4, dl=16, dr=4)
    pg = gen.make_paged(case, seed=72, extra_rows=25)
    ro, rl = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                            case.prefix_len, case.scale)
    po, pl = orc.mla_verify_paged(case.q_nope, case.q_rope, pg.pool_latent, pg.pool_rope, pg.kv_index,
                                  case.tree_parent, case.scale, prefix_len=case.prefix_len)
    assert np.array_equal(po, ro) and np.array_equal(pl, rl)


def test_paged_oracle_out_of_pool_entry_is_a_zero_row():
    case = gen.make_case(3, 10, tree="chain", seed=73, num_heads=2, dl=8, dr=2)
    pg = gen.make_paged(case, seed=74, extra_rows=5)
    idx = pg.kv_index.clone()
    idx[4] = -1
    idx[7] = pg.pool_latent.shape[0] + 3
    zeroed = gen.make_case(3, 10, tree="chain", seed=73, num_heads=2, dl=8, dr=2)
    zeroed.kv_latent[4] = 0
    zeroed.kv_latent[7] = 0
    zeroed.k_rope[4] = 0
    zeroed.k_rope[7] = 0
    ro, rl = orc.mla_verify(zeroed.q_nope, zeroed.q_rope, zeroed.kv_latent, zeroed.k_rope, zeroed.tree_parent,
                            10, zeroed.scale)
    po, pl = orc.mla_verify_paged(case.q_nope, case.q_rope, pg.pool_latent, pg.pool_rope, idx, case.tree_parent,
                                  case.scale, prefix_len=10)
    assert np.array_equal(po, ro) and np.array_equal(pl, rl)
    # a zero key still counts (score 0): the lse differs from dropping the row
    dropped = orc.mla_verify(case.q_nope, case.q_rope, np.delete(orc.to_f64(case.kv_latent), [4, 7], 0),
                             np.delete(orc.to_f64(case.k_rope), [4, 7], 0), case.tree_parent, 8, case.scale)
    assert not np.allclose(dropped[1], pl)
