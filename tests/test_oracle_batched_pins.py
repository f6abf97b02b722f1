"""Pins for the batched and paged-batched oracle and for the work counters.

The batched layout follows the ragged-prefix workload: sequence b owns KV rows
[off[b], off[b+1]) of one array, its prefix followed by its q tree tokens, so
its prefix length is off[b+1] - off[b] - q, and each sequence has its own tree
(this library's reading of the batched configuration; the pages benchmark
one stream only, page "The Decisive Microbench", section "The Message").

  * a pure-Python brute force over the concatenated arrays, with the offsets
    and every ancestor walk written out by hand, on a 3-sequence ragged toy
    batch with distinct trees (one sequence with an empty prefix);
  * a planted-mistake check: pairing sequence b's tree with sequence b+1's
    rows (or its queries) must fail the brute-force pin;
  * the paged batched branch: the same brute force over rows scattered
    through a page table;
  * the work counters: visible keys by explicit enumeration, and the byte
    count from the sizes of the tensors the call actually reads and writes.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle.mla_verify_oracle as orc
from mla_tree_verify_amd import gen

TOL = 1e-12


def _walk(parent, i):
    """Tree nodes visible to token i: i itself and every ancestor, by walking parents."""
    seen = []
    node = i
    while node != -1:
        seen.append(node)
        node = parent[node]
    return seen


def brute_force_batched(qn, qr, lat, rope, parents, offs, scale):
    """Pure-Python loops over plain nested lists. qn [B][q][H][Dl], lat [N][Dl],
    parents [B][q], offs [B+1] -> out [B][q][H][Dl], lse [B][q][H]."""
    sc = float(np.float32(scale))
    out, lse = [], []
    for b in range(len(parents)):
        q = len(parents[b])
        base = offs[b]
        prefix = offs[b + 1] - offs[b] - q
        ob, lb = [], []
        for i in range(q):
            rows = [base + j for j in range(prefix)] + [base + prefix + t for t in _walk(parents[b], i)]
            oi, li = [], []
            for h in range(len(qn[b][i])):
                s = []
                for r in rows:
                    terms = [qn[b][i][h][d] * lat[r][d] for d in range(len(lat[r]))]
                    terms += [qr[b][i][h][d] * rope[r][d] for d in range(len(rope[r]))]
                    s.append(sc * math.fsum(terms))
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                oi.append([math.fsum(e[k] * lat[rows[k]][d] for k in range(len(rows))) / tot
                           for d in range(len(lat[0]))])
                li.append(m + math.log(tot))
            ob.append(oi)
            lb.append(li)
        out.append(ob)
        lse.append(lb)
    return np.array(out), np.array(lse)


def toy_batch(seed: int = 41):
    """3 sequences, q = 4, prefixes 0, 3 and 6, a distinct tree each."""
    return gen.make_batched_case(3, 4, tree="random", num_heads=3, seed=seed, dl=8, dr=3, prefix_lens=[0, 3, 6])


def _as_lists(case):
    return (case.q_nope.double().tolist(), case.q_rope.double().tolist(), case.kv_latent.double().tolist(),
            case.k_rope.double().tolist(), case.tree_parent.tolist(), case.kv_offsets.tolist())


def batched_pin_error(case) -> float:
    qn, qr, lat, rope, parents, offs = _as_lists(case)
    bo, bl = brute_force_batched(qn, qr, lat, rope, parents, offs, case.scale)
    oo, ol = orc.mla_verify_batched(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                                    case.kv_offsets, case.scale)
    return max(np.abs(oo - bo).max(), np.abs(ol - bl).max())


def test_toy_batch_is_ragged_with_distinct_trees():
    case = toy_batch()
    offs = case.kv_offsets.tolist()
    assert [offs[b + 1] - offs[b] - 4 for b in range(3)] == [0, 3, 6]
    trees = [tuple(t) for t in case.tree_parent.tolist()]
    assert len(set(trees)) == 3


@pytest.mark.parametrize("seed", [41, 42, 43])
def test_batched_oracle_equals_brute_force(seed):
    assert batched_pin_error(toy_batch(seed)) < TOL


def test_batched_oracle_empty_prefix_sequence_is_self_attention_of_its_tree():
    """Sequence 0 has no prefix: a root token (parent -1) sees only its own row."""
    case = toy_batch()
    oo, ol = orc.mla_verify_batched(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                                    case.kv_offsets, case.scale)
    par = case.tree_parent[0].tolist()
    lat = case.kv_latent.double().numpy()
    rope = case.k_rope.double().numpy()
    sc = float(np.float32(case.scale))
    roots = [i for i, p in enumerate(par) if p == -1]
    assert roots
    for i in roots:
        assert np.abs(oo[0, i] - lat[i][None, :]).max() < TOL
        s = sc * (case.q_nope[0, i].double().numpy() @ lat[i] + case.q_rope[0, i].double().numpy() @ rope[i])
        assert np.abs(ol[0, i] - s).max() < TOL


# planted mistakes in a copy of the batched loop: each must fail the pin
def _batched_variant(tree_shift=0, query_shift=0, row_shift=0):
    def fn(q_nope, q_rope, kv_latent, k_rope, tree_parent, kv_offsets, scale):
        qn, qr = orc.to_f64(q_nope), orc.to_f64(q_rope)
        lat, rope = orc.to_f64(kv_latent), orc.to_f64(k_rope)
        offs = [int(v) for v in np.asarray(orc.to_f64(kv_offsets)).reshape(-1)]
        par = np.asarray(orc.to_f64(tree_parent)).astype(np.int64)
        b, q = par.shape
        outs, lses = [], []
        for s in range(b):
            lo, hi = offs[(s + row_shift) % b], offs[(s + row_shift) % b + 1]
            o, l = orc.mla_verify(qn[(s + query_shift) % b], qr[(s + query_shift) % b], lat[lo:hi], rope[lo:hi],
                                  par[(s + tree_shift) % b], hi - lo - q, scale)
            outs.append(o)
            lses.append(l)
        return np.stack(outs), np.stack(lses)
    return fn


@pytest.mark.parametrize("mistake", ["tree_of_next_sequence", "queries_of_next_sequence", "rows_of_next_sequence"])
def test_batched_pin_catches_planted_mistakes(mistake, monkeypatch):
    kw = {"tree_of_next_sequence": dict(tree_shift=1), "queries_of_next_sequence": dict(query_shift=1),
          "rows_of_next_sequence": dict(row_shift=1)}[mistake]
    monkeypatch.setattr(orc, "mla_verify_batched", _batched_variant(**kw))
    try:
        err = batched_pin_error(toy_batch())
        caught = not np.isfinite(err) or err > 1e-6
    except Exception:
        caught = True  # a shape error is also a detection
    assert caught


def test_batched_variant_without_mistake_passes():
    """The copy used for planting is faithful when nothing is planted."""
    case = toy_batch()
    a = _batched_variant()(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                           case.kv_offsets, case.scale)
    b = orc.mla_verify_batched(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                               case.kv_offsets, case.scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# paged batched branch
def test_paged_batched_oracle_equals_brute_force():
    case = toy_batch(44)
    pg = gen.make_paged(case, seed=45, extra_rows=11)
    po, pl = orc.mla_verify_paged(case.q_nope, case.q_rope, pg.pool_latent, pg.pool_rope, pg.kv_index,
                                  case.tree_parent, case.scale, kv_offsets=case.kv_offsets)
    # brute force over the logical rows read one by one through the page table
    pool_lat = pg.pool_latent.double().tolist()
    pool_rope = pg.pool_rope.double().tolist()
    idx = pg.kv_index.tolist()
    lat = [pool_lat[r] for r in idx]
    rope = [pool_rope[r] for r in idx]
    qn, qr, _, _, parents, offs = _as_lists(case)
    bo, bl = brute_force_batched(qn, qr, lat, rope, parents, offs, case.scale)
    assert max(np.abs(po - bo).max(), np.abs(pl - bl).max()) < TOL


def test_paged_batched_oracle_out_of_pool_entries():
    """Out-of-pool entries read as zero rows in the batched branch too."""
    case = toy_batch(46)
    pg = gen.make_paged(case, seed=47, extra_rows=3)
    idx = pg.kv_index.clone()
    bad = [1, 9]  # logical rows of sequences 1 and 2 (sequence 0 owns rows 0..3)
    idx[bad[0]] = -5
    idx[bad[1]] = int(pg.pool_latent.shape[0])
    po, pl = orc.mla_verify_paged(case.q_nope, case.q_rope, pg.pool_latent, pg.pool_rope, idx,
                                  case.tree_parent, case.scale, kv_offsets=case.kv_offsets)
    lat = case.kv_latent.clone()
    rope = case.k_rope.clone()
    lat[bad] = 0
    rope[bad] = 0
    qn, qr, _, _, parents, offs = _as_lists(case)
    bo, bl = brute_force_batched(qn, qr, lat.double().tolist(), rope.double().tolist(), parents, offs, case.scale)
    assert max(np.abs(po - bo).max(), np.abs(pl - bl).max()) < TOL


# --------------------------------------------------------------------------
# the work counters
# --------------------------------------------------------------------------
@pytest.mark.parametrize("tree,q,p,seed", [("random", 9, 100, 1), ("chain", 9, 0, 2), ("star", 5, 7, 3),
                                            ("bounded", 33, 50, 4)])
def test_visible_key_count_by_enumeration(tree, q, p, seed):
    parent = gen.make_tree(tree, q, torch.Generator().manual_seed(seed))
    count = 0
    for i in range(q):
        for j in range(p + q):
            # key j is visible to token i: a prefix key, or a tree node on i's path to the root
            count += 1 if j < p or (j - p) in _walk(parent, i) else 0
    assert orc.visible_key_count(parent, p) == count
    assert orc.algorithmic_flops(parent, p, num_heads=3, dl=5, dr=2) == 2 * 3 * (2 * 5 + 2) * count


@pytest.mark.parametrize("name", ["q9_p256", "q33_p16384_peaky"])
def test_algorithmic_bytes_equals_tensor_sizes(name):
    """Each input read once and each output written once: the sum of the sizes
    of the tensors a call takes, plus the fp32 out [q,H,512] and lse [q,H]."""
    case = gen.make_workload(name)
    q, h = case.q_len, case.num_heads
    reads = sum(t.numel() * t.element_size()
                for t in (case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent))
    out = torch.empty(q, h, 512, dtype=torch.float32)
    lse = torch.empty(q, h, dtype=torch.float32)
    writes = out.numel() * out.element_size() + lse.numel() * lse.element_size()
    n = int(case.kv_latent.shape[0])
    assert orc.algorithmic_bytes(q, n, num_heads=h) == reads + writes


def test_algorithmic_bytes_other_head_count():
    case = gen.make_case(9, 40, num_heads=8, seed=5)
    reads = sum(t.numel() * t.element_size()
                for t in (case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent))
    writes = 9 * 8 * 512 * 4 + 9 * 8 * 4
    assert orc.algorithmic_bytes(9, 49, num_heads=8) == reads + writes
