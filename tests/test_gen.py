"""The seeded input generator: determinism and the structure of its trees."""
import math

import torch

from mla_tree_verify_amd import gen


def _depths(parent):
    d = []
    for p in parent:
        d.append(1 if p < 0 else d[p] + 1)
    return d


def test_same_seed_same_bytes():
    a = gen.make_case(9, 300, seed=7)
    b = gen.make_case(9, 300, seed=7)
    for x, y in [(a.q_nope, b.q_nope), (a.q_rope, b.q_rope), (a.kv_latent, b.kv_latent),
                 (a.k_rope, b.k_rope), (a.tree_parent, b.tree_parent)]:
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
    c = gen.make_case(9, 300, seed=8)
    assert not torch.equal(a.kv_latent.view(torch.int16), c.kv_latent.view(torch.int16))


def test_shapes_and_dtypes():
    c = gen.make_case(33, 100, tree="bounded", seed=1)
    assert c.q_nope.shape == (33, 64, 512) and c.q_nope.dtype == torch.bfloat16
    assert c.q_rope.shape == (33, 64, 64)
    assert c.kv_latent.shape == (133, 512) and c.k_rope.shape == (133, 64)
    assert c.tree_parent.dtype == torch.int32 and c.tree_parent.shape == (33,)
    assert abs(c.scale - 1 / math.sqrt(192)) < 1e-7


def test_random_tree_parents_precede():
    g = torch.Generator().manual_seed(0)
    for q in (1, 2, 9, 33, 64):
        p = gen.random_tree(q, g)
        assert all(-1 <= x < i for i, x in enumerate(p))


def test_bounded_tree_limits():
    g = torch.Generator().manual_seed(1)
    for _ in range(50):
        p = gen.bounded_tree(33, g)
        assert all(-1 <= x < i for i, x in enumerate(p))
        assert max(_depths(p)) <= 8
        counts = {}
        for x in p:
            counts[x] = counts.get(x, 0) + 1
        assert max(counts.values()) <= 4


def test_chain_and_star():
    assert gen.chain_tree(4) == [-1, 0, 1, 2]
    assert gen.star_tree(3) == [-1, -1, -1]


def test_peaky_rows():
    c = gen.make_case(33, 1000, tree="bounded", seed=3, peaky_frac=0.01)
    rows = c.meta["peaky_rows"]
    assert len(rows) == round(0.01 * 1033) == len(set(rows.tolist()))
    ref = gen.make_case(33, 1000, tree="bounded", seed=3)  # same draws before the peaky step
    assert torch.equal(c.kv_latent[rows].float(), ref.kv_latent[rows].float() * 8)
    assert torch.equal(c.k_rope[rows].float(), ref.k_rope[rows].float() * 8)


def test_batched_offsets():
    c = gen.make_workload("b8_ragged_q33")
    offs = c.kv_offsets.tolist()
    assert len(offs) == 9 and offs[0] == 0
    for b in range(8):
        n = offs[b + 1] - offs[b]
        assert n == c.prefix_lens[b] + 33
        assert 1024 <= c.prefix_lens[b] <= 32768
    assert c.kv_latent.shape[0] == offs[-1]
    assert c.q_nope.shape == (8, 33, 64, 512) and c.tree_parent.shape == (8, 33)


def test_named_workloads_shapes():
    for name, spec in gen.WORKLOADS.items():
        if spec["kind"] != "single" or spec["prefix_len"] > 5000:
            continue
        c = gen.make_workload(name)
        assert c.kv_latent.shape[0] == spec["prefix_len"] + spec["q_len"]
