"""Seeded synthetic inputs for MLA tree-verify attention.

This module draws inputs only: random draft trees, ragged prefix lengths and
bf16 tensors. It holds none of the attention arithmetic, so both the fp64
oracle and the HIP path consume exactly the same bytes from it.

Shapes follow the absorbed MLA layout the pages describe (page "The Moment of
Truth: Benchmarking a Custom sm_120 Flash Attention Kernel", benchmark table
header: H=64, Dl=512, Dr=64; page "The Flash Attention Kernel That Had to Be
Built", section "What Input Knowledge Is Required": a 512-d latent kv_c plus a
64-d decoupled rope key per cached token, and an absorbed query split into a
512-d nope part and a 64-d rope part).

Recipe (all draws from one CPU ``torch.Generator``, in this fixed order):
  1. the draft tree(s)                 -- int32 parent array, parent[i] in {-1} U [0, i)
  2. ragged prefix lengths (batched)   -- log-uniform integers
  3. q_nope [q, H, Dl], 4. q_rope [q, H, Dr], 5. kv_latent [N, Dl], 6. k_rope [N, Dr]
     -- float32 N(0, 1) rounded to bfloat16 with round-to-nearest-even
  7. peaky key rows (optional)         -- rows chosen without replacement; the
     whole 576-d key row (latent and rope) is multiplied by 8 (exact in bf16)
KV rows are laid out prefix first, then the q tree tokens in node order
(tree node t lives at row P + t).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

H_DEFAULT = 64
DL = 512
DR = 64
SCALE_DEFAULT = float(torch.tensor(1.0 / math.sqrt(192.0), dtype=torch.float32).item())


# --------------------------------------------------------------------------
# draft trees
# --------------------------------------------------------------------------
def random_tree(q: int, g: torch.Generator) -> List[int]:
    """parent[i] uniform over {-1, 0, ..., i-1}."""
    parents = []
    for i in range(q):
        parents.append(int(torch.randint(-1, i, (1,), generator=g).item()))
    return parents


def bounded_tree(q: int, g: torch.Generator, max_depth: int = 8, max_children: int = 4) -> List[int]:
    """Random tree with depth <= max_depth and at most max_children per node.

    Node i picks its parent uniformly among the candidates that still have room:
    the prefix root (-1, itself capped at max_children children) and every
    earlier node j whose depth is below max_depth and that has fewer than
    max_children children. Depth counts edges from the prefix root, so a child
    of the root has depth 1.
    """
    parents: List[int] = []
    depth: List[int] = []
    children: Dict[int, int] = {-1: 0}
    for i in range(q):
        cands = [-1] if children[-1] < max_children else []
        cands += [j for j in range(i) if depth[j] < max_depth and children.get(j, 0) < max_children]
        if not cands:
            raise ValueError("tree budget exhausted")
        p = cands[int(torch.randint(0, len(cands), (1,), generator=g).item())]
        parents.append(p)
        depth.append(1 if p < 0 else depth[p] + 1)
        children[p] = children.get(p, 0) + 1
        children[i] = 0
    return parents


def chain_tree(q: int) -> List[int]:
    """Each draft token's parent is the previous one."""
    return [i - 1 for i in range(q)]


def star_tree(q: int) -> List[int]:
    """Every draft token hangs directly off the prefix root."""
    return [-1] * q


def make_tree(kind: str, q: int, g: torch.Generator) -> List[int]:
    if kind == "random":
        return random_tree(q, g)
    if kind == "bounded":
        return bounded_tree(q, g)
    if kind == "chain":
        return chain_tree(q)
    if kind == "star":
        return star_tree(q)
    raise ValueError(f"unknown tree kind {kind!r}")


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------
def _bf16_normal(shape, g: torch.Generator) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


@dataclass
class Case:
    """One verify call (or one batch of calls); all tensors live on the CPU."""

    q_nope: torch.Tensor  # bf16 [q, H, Dl]  (batched: [B, q, H, Dl])
    q_rope: torch.Tensor  # bf16 [q, H, Dr]  (batched: [B, q, H, Dr])
    kv_latent: torch.Tensor  # bf16 [N, Dl]  (batched: [sum N_b, Dl])
    k_rope: torch.Tensor  # bf16 [N, Dr]
    tree_parent: torch.Tensor  # int32 [q]  (batched: [B, q])
    prefix_len: int  # batched: max over sequences (informational)
    scale: float
    kv_offsets: Optional[torch.Tensor] = None  # int64 [B+1] for batched cases
    prefix_lens: Optional[List[int]] = None  # per sequence (batched)
    meta: dict = field(default_factory=dict)

    @property
    def batched(self) -> bool:
        return self.kv_offsets is not None

    @property
    def q_len(self) -> int:
        return int(self.tree_parent.shape[-1])

    @property
    def num_heads(self) -> int:
        return int(self.q_nope.shape[-2])


def make_case(
    q_len: int,
    prefix_len: int,
    tree: str = "random",
    num_heads: int = H_DEFAULT,
    seed: int = 0,
    peaky_frac: float = 0.0,
    peaky_mult: float = 8.0,
    dl: int = DL,
    dr: int = DR,
    scale: float = SCALE_DEFAULT,
    parents: Optional[List[int]] = None,
) -> Case:
    """One sequence: q_len tree tokens over a prefix of prefix_len cached tokens."""
    g = torch.Generator().manual_seed(seed)
    if parents is None:
        parents = make_tree(tree, q_len, g)
    assert len(parents) == q_len
    n = prefix_len + q_len
    q_nope = _bf16_normal((q_len, num_heads, dl), g)
    q_rope = _bf16_normal((q_len, num_heads, dr), g)
    kv_latent = _bf16_normal((n, dl), g)
    k_rope = _bf16_normal((n, dr), g)
    peaky_rows = None
    if peaky_frac > 0.0:
        k = int(round(peaky_frac * n))
        peaky_rows = torch.randperm(n, generator=g)[:k]
        kv_latent[peaky_rows] = (kv_latent[peaky_rows].float() * peaky_mult).to(torch.bfloat16)
        k_rope[peaky_rows] = (k_rope[peaky_rows].float() * peaky_mult).to(torch.bfloat16)
    return Case(
        q_nope=q_nope,
        q_rope=q_rope,
        kv_latent=kv_latent,
        k_rope=k_rope,
        tree_parent=torch.tensor(parents, dtype=torch.int32),
        prefix_len=prefix_len,
        scale=scale,
        meta={"tree": tree, "seed": seed, "peaky_rows": peaky_rows},
    )


def make_batched_case(
    batch: int,
    q_len: int,
    prefix_lo: int = 1024,
    prefix_hi: int = 32768,
    tree: str = "bounded",
    num_heads: int = H_DEFAULT,
    seed: int = 0,
    dl: int = DL,
    dr: int = DR,
    scale: float = SCALE_DEFAULT,
    prefix_lens: Optional[List[int]] = None,
) -> Case:
    """batch sequences, each with its own tree and a log-uniform prefix length.

    KV rows are stored contiguously per sequence: sequence b owns rows
    [off[b], off[b+1]) = its prefix followed by its q_len tree tokens.
    """
    g = torch.Generator().manual_seed(seed)
    trees = [make_tree(tree, q_len, g) for _ in range(batch)]
    if prefix_lens is None:
        lo, hi = math.log(prefix_lo), math.log(prefix_hi)
        u = torch.rand(batch, generator=g, dtype=torch.float64)
        prefix_lens = [int(round(math.exp(lo + (hi - lo) * float(x)))) for x in u]
    assert len(prefix_lens) == batch
    offs = [0]
    for p in prefix_lens:
        offs.append(offs[-1] + p + q_len)
    total = offs[-1]
    q_nope = _bf16_normal((batch, q_len, num_heads, dl), g)
    q_rope = _bf16_normal((batch, q_len, num_heads, dr), g)
    kv_latent = _bf16_normal((total, dl), g)
    k_rope = _bf16_normal((total, dr), g)
    return Case(
        q_nope=q_nope,
        q_rope=q_rope,
        kv_latent=kv_latent,
        k_rope=k_rope,
        tree_parent=torch.tensor(trees, dtype=torch.int32),
        prefix_len=max(prefix_lens),
        scale=scale,
        kv_offsets=torch.tensor(offs, dtype=torch.int64),
        prefix_lens=list(prefix_lens),
        meta={"tree": tree, "seed": seed},
    )


@dataclass
class Paged:
    """The KV rows of a case scattered over a larger pool (one token per page)."""

    pool_latent: torch.Tensor  # bf16 [pool_rows, Dl]
    pool_rope: torch.Tensor  # bf16 [pool_rows, Dr]
    kv_index: torch.Tensor  # int32 [N]: logical row -> pool row


def make_paged(case: Case, seed: int, extra_rows: int = 0, garbage: float = 100.0) -> Paged:
    """Scatter the case's N logical KV rows over a pool of N + extra_rows rows by
    a seeded random permutation; pool rows no logical row maps to hold large
    random values (garbage that must never be read)."""
    g = torch.Generator().manual_seed(seed)
    n = int(case.kv_latent.shape[0])
    pool_rows = n + extra_rows
    perm = torch.randperm(pool_rows, generator=g)[:n]
    dl, dr = int(case.kv_latent.shape[1]), int(case.k_rope.shape[1])
    pool_latent = (torch.randn(pool_rows, dl, generator=g) * garbage).to(torch.bfloat16)
    pool_rope = (torch.randn(pool_rows, dr, generator=g) * garbage).to(torch.bfloat16)
    pool_latent[perm] = case.kv_latent
    pool_rope[perm] = case.k_rope
    return Paged(pool_latent=pool_latent, pool_rope=pool_rope, kv_index=perm.to(torch.int32))


# --------------------------------------------------------------------------
# the named workloads (sizes as the benchmark tables on the pages use them)
# --------------------------------------------------------------------------
WORKLOADS = {
    # q_len 9 random tree over a 256-token prefix
    "q9_p256": dict(kind="single", q_len=9, prefix_len=256, tree="random", seed=1),
    # q_len 9 random tree over a 4096-token prefix
    "q9_p4096": dict(kind="single", q_len=9, prefix_len=4096, tree="random", seed=2),
    # q_len 9 random tree over a 16384-token prefix (headline shape)
    "q9_p16384": dict(kind="single", q_len=9, prefix_len=16384, tree="random", seed=16),
    # q_len 33 bounded tree (depth <= 8, <= 4 children), 1% of keys scaled by 8
    "q33_p16384_peaky": dict(kind="single", q_len=33, prefix_len=16384, tree="bounded", seed=3, peaky_frac=0.01),
    # q_len 9 chain over a 65536-token prefix
    "q9_p65536_chain": dict(kind="single", q_len=9, prefix_len=65536, tree="chain", seed=4),
    # 8 sequences, ragged log-uniform prefixes in [1024, 32768], q_len 33 trees
    "b8_ragged_q33": dict(kind="batched", batch=8, q_len=33, prefix_lo=1024, prefix_hi=32768, tree="bounded", seed=5),
}


def make_workload(name: str) -> Case:
    spec = dict(WORKLOADS[name])
    kind = spec.pop("kind")
    if kind == "single":
        return make_case(**spec)
    return make_batched_case(**spec)


def make_mla_weights(num_heads: int, d_nope: int, d_v: int, dl: int, seed: int):
    """Random per-head up-projections W_UK [H, d_nope, Dl] and W_UV [H, d_v, Dl]
    (float64) for checks of the absorbed form against the unabsorbed one."""
    g = torch.Generator().manual_seed(seed)
    w_uk = torch.randn(num_heads, d_nope, dl, generator=g, dtype=torch.float64) / math.sqrt(dl)
    w_uv = torch.randn(num_heads, d_v, dl, generator=g, dtype=torch.float64) / math.sqrt(dl)
    return w_uk, w_uv
