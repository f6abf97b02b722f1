"""fp64 CPU oracle for absorbed-MLA tree-verify attention.

TEST INFRASTRUCTURE ONLY. This module is the plain definition of what the
verify step computes, written for a reader to check by eye. Only the tests,
the smoke check and the CPU-baseline leg of the benchmark may import it; the
library path never does, and it shares no code with the HIP kernels.

What it computes (one sequence, q draft-tree tokens, H heads):

* Key j is a 576-d row: the 512-d compressed latent kv_c[j] followed by the
  64-d decoupled rope key k_pe[j]; the value of key j is the latent kv_c[j]
  alone. The query of (token i, head h) is the absorbed 512-d q_nope plus the
  64-d q_pe. (Page "The Flash Attention Kernel That Had to Be Built",
  section "What Input Knowledge Is Required", the MLA paragraph; page "The
  Moment of Truth", section "Input Knowledge Required", the nope/rope split
  with Dl=512 and Dr=64.)
* Score s_ij = scale * (q_nope[i,h] . kv_c[j] + q_pe[i,h] . k_pe[j]).
* Tree mask: token i sees every cached prefix key and, among the draft
  tokens, itself and its ancestors; every other score is -inf before the
  softmax. (Page "The Flash Attention Kernel That Had to Be Built", section
  "Strategic Context" -- scores against every cached key, then the tree
  mask -- and the DFlash paragraph of "What Input Knowledge Is Required" --
  masked positions set to -inf. Self-visibility is this module's reading of
  a point the pages leave open.)
* out[i,h] = softmax(s_i) @ kv_c, lse[i,h] = ln(sum_j exp(s_ij)) over the
  visible keys (natural log of the scaled scores).
* Flash-style online softmax and the KV-split combine are exact
  reformulations of the same result (page "The Decisive Microbench", section
  "The KV-Split Solution"), so the oracle is the direct definition and
  ``lse_merge`` is the combine formula written out.

Everything runs in float64 on the exactly-widened bf16 input values; the
fp32 ``scale`` argument is widened exactly as well.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def to_f64(x) -> np.ndarray:
    """Widen a numpy array or a CPU torch tensor (bf16/fp32/...) to float64."""
    if hasattr(x, "detach"):  # torch tensor: bf16 has no numpy dtype
        x = x.detach().cpu()
        if x.is_floating_point():
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def fp32_scale(scale: float) -> float:
    """The kernel receives an fp32 scale; the oracle uses that exact value."""
    return float(np.float32(scale))


# --------------------------------------------------------------------------
# the draft tree
# --------------------------------------------------------------------------
def check_tree(parent: Sequence[int]) -> None:
    """parent[i] must be -1 (child of the prefix root) or an earlier node."""
    for i, p in enumerate(parent):
        if not (p == -1 or 0 <= p < i):
            raise ValueError(f"parent[{i}] = {p} is not in {{-1}} U [0, {i})")


def ancestors_inclusive(parent: Sequence[int]) -> List[List[int]]:
    """anc*(i) = {i, parent(i), parent(parent(i)), ...}, stopping at -1."""
    parent = [int(p) for p in parent]
    check_tree(parent)
    out = []
    for i in range(len(parent)):
        chain = []
        node = i
        while node != -1:
            chain.append(node)
            node = parent[node]
        out.append(sorted(chain))
    return out


# --------------------------------------------------------------------------
# attention over an explicit key set
# --------------------------------------------------------------------------
def attend_rows(q_nope: np.ndarray, q_rope: np.ndarray, lat: np.ndarray, rope: np.ndarray,
                scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of H query rows over K explicit keys.

    q_nope [H, Dl], q_rope [H, Dr], lat [K, Dl] (keys' latent = values),
    rope [K, Dr]. Returns out [H, Dl] and lse [H]. With K = 0 the result is
    out = 0 and lse = -inf (an empty key set)."""
    sc = fp32_scale(scale)
    h = q_nope.shape[0]
    if lat.shape[0] == 0:
        return np.zeros((h, lat.shape[1])), np.full(h, -np.inf)
    s = sc * (q_nope @ lat.T + q_rope @ rope.T)  # [H, K]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ lat) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def mla_verify(q_nope, q_rope, kv_latent, k_rope, tree_parent, prefix_len: int,
               scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One sequence.

    q_nope [q, H, Dl], q_rope [q, H, Dr], kv_latent [P+q, Dl], k_rope [P+q, Dr],
    tree_parent [q]. Returns out [q, H, Dl] and lse [q, H] in float64."""
    qn, qr = to_f64(q_nope), to_f64(q_rope)
    lat, rope = to_f64(kv_latent), to_f64(k_rope)
    parent = [int(p) for p in np.asarray(to_f64(tree_parent)).reshape(-1)]
    q, h, dl = qn.shape
    assert lat.shape[0] == prefix_len + q, "kv rows must be the prefix followed by the q tree tokens"
    out = np.empty((q, h, dl))
    lse = np.empty((q, h))
    for i, anc in enumerate(ancestors_inclusive(parent)):
        tree_rows = prefix_len + np.asarray(anc, dtype=np.int64)
        # prefix rows are a contiguous slice (a view); the tree rows a small gather
        keys_lat = np.concatenate([lat[:prefix_len], lat[tree_rows]])
        keys_rope = np.concatenate([rope[:prefix_len], rope[tree_rows]])
        out[i], lse[i] = attend_rows(qn[i], qr[i], keys_lat, keys_rope, scale)
    return out, lse


def mla_verify_batched(q_nope, q_rope, kv_latent, k_rope, tree_parent, kv_offsets,
                       scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """B independent sequences; sequence b owns KV rows [off[b], off[b+1]),
    its prefix followed by its q tree tokens, so P_b = off[b+1] - off[b] - q.
    q_nope [B, q, H, Dl], tree_parent [B, q]. Returns out [B, q, H, Dl], lse [B, q, H]."""
    qn, qr = to_f64(q_nope), to_f64(q_rope)
    lat, rope = to_f64(kv_latent), to_f64(k_rope)
    offs = [int(v) for v in np.asarray(to_f64(kv_offsets)).reshape(-1)]
    par = np.asarray(to_f64(tree_parent)).astype(np.int64)
    b, q = par.shape
    outs, lses = [], []
    for s in range(b):
        lo, hi = offs[s], offs[s + 1]
        o, l = mla_verify(qn[s], qr[s], lat[lo:hi], rope[lo:hi], par[s], hi - lo - q, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def gather_pages(pool_latent, pool_rope, kv_index) -> Tuple[np.ndarray, np.ndarray]:
    """Paged KV with one token per page: logical KV row r is row kv_index[r]
    of the pool (page "The Moment of Truth", section "Output Knowledge
    Created": the serving cache uses page_size=1, so attention gathers scattered
    rows). An entry outside [0, pool_rows) is read as a row of zeros (this
    library's reading; the pages do not say). Returns the logical rows in
    order, float64."""
    lat, rope = to_f64(pool_latent), to_f64(pool_rope)
    idx = np.asarray(to_f64(kv_index)).astype(np.int64).reshape(-1)
    ok = (idx >= 0) & (idx < lat.shape[0])
    safe = np.where(ok, idx, 0)
    g_lat = np.where(ok[:, None], lat[safe], 0.0)
    g_rope = np.where(ok[:, None], rope[safe], 0.0)
    return g_lat, g_rope


def mla_verify_paged(q_nope, q_rope, pool_latent, pool_rope, kv_index, tree_parent, scale: float,
                     prefix_len: int = None, kv_offsets=None) -> Tuple[np.ndarray, np.ndarray]:
    """The verify step over a paged KV pool: gather the logical rows through
    the page table, then the plain definition. One sequence (prefix_len) or a
    batch (kv_offsets into the logical rows, as mla_verify_batched)."""
    lat, rope = gather_pages(pool_latent, pool_rope, kv_index)
    if kv_offsets is None:
        return mla_verify(q_nope, q_rope, lat, rope, tree_parent, prefix_len, scale)
    return mla_verify_batched(q_nope, q_rope, lat, rope, tree_parent, kv_offsets, scale)


# --------------------------------------------------------------------------
# the combine formula for KV-split partials
# --------------------------------------------------------------------------
def lse_merge(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Merge partial results computed over disjoint key subsets.

    Each part s gives a normalised o_s [..., D] and lse_s [...]. With
    M = max_s lse_s and w_s = exp(lse_s - M): out = sum_s w_s o_s / sum_s w_s
    and lse = M + ln(sum_s w_s). Rows where every part is empty (M = -inf)
    give out = 0 and lse = -inf."""
    o = np.stack([to_f64(x) for x in outs])  # [S, ..., D]
    l = np.stack([to_f64(x) for x in lses])  # [S, ...]
    m = l.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(l), np.exp(l - m_safe), 0.0)
    wsum = w.sum(axis=0)
    out = np.where(finite[..., None], (w[..., None] * o).sum(axis=0) / np.where(finite, wsum, 1.0)[..., None], 0.0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, wsum, 1.0)), -np.inf)
    return out, lse


# --------------------------------------------------------------------------
# work accounting for the benchmark (what the method must compute or move)
# --------------------------------------------------------------------------
def visible_key_count(tree_parent, prefix_len: int) -> int:
    """sum_i |V(i)| = q * P + sum_i |anc*(i)|."""
    parent = [int(p) for p in np.asarray(to_f64(tree_parent)).reshape(-1)]
    return sum(prefix_len + len(a) for a in ancestors_inclusive(parent))


def algorithmic_flops(tree_parent, prefix_len: int, num_heads: int = 64, dl: int = 512, dr: int = 64) -> int:
    """2 * H * (Dl + Dr) multiply-adds for the score and 2 * H * Dl for the
    value product, per visible (token, key) pair."""
    return 2 * num_heads * (2 * dl + dr) * visible_key_count(tree_parent, prefix_len)


def algorithmic_bytes(q_len: int, kv_len: int, num_heads: int = 64, dl: int = 512, dr: int = 64) -> int:
    """Each input read once, each output written once: bf16 KV rows and
    queries, int32 parents, fp32 out and lse."""
    kv = kv_len * (dl + dr) * 2
    q = q_len * num_heads * (dl + dr) * 2
    out = q_len * num_heads * dl * 4
    lse = q_len * num_heads * 4
    return kv + q + out + lse + 4 * q_len
