"""fp64 CPU oracle of the selection variants of MC-Sparse's oracle analysis.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import or run this module.  It shares no code with the HIP
library and imports nothing from it.

Sources (the same pages as mcs_oracle):
  [onedev] "how it works": at one attention density, KV sets are chosen with
           exact dense attention probabilities by a block oracle (KV blocks per
           query block), a token oracle (one set of individual KV tokens shared
           by a query block) and a per-query oracle (each query its own
           tokens), and compared with vanilla block-sparse attention (BSA),
           which ranks blocks by mean-pooled query and key representations.
  [onedev] "what is different" / system and ablation paragraph: the ablation
           ladder starts from vanilla BSA and adds, in turn, exact KV selection
           with cross-step reuse, token-level KV granularity, query grouping and
           residual compensation.
  [n884]   "Development": the three sources of loss (grouping constraint,
           inaccurate selection, discarded contributions).

Readings (R-numbers continue the design notes' register):
  R27  KV blocks tile the valid keys [0, n_valid) in token order, B keys each;
       the last block may be shorter.  Query blocks of the block variants are
       the groups of the partition they are given (contiguous token blocks
       for BSA and the oracles, i.e. the identity partition).
  R28  Equal density: a block variant keeps n_b = max(1, round(k / B)) blocks
       (at most the number of blocks), k = ceil(density * N) being the token
       budget of the token variants.
  R29  Block oracle score of (group g, block b): the sum over the block's keys
       of the group score of mcs_oracle.group_scores, i.e. the exact
       probability mass the group's valid queries put on the block.
  R30  Vanilla BSA score of (group g, block b): scale * qbar_g . kbar_b, with
       qbar_g the mean of the group's valid member queries and kbar_b the mean
       of the block's keys (the softmax over blocks is monotone, so ranking
       the logits ranks the pooled probabilities).
  R31  Block ranking: higher score first, ties to the lower block index
       (the token rule R4 applied to blocks); the selected blocks expand to
       their tokens in ascending order.
  R32  Per-query oracle: each valid query keeps its own k keys with the
       largest exact probability (equivalently logit), ties to the lower key
       index, and attends only to them.

Parity status: every function here is pinned by tests/test_oracle_variants.py
(reductions to the token and per-query cases, closed forms, invariants and
brute force).
"""
from __future__ import annotations

import numpy as np

from .mcs_oracle import group_scores, topk_select

__all__ = [
    "identity_perm", "kv_blocks", "block_budget", "block_oracle_scores", "meanpool_scores",
    "select_blocks", "expand_blocks", "per_query_attention", "retained_mass",
    "group_sets_per_query",
]


def identity_perm(n_pad):
    """The partition whose groups are contiguous token blocks (R27)."""
    return np.arange(n_pad, dtype=np.int64)


def kv_blocks(n_valid, B):
    """(start, end) of every KV block: B consecutive valid keys, the last one
    possibly shorter (R27)."""
    return [(s, min(s + B, n_valid)) for s in range(0, n_valid, B)]


def block_budget(topk, B, n_blocks):
    """Blocks kept at the density of a `topk`-token budget (R28)."""
    return int(min(n_blocks, max(1, (topk + B // 2) // B)))


def block_oracle_scores(a, n_valid, B):
    """Exact block scores from group scores `a` [G, n_valid] (R29)."""
    a = np.asarray(a, np.float64)
    return np.stack([a[:, s:e].sum(axis=1) for s, e in kv_blocks(n_valid, B)], axis=1)


def meanpool_scores(q, k, perm, n_valid, C, B, scale):
    """Vanilla BSA block scores [G, n_blocks] from mean-pooled queries and keys
    (R30).  A group without valid members scores 0 everywhere."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    G = q.shape[0] // C
    kbar = np.stack([k[s:e].mean(axis=0) for s, e in kv_blocks(n_valid, B)])
    out = np.zeros((G, kbar.shape[0]))
    for g in range(G):
        mem = np.asarray(perm[g * C:(g + 1) * C])
        mem = mem[mem < n_valid]
        if mem.size:
            out[g] = scale * (kbar @ q[mem].mean(axis=0))
    return out


def select_blocks(scores, n_b):
    """The n_b best blocks of every group, ascending (R31)."""
    return topk_select(scores, n_b)


def expand_blocks(block_idx, n_valid, B):
    """Token indices (ascending) of each group's selected blocks (R27, R31)."""
    blocks = kv_blocks(n_valid, B)
    out = []
    for row in np.asarray(block_idx):
        out.append(np.concatenate([np.arange(*blocks[b]) for b in sorted(int(x) for x in row)]))
    return out


def per_query_attention(q, k, v, n_valid, topk, scale):
    """Attention where every valid query keeps its own top-k keys by exact
    probability (R32); rows of padded queries are 0."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)[:n_valid]
    v = np.asarray(v, np.float64)[:n_valid]
    o = np.zeros((q.shape[0], v.shape[1]))
    j = np.arange(n_valid)
    for i in range(n_valid):
        s = scale * (k @ q[i])
        sel = np.sort(np.lexsort((j, -s))[:topk])
        t = s[sel] - s[sel].max()
        p = np.exp(t)
        o[i] = (p / p.sum()) @ v[sel]
    return o


def retained_mass(q, k, n_valid, scale, lse, sets_per_query):
    """Exact dense probability mass each valid query keeps on its KV set
    (1 - the discarded tail of [onedev] "how it works").  `sets_per_query[i]`
    is the set of query i (None: no set, mass NaN)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    lse = np.asarray(lse, np.float64)
    out = np.zeros(n_valid)
    for i in range(n_valid):
        if sets_per_query[i] is None:
            out[i] = np.nan
            continue
        sel = np.asarray(sets_per_query[i])
        out[i] = np.exp(scale * (k[sel] @ q[i]) - lse[i]).sum()
    return out


def group_sets_per_query(perm, kv_sets, n_valid, C):
    """Expand one KV set per group to the set of every valid member query."""
    sets = [None] * n_valid
    for g, sel in enumerate(kv_sets):
        for i in np.asarray(perm[g * C:(g + 1) * C]):
            if i < n_valid:
                sets[int(i)] = np.asarray(sel)
    return sets

