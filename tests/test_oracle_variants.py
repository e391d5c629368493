"""Pins of the oracle-analysis selection variants (oracle/variants.py).

onedev.kr summary, "how it works": block oracle, token oracle and per-query
oracle (exact probabilities) against mean-pooled vanilla BSA, all at one
density.  Pins: the variants' reductions to one another (unit blocks make the
block oracle the token oracle; single-query groups make the token oracle and
unit-block BSA the per-query oracle; all blocks make any variant dense
attention), a hand-computed mean-pooling case, the probability-mass invariant
of the block scores, brute force over all k-subsets for the per-query oracle,
and the retained-mass ordering the oracles guarantee by construction.
"""
import itertools

import numpy as np

from oracle import mcs_oracle as orc
from oracle import variants as var


def layer(n=256, nv=250, d=16, seed=0, clusters=6):
    rng = np.random.default_rng(seed)
    c = rng.standard_normal((clusters, d))
    lab = rng.integers(0, clusters, n)
    q = c[lab] + 0.3 * rng.standard_normal((n, d))
    k = c[lab] + 0.3 * rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    q[nv:] = k[nv:] = v[nv:] = 0
    return q, k, v, nv, orc.softmax_scale(d)


def test_kv_blocks_and_budget():
    assert var.kv_blocks(10, 4) == [(0, 4), (4, 8), (8, 10)]
    assert var.kv_blocks(8, 4) == [(0, 4), (4, 8)]
    assert var.block_budget(8190, 128, 256) == 64        # round(63.98)
    assert var.block_budget(10, 128, 256) == 1           # at least one block
    assert var.block_budget(1000, 4, 100) == 100         # at most all blocks
    assert var.block_budget(6, 4, 100) == 2              # 1.5 rounds up


def test_expand_blocks_with_short_tail():
    toks = var.expand_blocks([[2, 0], [1, 2]], 10, 4)
    assert toks[0].tolist() == [0, 1, 2, 3, 8, 9]
    assert toks[1].tolist() == [4, 5, 6, 7, 8, 9]


def test_meanpool_closed_form():
    # q rows: group 0 = {[1,0],[0,1]} -> qbar [0.5,0.5]; group 1 = {[2,2],[0,0]}
    # k blocks of 2: {[1,0],[3,0]} -> kbar [2,0]; {[0,1],[0,-1]} -> kbar [0,0]
    q = np.array([[1, 0], [0, 1], [2, 2], [0, 0]], float)
    k = np.array([[1, 0], [3, 0], [0, 1], [0, -1]], float)
    perm = np.arange(4)
    s = var.meanpool_scores(q, k, perm, 4, 2, 2, 1.0)
    np.testing.assert_array_equal(s, [[1.0, 0.0], [2.0, 0.0]])
    # n_valid = 3: block 1 is {[0,1]} alone and query 3 is padding, so group 1
    # pools only [2,2]: scores g0 = [1, 0.5], g1 = [4, 2]
    s3 = var.meanpool_scores(q, k, perm, 3, 2, 2, 1.0)
    np.testing.assert_array_equal(s3, [[1.0, 0.5], [4.0, 2.0]])
    # equal scores go to the lower block index
    assert var.select_blocks([[1.0, 1.0, 0.5]], 1).tolist() == [[0]]


def test_block_scores_conserve_probability_mass():
    q, k, v, nv, sc = layer()
    _, lse = orc.dense_attention(q, k, v, nv, sc)
    C, B = 32, 16
    perm = var.identity_perm(len(q))
    a = orc.group_scores(q, k, perm, lse, nv, C, sc)
    bs = var.block_oracle_scores(a, nv, B)
    assert bs.shape == (len(q) // C, len(var.kv_blocks(nv, B)))
    members = [(perm[g * C:(g + 1) * C] < nv).sum() for g in range(len(q) // C)]
    np.testing.assert_allclose(bs.sum(axis=1), members, atol=1e-10)


def test_unit_blocks_make_the_block_oracle_the_token_oracle():
    q, k, v, nv, sc = layer(seed=1)
    _, lse = orc.dense_attention(q, k, v, nv, sc)
    C, topk = 32, 40
    perm = var.identity_perm(len(q))
    a = orc.group_scores(q, k, perm, lse, nv, C, sc)
    bs = var.block_oracle_scores(a, nv, 1)
    np.testing.assert_array_equal(bs, a)
    nb = var.block_budget(topk, 1, nv)
    toks = var.expand_blocks(var.select_blocks(bs, nb), nv, 1)
    np.testing.assert_array_equal(np.stack(toks), orc.topk_select(a, topk))


def test_all_blocks_give_dense_attention():
    q, k, v, nv, sc = layer(seed=2)
    C, B = 32, 16
    perm = var.identity_perm(len(q))
    o_dense, lse = orc.dense_attention(q, k, v, nv, sc)
    for scores in (var.block_oracle_scores(orc.group_scores(q, k, perm, lse, nv, C, sc), nv, B),
                   var.meanpool_scores(q, k, perm, nv, C, B, sc)):
        nb = scores.shape[1]
        toks = var.expand_blocks(var.select_blocks(scores, nb), nv, B)
        o = orc.sparse_attention(q, k, v, perm, toks, nv, C, sc)
        np.testing.assert_allclose(o[:nv], o_dense[:nv], atol=1e-12)


def test_single_query_groups_reduce_to_the_per_query_oracle():
    q, k, v, nv, sc = layer(n=64, nv=60, seed=3)
    topk = 12
    perm = var.identity_perm(len(q))
    o_pq = var.per_query_attention(q, k, v, nv, topk, sc)
    _, lse = orc.dense_attention(q, k, v, nv, sc)
    # token oracle with C = 1: a group's score of key j is p_ij itself
    a = orc.group_scores(q, k, perm, lse, nv, 1, sc)
    kv = orc.topk_select(a[:nv], topk)
    kv_all = list(kv) + [kv[0]] * (len(q) - nv)
    o_tok = orc.sparse_attention(q, k, v, perm, kv_all, nv, 1, sc)
    np.testing.assert_allclose(o_tok[:nv], o_pq[:nv], atol=1e-12)
    # vanilla BSA with one query per group and one key per block ranks the
    # logits themselves, which order p_ij the same way for a fixed query
    s = var.meanpool_scores(q, k, perm, nv, 1, 1, sc)
    toks = var.expand_blocks(var.select_blocks(s[:nv], topk), nv, 1)
    np.testing.assert_array_equal(np.stack(toks), kv)
    assert np.all(o_pq[nv:] == 0)


def test_per_query_oracle_brute_force():
    rng = np.random.default_rng(4)
    n, d, topk = 7, 3, 3
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    sc = 0.7
    o = var.per_query_attention(q, k, v, n, topk, sc)
    for i in range(n):
        p = np.exp(sc * k @ q[i])
        best = max(itertools.combinations(range(n), topk), key=lambda c: p[list(c)].sum())
        w = p[list(best)] / p[list(best)].sum()
        np.testing.assert_allclose(o[i], w @ v[list(best)], atol=1e-12)


def test_retained_mass_ordering_of_the_oracles():
    """Per query, the per-query oracle keeps at least the token oracle's mass;
    per group, the token oracle keeps at least the block oracle's mass at the
    same token count (each is the best set of its size for its objective)."""
    q, k, v, nv, sc = layer(seed=5)
    _, lse = orc.dense_attention(q, k, v, nv, sc)
    C, B, topk = 32, 8, 48
    G = len(q) // C
    perm = var.identity_perm(len(q))
    a = orc.group_scores(q, k, perm, lse, nv, C, sc)
    tok = orc.topk_select(a, topk)
    m_tok = var.retained_mass(q, k, nv, sc, lse, var.group_sets_per_query(perm, tok, nv, C))
    pq_sets = [np.lexsort((np.arange(nv), -(k[:nv] @ q[i])))[:topk] for i in range(nv)]
    m_pq = var.retained_mass(q, k, nv, sc, lse, pq_sets)
    assert np.all(m_pq >= m_tok - 1e-12)
    blocks = var.expand_blocks(var.select_blocks(var.block_oracle_scores(a, nv, B),
                                                 var.block_budget(topk, B, len(var.kv_blocks(nv, B)))), nv, B)
    m_blk = var.retained_mass(q, k, nv, sc, lse, var.group_sets_per_query(perm, blocks, nv, C))
    for g in range(G):
        same = orc.topk_select(a[[g]], len(blocks[g]))[0]
        m_same = var.retained_mass(q, k, nv, sc, lse, var.group_sets_per_query(perm[g * C:], [same], nv, C))
        mem = [i for i in perm[g * C:(g + 1) * C] if i < nv]
        assert sum(m_same[i] for i in mem) >= sum(m_blk[i] for i in mem) - 1e-12
