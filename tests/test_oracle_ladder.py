"""The oracle analysis of the onedev.kr summary ("how it works") on a small
synthetic layer, all in the fp64 oracle: per-query, token and block oracles
(exact probabilities) and mean-pooled vanilla BSA at one density.  The per-
query oracle exists only here (CPU).  Checked: the retained-mass orderings the
oracles guarantee (per query: per-query >= token; per group at equal token
count: token >= block); the output errors are printed for the record."""
import dataclasses

import numpy as np
import pytest

import synthdata as sd
from oracle import mcs_oracle as orc
from oracle import variants as var
from tests import parity as par


@pytest.mark.parametrize("layout", ["random", "grid"])
def test_oracle_ladder(layout):
    cfg = dataclasses.replace(sd.CONFIGS["tiny"], layout=layout)
    q, k, v = (par.bf16_to_f64(t[0, 0]) for t in sd.generate(cfg, steps=1)[0])
    nv, C, sc, topk = cfg.n_valid, cfg.group_size, cfg.scale, cfg.topk
    B = C
    nb = var.block_budget(topk, B, len(var.kv_blocks(nv, B)))
    pid = var.identity_perm(cfg.n_pad)
    o_d, lse = orc.dense_attention(q, k, v, nv, sc)
    rel = lambda o: float(np.linalg.norm(o[:nv] - o_d[:nv]) / np.linalg.norm(o_d[:nv]))  # noqa: E731

    o_pq = var.per_query_attention(q, k, v, nv, topk, sc)
    a = orc.group_scores(q, k, pid, lse, nv, C, sc)
    tok = orc.topk_select(a, topk)
    o_tok = orc.sparse_attention(q, k, v, pid, tok, nv, C, sc)
    blk = var.expand_blocks(var.select_blocks(var.block_oracle_scores(a, nv, B), nb), nv, B)
    o_blk = orc.sparse_attention(q, k, v, pid, blk, nv, C, sc)
    bsa = var.expand_blocks(var.select_blocks(var.meanpool_scores(q, k, pid, nv, C, B, sc), nb), nv, B)
    o_bsa = orc.sparse_attention(q, k, v, pid, bsa, nv, C, sc)
    errs = {"per-query oracle": rel(o_pq), "token oracle": rel(o_tok), "block oracle": rel(o_blk),
            "vanilla BSA": rel(o_bsa)}
    print(f"tiny, {layout} labels, k={topk} ({nb} blocks of {B}):",
          ", ".join(f"{n} {e:.4f}" for n, e in errs.items()))

    pq_sets = [np.lexsort((np.arange(nv), -(k[:nv] @ q[i])))[:topk] for i in range(nv)]
    m_pq = var.retained_mass(q, k, nv, sc, lse, pq_sets)
    m_tok = var.retained_mass(q, k, nv, sc, lse, var.group_sets_per_query(pid, tok, nv, C))
    assert np.all(m_pq >= m_tok - 1e-12)
    m_blk = var.retained_mass(q, k, nv, sc, lse, var.group_sets_per_query(pid, blk, nv, C))
    m_bsa = var.retained_mass(q, k, nv, sc, lse, var.group_sets_per_query(pid, bsa, nv, C))
    for g in range(cfg.groups):
        mem = [i for i in pid[g * C:(g + 1) * C] if i < nv]
        same = orc.topk_select(a[[g]], len(blk[g]))[0]
        m_same = var.retained_mass(q, k, nv, sc, lse, var.group_sets_per_query(pid[g * C:], [same], nv, C))
        assert sum(m_same[i] for i in mem) >= sum(m_blk[i] for i in mem) - 1e-12
        # the block oracle keeps at least the mass of any other choice of nb blocks
        assert sum(m_blk[i] for i in mem) >= sum(m_bsa[i] for i in mem) - 1e-12
