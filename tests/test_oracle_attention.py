"""Pins of the oracle's dense pass, sparse pass, residual and reuse step.

Each check ties the oracle to something other than itself: a library routine
(torch's fp64 scaled_dot_product_attention / softmax), hand-derived closed forms
(tests/golden/closed_forms.json), special cases with a closed-form answer, and
invariants of the anchor/reuse formula O_t = SparseAttn(...) + R with
R = O_full - O_sparse (onedev.kr summary, "what is different").
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mcs_oracle as orc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def rand_head(n, d, seed, n_valid=None, mean=0.0):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((n, d)) + mean for _ in range(3))
    if n_valid is not None:
        q[n_valid:] = k[n_valid:] = v[n_valid:] = 0.0
    return q, k, v


def sdpa(q, k, v, scale):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], scale=scale)
    return out[0].numpy()


# ---------------------------------------------------------------- dense ----
@pytest.mark.parametrize("n,n_valid,d", [(128, 128, 64), (192, 170, 32), (64, 1, 16)])
def test_dense_matches_torch_sdpa(n, n_valid, d):
    q, k, v = rand_head(n, d, 1, n_valid)
    sc = orc.softmax_scale(d)
    o, lse = orc.dense_attention(q, k, v, n_valid, sc, block=50)
    ref = sdpa(q[:n_valid], k[:n_valid], v[:n_valid], sc)
    np.testing.assert_allclose(o[:n_valid], ref, atol=1e-12, rtol=0)
    assert np.all(o[n_valid:] == 0) and np.all(lse[n_valid:] == 0)
    # LSE normalises the exact probabilities: sum_j exp(s_ij - LSE_i) = 1
    s = sc * q[:n_valid] @ k[:n_valid].T
    np.testing.assert_allclose(np.exp(s - lse[:n_valid, None]).sum(1), 1.0, atol=1e-12)
    ref_lse = torch.logsumexp(torch.from_numpy(s), dim=1).numpy()
    np.testing.assert_allclose(lse[:n_valid], ref_lse, atol=1e-12)


def test_dense_row_subset_matches_full():
    q, k, v = rand_head(160, 16, 21, 150)
    o, lse = orc.dense_attention(q, k, v, 150, 0.25)
    rows = np.array([155, 3, 149, 77, 0])
    o2, l2 = orc.dense_attention(q, k, v, 150, 0.25, rows=rows)
    np.testing.assert_array_equal(o2, o[rows])
    np.testing.assert_array_equal(l2, lse[rows])


def test_dense_closed_form_two_keys():
    g = GOLD["two_key_attention"]
    q, k, v = (np.array(g[x], np.float64) for x in ("q", "k", "v"))
    o, lse = orc.dense_attention(q, k, v, 2, 1 / math.sqrt(2))
    np.testing.assert_allclose(o, g["o"], atol=1e-15)
    np.testing.assert_allclose(lse, g["lse"], atol=1e-15)


def test_dense_zero_query_is_mean_and_log_n():
    q, k, v = rand_head(96, 16, 2, 80)
    q[:] = 0.0
    o, lse = orc.dense_attention(q, k, v, 80, 0.25)
    np.testing.assert_allclose(o[:80], np.broadcast_to(v[:80].mean(0), (80, 16)), atol=1e-13)
    np.testing.assert_allclose(lse[:80], math.log(80), atol=1e-13)


def test_padding_does_not_change_valid_rows():
    q, k, v = rand_head(256, 32, 3, 200)
    sc = orc.softmax_scale(32)
    o_p, lse_p = orc.dense_attention(q, k, v, 200, sc)
    o_u, lse_u = orc.dense_attention(q[:200], k[:200], v[:200], 200, sc)
    np.testing.assert_allclose(o_p[:200], o_u, atol=1e-12)
    np.testing.assert_allclose(lse_p[:200], lse_u, atol=1e-12)


# --------------------------------------------------------------- sparse ----
def test_sparse_closed_form_three_keys():
    g = GOLD["three_key_sparse"]
    q, k, v = (np.array(g[x], np.float64) for x in ("q", "k", "v"))
    sc = 1 / math.sqrt(2)
    o_full, _ = orc.dense_attention(q, k, v, 3, sc)
    o_sp = orc.sparse_attention(q, k, v, np.array([0]), np.array([g["kv_idx"]]), 1, 1, sc)
    r = orc.residual(o_full, o_sp, 1)
    np.testing.assert_allclose(o_full, g["o_full"], atol=1e-15)
    np.testing.assert_allclose(o_sp, g["o_sparse"], atol=1e-15)
    np.testing.assert_allclose(r, g["r"], atol=1e-15)


def test_sparse_full_density_equals_dense():
    n, nv, C, d = 256, 240, 64, 32
    q, k, v = rand_head(n, d, 4, nv)
    sc = orc.softmax_scale(d)
    perm = np.random.default_rng(5).permutation(n)
    G = n // C
    kv = np.tile(np.arange(nv), (G, 1))
    o_sp = orc.sparse_attention(q, k, v, perm, kv, nv, C, sc)
    ref = np.zeros((n, d))
    ref[:nv] = sdpa(q[:nv], k[:nv], v[:nv], sc)
    np.testing.assert_allclose(o_sp, ref, atol=1e-12)


def test_sparse_single_key_is_that_value_row():
    n, C, d = 128, 32, 16
    q, k, v = rand_head(n, d, 6)
    perm = np.random.default_rng(7).permutation(n)
    kv = np.array([[5], [77], [0], [127]])
    o = orc.sparse_attention(q, k, v, perm, kv, n, C, 0.25)
    for g in range(4):
        for i in perm[g * C:(g + 1) * C]:
            np.testing.assert_array_equal(o[i], v[kv[g, 0]])


def test_sparse_constant_values_and_zero_queries():
    n, C, d = 128, 64, 16
    q, k, v = rand_head(n, d, 8)
    perm = np.arange(n)
    rng = np.random.default_rng(9)
    kv = np.sort(np.stack([rng.choice(n, 20, replace=False) for _ in range(2)]), axis=1)
    u = rng.standard_normal(d)
    vc = np.broadcast_to(u, (n, d)).copy()
    o_full, _ = orc.dense_attention(q, k, vc, n, 0.25)
    o_sp = orc.sparse_attention(q, k, vc, perm, kv, n, C, 0.25)
    np.testing.assert_allclose(o_full, vc, atol=1e-13)
    np.testing.assert_allclose(o_sp, vc, atol=1e-13)
    np.testing.assert_allclose(orc.residual(o_full, o_sp, n), 0.0, atol=1e-13)
    o0 = orc.sparse_attention(np.zeros_like(q), k, v, perm, kv, n, C, 0.25)
    for g in range(2):
        np.testing.assert_allclose(o0[g * C:(g + 1) * C], np.broadcast_to(v[kv[g]].mean(0), (C, d)), atol=1e-13)


def test_anchor_identity_and_zero_drift_reuse():
    n, nv, C, d = 256, 250, 64, 32
    q, k, v = rand_head(n, d, 10, nv)
    sc = orc.softmax_scale(d)
    res = orc.anchor_pipeline(q, k, v, nv, C, 40, sc, power_iters=20)
    np.testing.assert_allclose(res["o_sparse"] + res["r"], res["o_full"], atol=1e-12)
    o_t = orc.reuse_step(q, k, v, res["perm"], res["kv_idx"], res["r"], nv, C, sc)
    np.testing.assert_allclose(o_t, res["o_full"], atol=1e-12)
    assert np.all(o_t[nv:] == 0)


def test_reuse_group_subset_matches_full():
    n, C, d = 256, 64, 16
    q, k, v = rand_head(n, d, 11)
    sc = 0.25
    perm = np.random.default_rng(12).permutation(n)
    rng = np.random.default_rng(13)
    kv = np.sort(np.stack([rng.choice(n, 30, replace=False) for _ in range(4)]), axis=1)
    r = rng.standard_normal((n, d))
    full = orc.reuse_step(q, k, v, perm, kv, r, n, C, sc)
    sub = orc.reuse_step(q, k, v, perm, kv[[1, 3]], r, n, C, sc, groups=[1, 3])
    for g in (1, 3):
        rows = perm[g * C:(g + 1) * C]
        np.testing.assert_allclose(sub[rows], full[rows], atol=1e-13)
