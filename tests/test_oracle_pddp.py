"""Pins of the oracle's Fast PDDP grouping.

onedev.kr summary, "how it is used", component 2: equal-size groups of exactly
the query tile C, built by recursive median splits along each node's principal
direction, computed with power iteration.  Pins: the principal direction from
numpy.linalg.eigh of the centred covariance (a library routine), exact
partition/size invariants, recovery of two separated clusters, a brute-force
sort by the eigh projection for one split, and the hand-derived fixtures.
"""
import json
import os

import numpy as np
import pytest

from oracle import mcs_oracle as orc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def elongated(n, d, seed, mean_shift=5.0, gap=10.0):
    """Rows with one dominant centred direction and a large common mean that is
    orthogonal to it (an uncentred iteration would lock onto the mean)."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    m = rng.standard_normal(d)
    m -= (m @ u) * u
    m *= mean_shift / np.linalg.norm(m)
    t = rng.standard_normal(n) * gap
    return m + np.outer(t, u) + 0.3 * rng.standard_normal((n, d)), u


def top_eigvec(x):
    y = x - x.mean(0)
    w, vecs = np.linalg.eigh(y.T @ y)
    return vecs[:, -1], w


def test_node_table_fixture():
    lv = GOLD["node_table_G5"]["levels"]
    for depth, nodes in enumerate(lv):
        assert orc.pddp_node_table(5, depth) == [tuple(n) for n in nodes]


def test_line_split_fixture():
    g = GOLD["line_split"]
    x = np.array(g["x"])
    mu, v = orc.pddp_node_direction(x, 20)
    np.testing.assert_allclose(v, g["direction"], atol=1e-15)
    np.testing.assert_allclose((x - mu) @ v, g["projections"], atol=1e-14)
    assert list(orc.pddp_groups(x, g["C"])) == g["perm"]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_direction_matches_eigh(seed):
    x, u = elongated(300, 24, seed)
    vec, w = top_eigvec(x)
    assert (w[-2] / w[-1]) ** 40 < 1e-9
    _, v = orc.pddp_node_direction(x, 20)
    assert 1 - abs(v @ vec) < 1e-9
    j = int(np.argmax(np.abs(v)))
    assert v[j] > 0 and np.isclose(np.linalg.norm(v), 1.0)


def test_sign_rule_ties_take_lowest_index():
    # direction (-1, 1)/sqrt(2): both components have equal magnitude, so the
    # first one is made positive.
    t = np.array([-3.0, -1.0, 1.0, 3.0])
    x = np.outer(t, [-1.0, 1.0]) / np.sqrt(2)
    _, v = orc.pddp_node_direction(x, 20)
    np.testing.assert_allclose(v, [1 / np.sqrt(2), -1 / np.sqrt(2)], atol=1e-15)


def test_zero_spread_node_keeps_initial_direction():
    x = np.ones((8, 4)) * 2.5
    mu, v = orc.pddp_node_direction(x, 20)
    np.testing.assert_allclose(v, np.full(4, 0.5))
    np.testing.assert_allclose(mu, 2.5)


def test_single_split_is_sort_by_eigh_projection():
    C = 64
    x, _ = elongated(2 * C, 16, 7)
    vec, _ = top_eigvec(x)
    j = int(np.argmax(np.abs(vec)))
    vec = vec if vec[j] > 0 else -vec
    p = (x - x.mean(0)) @ vec
    left = np.sort(np.argsort(p, kind="stable")[:C])
    perm = orc.pddp_groups(x, C)
    np.testing.assert_array_equal(perm[:C], left)


def test_two_clusters_recovered_by_one_split():
    rng = np.random.default_rng(3)
    C, d = 32, 8
    a = rng.standard_normal(d) * 4
    lab = rng.permutation(np.repeat([0, 1], C))
    x = np.where(lab[:, None] == 0, a, -a) + 0.1 * rng.standard_normal((2 * C, d))
    perm = orc.pddp_groups(x, C)
    assert len(set(lab[perm[:C]])) == 1 and len(set(lab[perm[C:]])) == 1


@pytest.mark.parametrize("n_groups,C", [(5, 8), (7, 16), (16, 4), (13, 8)])
def test_partition_and_sizes(n_groups, C):
    rng = np.random.default_rng(n_groups)
    n = n_groups * C
    x = rng.standard_normal((n, 6))
    x[n - 3:] = 0.0                        # a few identical (padding-like) rows
    L = int(np.ceil(np.log2(n_groups)))
    perm = np.arange(n)
    for lv in range(L):
        new = orc.pddp_split_level(x, perm, C, n_groups, lv)
        # children are subsets of their parent node
        for s, m in orc.pddp_node_table(n_groups, lv):
            assert set(new[s * C:(s + m) * C]) == set(perm[s * C:(s + m) * C])
        perm = new
    assert sorted(perm) == list(range(n))
    for g in range(n_groups):
        grp = perm[g * C:(g + 1) * C]
        assert len(grp) == C and np.all(np.diff(grp) > 0)
    assert np.array_equal(perm, orc.pddp_groups(x, C))
    assert all(m == 1 for _, m in orc.pddp_node_table(n_groups, L))


@pytest.mark.parametrize("n_groups,C", [(5, 8), (7, 4), (11, 4)])
def test_left_child_holds_the_floor_half_smallest_projections(n_groups, C):
    """Every split puts exactly floor(m/2)*C members, the ones with the smallest
    projections on the node's direction, into the left child."""
    rng = np.random.default_rng(100 + n_groups)
    n = n_groups * C
    x = rng.standard_normal((n, 5)) * np.array([6.0, 3.0, 1.0, 0.5, 0.2])
    perm = np.arange(n)
    L = int(np.ceil(np.log2(n_groups)))
    for lv in range(L):
        new = orc.pddp_split_level(x, perm, C, n_groups, lv)
        for s, m in orc.pddp_node_table(n_groups, lv):
            if m < 2:
                continue
            mem = np.sort(perm[s * C:(s + m) * C])
            mu, v = orc.pddp_node_direction(x[mem], 20)
            h = m // 2
            left = new[s * C:(s + h) * C]
            right = new[(s + h) * C:(s + m) * C]
            assert len(left) == h * C
            assert ((x[left] - mu) @ v).max() <= ((x[right] - mu) @ v).min()
        perm = new
