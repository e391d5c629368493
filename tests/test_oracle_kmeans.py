"""Pins of the size-balanced k-means oracle (oracle/kmeans.py) against things
fixed outside it: hand-worked bf16 roundings and a library conversion, the
plain squared distance, a library stable sort, and well-separated clusters
that any correct k-means recovers exactly."""
import numpy as np
import pytest
import torch

from oracle import kmeans as km


def test_bf16_round_worked_examples():
    # 8 significant bits: the neighbours of 1 are 1 - 2^-8 and 1 + 2^-7
    cases = [
        (1.0 + 2.0 ** -8, 1.0),                 # halfway, to the even neighbour
        (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),  # halfway, to the even neighbour
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),  # just above halfway
        (-(1.0 + 2.0 ** -8 + 2.0 ** -30), -(1.0 + 2.0 ** -7)),
        (3.0, 3.0),
        (0.0, 0.0),
        (2.0 ** -133, 2.0 ** -133),            # smallest bf16 subnormal
        (2.0 ** -135, 0.0),                    # below half of it
    ]
    for x, want in cases:
        assert km.bf16_round(x) == want, x


def test_bf16_round_matches_library_on_fp32_values():
    # values exactly representable in fp32: torch's fp32 -> bf16 conversion
    # (round to nearest even) rounds once, so it must agree
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-30,
                        rng.standard_normal(2000) * 1e30]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(km.bf16_round(x.astype(np.float64)), want)


def test_distances_rank_like_the_squared_distance():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 16))
    mu = km.bf16_round(rng.standard_normal((12, 16)))
    direct = ((x[:, None, :] - mu[None, :, :]) ** 2).sum(axis=2)
    # the two differ by ||x||^2 only
    assert np.allclose(km.distances(x, mu) + (x * x).sum(axis=1)[:, None], direct, atol=1e-10)
    assert np.array_equal(km.assign(x, mu), np.argmin(direct, axis=1))


def test_assign_ties_go_to_the_lower_centroid():
    mu = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 0.0]])
    x = np.array([[1.0, 1.0], [2.0, 0.0], [0.0, 0.0]])
    assert list(km.assign(x, mu)) == [0, 0, 0]


def test_centroids_are_rounded_group_means():
    x = np.arange(24, dtype=np.float64).reshape(8, 3) / 7.0
    perm = np.array([7, 0, 5, 2, 1, 3, 4, 6])
    mu = km.centroids(x, perm, 4)
    want = np.stack([x[[7, 0, 5, 2]].mean(axis=0), x[[1, 3, 4, 6]].mean(axis=0)])
    assert np.array_equal(mu, km.bf16_round(want))
    # identical members: the centroid is the (rounded) row itself
    y = np.tile(np.array([[0.3, -1.7]]), (6, 1))
    assert np.array_equal(km.centroids(y, np.arange(6), 3), km.bf16_round(y[:2]))


def test_balance_is_a_stable_sort_by_label():
    rng = np.random.default_rng(3)
    lab = rng.integers(0, 7, size=64)
    perm = km.balance(lab, 8)
    assert np.array_equal(perm, np.lexsort((np.arange(64), lab)))
    assert sorted(perm) == list(range(64))
    # labels are non-decreasing along the order, indices increase inside a label
    assert np.all(np.diff(lab[perm]) >= 0)


def test_zero_iterations_is_the_identity():
    x = np.random.default_rng(4).standard_normal((32, 4))
    assert np.array_equal(km.balanced_kmeans(x, 8, 0), np.arange(32))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_well_separated_equal_clusters_are_recovered(seed):
    """G clusters of exactly C points around far-apart centres; each initial
    block of C tokens holds C-2 points of its own cluster and one of each
    neighbouring cluster (cyclic exchanges), so the first centroids sit near
    the true centres and
    one iteration must return the clusters exactly, group g = cluster g, with
    the SSE of their closed-form spread; further iterations keep it."""
    rng = np.random.default_rng(seed)
    G, C, d = 6, 8, 5
    centres = 40.0 * rng.standard_normal((G, d))
    noise = 0.1 * rng.standard_normal((G * C, d))
    truth = np.repeat(np.arange(G), C)
    order = np.arange(G * C)
    for g in range(G):                  # swap the last token of block g with the first of g+1
        a, b = g * C + C - 1, ((g + 1) % G) * C
        order[a], order[b] = order[b], order[a]
    x = (centres[truth] + noise)[order]
    lab_true = truth[order]
    for iters in (1, 3):
        perm = km.balanced_kmeans(x, C, iters)
        for g in range(G):
            assert set(lab_true[perm[g * C:(g + 1) * C]]) == {g}
    sse_true = sum(((noise[truth == g] - noise[truth == g].mean(axis=0)) ** 2).sum() for g in range(G))
    assert km.group_sse(x, perm, C) == pytest.approx(sse_true, rel=1e-9)
    assert km.group_sse(x, np.arange(G * C), C) > 10 * sse_true


def test_group_sse_closed_form():
    # two groups {0, 2} and {1, 3} of 1-D points: SSE = (a-b)^2/2 per pair
    x = np.array([[0.0], [10.0], [4.0], [13.0]])
    assert km.group_sse(x, np.array([0, 2, 1, 3]), 2) == pytest.approx(8.0 + 4.5)
