"""fp64 CPU oracle of the size-balanced k-means grouping (the comparator of
Fast PDDP).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import or run this module.  It shares no code with the HIP
library and imports nothing from it.

Source: [onedev] "how it is used", component 2: the query tile needs groups of
exactly C; k-means does not give equal sizes and a forced balance constraint
makes its assignment dearer, which is why the method splits by PDDP medians.
The system paragraph compares Fast PDDP's grouping cost with Flash-KMeans.
The pages define no balanced k-means of their own; the comparator is this
reading of one (the R-numbers continue the design notes' register):

  R37  Initial partition: contiguous token blocks of C (the identity perm).
  R38  One iteration from partition P: centroid mu_g = mean of group g's C
       rows, computed in fp64 and rounded once to bf16 (round to nearest,
       ties to even), the precision the distance products take on matrix
       cores.
  R39  Assignment: label_i = argmin_g ||x_i - mu_g||^2, ties to the lower g.
       ||x_i||^2 is the same for every g, so the GPU compares
       ||mu_g||^2 - 2 x_i . mu_g; the oracle compares the same quantity in
       fp64, and the checker accepts a GPU label within an fp32 rounding
       margin of the best (where floating point decides an index, only the
       unambiguous decisions are unique).
  R40  Balance: tokens ordered by (label, token index); group g takes
       positions g*C .. g*C+C-1.  A cluster larger than C spills into the next
       group, a smaller one shares its group with the next label's tokens:
       the cheapest way to tile-aligned groups, so the comparison favours
       k-means.
  R41  Padded rows (>= n_valid) take part as all-zero rows, as in PDDP.

Parity status: every function is pinned by tests/test_oracle_kmeans.py
(rounding examples and a library conversion, brute-force distances,
well-separated clusters recovered exactly, a library stable sort,
invariants).
"""
from __future__ import annotations

import numpy as np

__all__ = ["bf16_round", "centroids", "distances", "assign", "balance", "iterate",
           "balanced_kmeans", "group_sse"]


def bf16_round(x):
    """Round fp64 values to the nearest bf16 value, ties to even (8
    significant bits, the fp32 exponent range; R38)."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # below 2^-126 the quantum stays 2^-133
    scaled = np.ldexp(x, 8 - e)             # exact: a power-of-two scaling
    return np.ldexp(np.rint(scaled), e - 8)  # rint rounds half to even


def centroids(x, perm, C):
    """mu [G, d]: fp64 mean of each group's C rows, rounded to bf16 (R38)."""
    x = np.asarray(x, np.float64)
    perm = np.asarray(perm)
    G = perm.shape[0] // C
    mu = x[perm].reshape(G, C, x.shape[1]).mean(axis=1)
    return bf16_round(mu)


def distances(x, mu):
    """[N, G]: ||mu_g||^2 - 2 x_i . mu_g in fp64 (R39)."""
    x = np.asarray(x, np.float64)
    mu = np.asarray(mu, np.float64)
    return (mu * mu).sum(axis=1)[None, :] - 2.0 * (x @ mu.T)


def assign(x, mu):
    """label_i = argmin over g, ties to the lower g (np.argmin keeps the
    first minimum)."""
    return np.argmin(distances(x, mu), axis=1)


def balance(labels, C):
    """Tokens ordered by (label, token index), cut into groups of C (R40)."""
    labels = np.asarray(labels)
    assert labels.shape[0] % C == 0
    return np.argsort(labels, kind="stable").astype(np.int64)


def iterate(x, perm, C):
    """One iteration from partition perm: (labels, new perm)."""
    lab = assign(x, centroids(x, perm, C))
    return lab, balance(lab, C)


def balanced_kmeans(x, C, iters):
    """perm [N_pad] after `iters` iterations from contiguous blocks (R37)."""
    perm = np.arange(np.asarray(x).shape[0])
    for _ in range(iters):
        _, perm = iterate(x, perm, C)
    return perm


def group_sse(x, perm, C):
    """Within-group sum of squared distances to the group mean (fp64), the
    quantity both k-means and the PDDP splits try to keep small."""
    x = np.asarray(x, np.float64)
    perm = np.asarray(perm)
    G = perm.shape[0] // C
    xg = x[perm].reshape(G, C, x.shape[1])
    return float(((xg - xg.mean(axis=1, keepdims=True)) ** 2).sum())
