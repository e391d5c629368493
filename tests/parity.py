"""Comparison rules between the HIP path and the fp64 oracle (test helpers).

Floating-point outputs (bf16 with fp32 accumulation): max abs error <= 2e-2 and
mean abs error <= 1e-3 over valid rows.

KV index sets: bit-exact, except where the oracle's k-th and (k+1)-th largest
aggregated probabilities are closer than EPS_SEL = 1e-6; inside such a band the
GPU set must still contain every key the oracle scores above tau + eps, hold
only keys scoring at least tau' - eps, and have exactly k distinct members.

Grouping: level by level, the GPU's partition at depth l-1 is fed to the
oracle's split; the children must match as sets, except for rows whose oracle
projection lies within EPS_PDDP * max|p| of the node's split boundary.

Balanced k-means (the PDDP comparator): iteration by iteration, the GPU's
previous partition is fed to the oracle.  Centroids (fp64 means rounded once
to bf16) are the same on both sides; a GPU label must be a nearest centroid up
to the fp32 accumulation margin EPS_KM * (2 sum|x.mu| + ||mu||^2), and equal to
the oracle's wherever the best centroid beats every other by more than the
margins; the GPU's new partition must be exactly the oracle's balance of the
GPU's labels.
"""
from __future__ import annotations

import numpy as np

from oracle import mcs_oracle as orc

MAX_ABS = 2e-2
MEAN_ABS = 1e-3
EPS_SEL = 1e-6
EPS_PDDP = 1e-9
# block selections (oracle-analysis variants): block scores are fp64 sums
# ranked in fp32 on the GPU; ties are resolved within EPS_BLK * max|score|
EPS_BLK = 1e-5
# k-means distances: bf16 dot products of d <= 128 terms accumulated in fp32
# (|error| <= d * 2^-24 * sum|x.mu| ~ 2^-17 of it), then one fma with the fp32
# ||mu||^2; 2^-14 covers both, with a factor 4 to spare
EPS_KM = 2.0 ** -14


def bf16_to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, rows=None, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max abs {mx:.3e}, mean abs {mean:.3e}"
    return mx, mean


def check_selection(gpu_idx, a_row, k):
    """Compare one group's GPU index set with the oracle scores a_row.
    Returns 'strict' or 'band' (which rule applied)."""
    gpu_idx = np.asarray(gpu_idx)
    assert len(gpu_idx) == k
    assert np.all(np.diff(gpu_idx) > 0), "indices not strictly ascending"
    assert gpu_idx.min() >= 0 and gpu_idx.max() < len(a_row), "index out of range"
    ref = orc.topk_select(a_row[None], k)[0]
    srt = np.sort(a_row)[::-1]
    tau = srt[k - 1]
    tau_next = srt[k] if k < len(a_row) else -np.inf
    if tau - tau_next >= EPS_SEL:
        assert np.array_equal(gpu_idx, ref), "selection differs outside the tie band"
        return "strict"
    must = np.nonzero(a_row > tau + EPS_SEL)[0]
    assert np.all(np.isin(must, gpu_idx)), "a clearly selected key is missing"
    assert np.all(a_row[gpu_idx] >= tau_next - EPS_SEL), "a clearly rejected key was selected"
    return "band"


def check_selection_exact(gpu_idx, gpu_scores_row, k):
    """Index work on the same inputs: the GPU's kv_idx row must be exactly the
    oracle's top-k (ties to the lower key index, ascending) of the fp32 scores
    the GPU ranked (fp32 -> fp64 is exact, so the order is the same)."""
    ref = orc.topk_select(np.asarray(gpu_scores_row, np.float64)[None], k)[0]
    assert np.array_equal(np.asarray(gpu_idx, np.int64), ref), \
        "selection differs from the top-k of the GPU's own scores"


# fp32 error of the score pass, per term exp2(x) with
#   x = fma(s, c2, -lse2),  s = q.k accumulated in fp32 from exact bf16
#   products, c2 = fp32(fp32(scale) * fp32(log2 e)), lse2 = fp32(lse * log2 e),
# against the fp64 value with the same (fp32) lse:
#   |dx| <= c2 * d * 2^-23 * sum|q_e k_e|          (accumulation of d products,
#                                                    2u per add for safety)
#         + 2^-24 * (3 |s| c2 + |x| + 2 |lse| log2 e) (scale, fma, lse2 roundings)
#   the term's relative error <= ln2 |dx| + 2^-22    (v_exp_f32, 4 ulp allowed)
# then the sum of the group's C terms (16 in a lane, the other half-wave, the
# wavefront partials: 20 adds deep) <= 40 * 2^-24 of the sum, and every term
# may flush to zero below 2^-126.
def score_error_bound(q_rows, k, lse_rows, scale, n_valid):
    """Elementwise bound on |a_gpu - a| for one group (q_rows: its valid
    members, lse_rows their fp32 lse as fp64; k: [n_valid, d])."""
    q_rows = np.asarray(q_rows, np.float64)
    k = np.asarray(k, np.float64)[:n_valid]
    lse_rows = np.asarray(lse_rows, np.float64)
    d = q_rows.shape[1]
    log2e = 1.0 / np.log(2.0)
    c2 = scale * log2e
    s = q_rows @ k.T
    sabs = np.abs(q_rows) @ np.abs(k).T
    x = (scale * s - lse_rows[:, None]) * log2e
    t = np.exp2(x)
    dx = c2 * d * 2.0 ** -23 * sabs + 2.0 ** -24 * (3 * np.abs(s) * c2 + np.abs(x)
                                                     + 2 * np.abs(lse_rows)[:, None] * log2e)
    per_term = t * (np.log(2.0) * dx + 2.0 ** -22)
    a = t.sum(axis=0)
    return per_term.sum(axis=0) + 40 * 2.0 ** -24 * a + q_rows.shape[0] * 2.0 ** -126


def check_scores(gpu_row, ref_row, bound_row):
    """fp32 group scores against the oracle's (computed with the GPU's lse),
    elementwise within score_error_bound.  Returns (max relative error, max
    error / bound)."""
    gpu_row = np.asarray(gpu_row, np.float64)
    ref_row = np.asarray(ref_row, np.float64)
    err = np.abs(gpu_row - ref_row)
    bad = err > bound_row
    assert not bad.any(), (f"{int(bad.sum())} scores outside the fp32 bound, worst key "
                           f"{int(np.argmax(err / bound_row))}")
    rel = float((err / np.maximum(ref_row, 1e-300)).max())
    return rel, float((err / bound_row).max())


def selection_stats(gpu_idx, a_row, k):
    """Diagnostics of one group against the fp64 scores: the population of the
    tie band [tau' - eps, tau + eps] and the fraction of the GPU set the fp64
    top-k shares."""
    a_row = np.asarray(a_row, np.float64)
    srt = np.sort(a_row)[::-1]
    tau = srt[k - 1]
    tau_next = srt[k] if k < len(a_row) else -np.inf
    band = int(((a_row >= tau_next - EPS_SEL) & (a_row <= tau + EPS_SEL)).sum())
    ref = orc.topk_select(a_row[None], k)[0]
    agree = np.intersect1d(np.asarray(gpu_idx), ref).size / k
    return band, agree


def check_block_selection(gpu_blocks, scores_row, n_b):
    """Compare one group's GPU block set with the oracle's block scores: equal
    outside a relative tie band, else every clearly better block present and no
    clearly worse one.  Returns 'strict' or 'band'."""
    gpu_blocks = np.asarray(gpu_blocks)
    scores_row = np.asarray(scores_row, np.float64)
    assert len(gpu_blocks) == n_b
    assert np.all(np.diff(gpu_blocks) > 0), "blocks not strictly ascending"
    eps = EPS_BLK * max(1e-30, float(np.abs(scores_row).max()))
    ref = orc.topk_select(scores_row[None], n_b)[0]
    srt = np.sort(scores_row)[::-1]
    tau = srt[n_b - 1]
    tau_next = srt[n_b] if n_b < len(scores_row) else -np.inf
    if tau - tau_next >= eps:
        assert np.array_equal(gpu_blocks, ref), "block selection differs outside the tie band"
        return "strict"
    must = np.nonzero(scores_row > tau + eps)[0]
    assert np.all(np.isin(must, gpu_blocks)), "a clearly selected block is missing"
    assert np.all(scores_row[gpu_blocks] >= tau_next - eps), "a clearly rejected block was selected"
    return "band"


def check_split_level(q_head, perm_prev, perm_gpu, C, G, level, power_iters=20):
    """Check the GPU's depth-`level` splits against the oracle's, given the
    GPU's partition before that depth.  Returns the number of band swaps."""
    q_head = np.asarray(q_head, np.float64)
    perm_prev = np.asarray(perm_prev, np.int64)
    perm_gpu = np.asarray(perm_gpu, np.int64)
    swaps = 0
    for s, m in orc.pddp_node_table(G, level):
        seg_prev = perm_prev[s * C:(s + m) * C]
        seg_gpu = perm_gpu[s * C:(s + m) * C]
        assert set(seg_prev.tolist()) == set(seg_gpu.tolist()), "node membership changed"
        if m < 2:
            assert np.array_equal(seg_prev, seg_gpu)
            continue
        idx = np.sort(seg_prev)
        mu, v = orc.pddp_node_direction(q_head[idx], power_iters)
        p = (q_head[idx] - mu) @ v
        order = np.lexsort((idx, p))
        n_left = (m // 2) * C
        ref_left = set(idx[order[:n_left]].tolist())
        gl = seg_gpu[:n_left]
        gr = seg_gpu[n_left:]
        assert np.all(np.diff(gl) > 0) and np.all(np.diff(gr) > 0), "children not ascending"
        got_left = set(gl.tolist())
        if got_left != ref_left:
            srt = p[order]
            boundary = 0.5 * (srt[n_left - 1] + srt[n_left])
            band = np.abs(p - boundary) <= EPS_PDDP * np.abs(p).max()
            band_tok = set(idx[band].tolist())
            diff = got_left.symmetric_difference(ref_left)
            assert diff <= band_tok, f"split differs outside the band ({len(diff - band_tok)} rows)"
            swaps += len(diff) // 2
    return swaps


def check_kmeans_step(x_head, perm_prev, labels_gpu, perm_gpu, C):
    """Check one GPU k-means iteration given the GPU's partition before it.
    Returns the number of tokens whose GPU label differs from the oracle's
    inside the rounding margin."""
    from oracle import kmeans as okm

    x = np.asarray(x_head, np.float64)
    lab = np.asarray(labels_gpu, np.int64)
    mu = okm.centroids(x, perm_prev, C)
    dist = okm.distances(x, mu)
    margin = EPS_KM * (2.0 * (np.abs(x) @ np.abs(mu).T) + (mu * mu).sum(axis=1)[None, :])
    rows = np.arange(x.shape[0])
    assert lab.min() >= 0 and lab.max() < mu.shape[0], "label out of range"
    lo = dist - margin
    hi = dist + margin
    # the GPU's choice may not be beaten by any centroid outside the margins
    assert np.all(lo[rows, lab] <= hi.min(axis=1)), "a GPU label is not a nearest centroid"
    best = okm.assign(x, mu)
    hi_best = hi[rows, best]
    lo_other = lo.copy()
    lo_other[rows, best] = np.inf
    unique = hi_best < lo_other.min(axis=1)
    assert np.array_equal(lab[unique], best[unique]), "an unambiguous label differs"
    assert np.array_equal(np.asarray(perm_gpu, np.int64), okm.balance(lab, C)), \
        "partition is not the balance of the labels"
    return int((lab != best).sum())
