"""Plain fp64 CPU oracle of the MC-Sparse attention hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import or run this module.  It shares no code with the HIP
library and imports nothing from it.

Sources (web pages about "MC-Sparse: Analyzing and Bridging the Dense-Sparse
Attention Gap in Diffusion Transformers"):
  [onedev]   onedev.kr paper summary (Korean), sections "what is different"
             (anchor/reuse formula), "how it is used" (components 1-3),
             "how it works" (oracle analysis).
  [aifeeds]  ai-feeds.com structured summary (Chinese), section "method"
             (key modules 1-4, output) and "integration interface".
  [n884]     n884.com article, sections "Key Takeaways" and "Development".

Every function works on one (batch, head) slice; inputs are the bf16 values the
GPU sees, upcast exactly to float64.  Where the pages leave a step open, the
reading taken is stated in the docstring (R-numbers refer to the readings
register of the project's design notes).

Parity status: every function here is pinned by tests against library routines,
closed forms, invariants or brute force (see tests/test_oracle_*.py).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "softmax_scale", "dense_attention", "pddp_node_direction", "pddp_split_level",
    "pddp_groups", "pddp_node_table", "group_scores", "topk_select",
    "sparse_attention", "residual", "reuse_step", "anchor_pipeline",
]


def softmax_scale(d: int) -> float:
    """Softmax scale 1/sqrt(d) in fp64 (the layer configs fix it; reading R7)."""
    return 1.0 / math.sqrt(d)


# ---------------------------------------------------------------------------
# O2  dense attention (anchor pass 1)
# ---------------------------------------------------------------------------
def dense_attention(q, k, v, n_valid, scale, block=256, rows=None):
    """Dense softmax attention and its log-sum-exp.

    [onedev] "what is different": at the anchor step dense attention is run and
    its output is the layer output; its softmax statistics feed the exact
    selection ("how it is used", component 3).

    s_ij = scale * q_i . k_j over keys j < n_valid (padded keys never take
    part); LSE_i = log sum_j exp(s_ij) (natural log); O_i = sum_j
    exp(s_ij - LSE_i) v_j.  Rows i >= n_valid (padding) get O = 0 and LSE = 0.
    Row blocks only bound memory; each row is computed on its own.  With
    `rows` (token indices), only those rows are computed and returned, in the
    order given.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)[:n_valid]
    v = np.asarray(v, np.float64)[:n_valid]
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    o = np.zeros((len(idx), v.shape[1]))
    lse = np.zeros(len(idx))
    live = np.nonzero(idx < n_valid)[0]
    for b0 in range(0, len(live), block):
        sel = live[b0:b0 + block]
        s = scale * (q[idx[sel]] @ k.T)
        m = s.max(axis=1, keepdims=True)
        l = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
        p = np.exp(s - l[:, None])
        o[sel] = p @ v
        lse[sel] = l
    return o, lse


# ---------------------------------------------------------------------------
# O3  Fast PDDP grouping
# ---------------------------------------------------------------------------
def pddp_node_table(groups, level):
    """Nodes (start_group, n_groups) present at tree depth `level`.

    [onedev] "how it is used", component 2: groups must have exactly the query
    tile size C, so every split is C-aligned.  Reading R11: a node of m groups
    splits into a left child of floor(m/2) groups and a right child of the rest;
    a node of one group is a leaf and is carried to the next level unchanged.
    """
    nodes = [(0, groups)]
    for _ in range(level):
        nxt = []
        for s, m in nodes:
            if m >= 2:
                h = m // 2
                nxt += [(s, h), (s + h, m - h)]
            else:
                nxt.append((s, m))
        nodes = nxt
    return nodes


def pddp_node_direction(x, power_iters=20):
    """Principal direction of a node's centred rows by power iteration.

    [onedev] "how it is used", component 2: project each node on its principal
    direction and split at the median; Fast PDDP computes the direction with
    batched power iteration.  Readings R9/R10: start from v0 = 1/sqrt(d) in every
    component, run exactly `power_iters` steps of
        w = sum_i ((x_i - mu) . v) (x_i - mu);  v = w / ||w||  (if ||w|| > 0),
    then flip v so that its largest-magnitude component is positive (lowest
    component index on ties).  Returns (mu, v).
    """
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=0)
    y = x - mu
    d = x.shape[1]
    v = np.full(d, 1.0 / math.sqrt(d))
    for _ in range(power_iters):
        t = y @ v                      # projections on the current direction
        w = y.T @ t                    # sum_i t_i (x_i - mu)
        nrm = math.sqrt(float(w @ w))
        if nrm > 0.0:
            v = w / nrm
    j = int(np.argmax(np.abs(v)))      # argmax returns the first (lowest) index on ties
    if v[j] < 0:
        v = -v
    return mu, v


def pddp_split_level(q, perm, C, groups, level, power_iters=20):
    """Apply the splits of tree depth `level` to a partition `perm`.

    `perm` lists the token indices of each node contiguously (node = groups
    [s, s+m) occupies perm[s*C:(s+m)*C]).  Each node with m >= 2 groups is
    projected on its principal direction; its members ordered by (p_i, i)
    ascending give the left child (the first floor(m/2)*C) and the right child
    (the rest).  Members inside each child are stored in ascending token order
    (reading R12).  Only the index array is carried between levels ([onedev]
    "how it is used", component 2).
    """
    q = np.asarray(q, np.float64)
    out = np.array(perm, dtype=np.int64, copy=True)
    for s, m in pddp_node_table(groups, level):
        if m < 2:
            continue
        idx = np.sort(out[s * C:(s + m) * C])
        mu, v = pddp_node_direction(q[idx], power_iters)
        p = (q[idx] - mu) @ v
        p = np.where(p == 0.0, 0.0, p)          # -0.0 and +0.0 are the same value
        order = np.lexsort((idx, p))            # by p, then by token index
        n_left = (m // 2) * C
        left = np.sort(idx[order[:n_left]])
        right = np.sort(idx[order[n_left:]])
        out[s * C:(s + m) * C] = np.concatenate([left, right])
    return out


def pddp_groups(q, C, power_iters=20, levels=None):
    """Fast PDDP grouping of one head's queries into tile-aligned groups.

    All N_pad rows take part (padded rows are ordinary all-zero rows, reading
    R8).  Runs `levels` tree depths (default ceil(log2 G), i.e. until every node
    holds one group).  Leaves are numbered left to right: group g is
    perm[g*C:(g+1)*C], members ascending (R12).
    """
    n_pad = q.shape[0]
    assert n_pad % C == 0
    G = n_pad // C
    L = 0
    while (1 << L) < G:
        L += 1
    if levels is None:
        levels = L
    perm = np.arange(n_pad, dtype=np.int64)
    for lv in range(levels):
        perm = pddp_split_level(q, perm, C, G, lv, power_iters)
    return perm


# ---------------------------------------------------------------------------
# O4/O5  exact-probability group scores and per-group top-k
# ---------------------------------------------------------------------------
def group_scores(q, k, perm, lse, n_valid, C, scale, groups=None):
    """Aggregated exact attention probability of every key for each group.

    [onedev] "what is different": KV tokens are selected with the exact (dense)
    attention probabilities; "how it is used", component 3: a second pass
    recomputes the logits because the dense kernel does not expose them.
    Reading R1: one KV set per query group; R2: the group's score of key j is
    the sum over its valid members i (< n_valid) of exp(s_ij - LSE_i).
    Returns a [len(groups), n_valid] array.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)[:n_valid]
    G = q.shape[0] // C
    gl = range(G) if groups is None else groups
    a = np.zeros((len(gl), n_valid))
    for r, g in enumerate(gl):
        mem = np.asarray(perm[g * C:(g + 1) * C])
        mem = mem[mem < n_valid]
        if mem.size == 0:
            continue
        s = scale * (q[mem] @ k.T)
        a[r] = np.exp(s - np.asarray(lse)[mem][:, None]).sum(axis=0)
    return a


def topk_select(a, topk):
    """The `topk` keys with the largest group score, in ascending key order.

    [onedev] "how it is used", component 1: selection is per individual KV
    token, across block boundaries.  Reading R4: a higher score wins; equal
    scores go to the lower key index; the selected set is stored ascending.
    """
    a = np.asarray(a, np.float64)
    out = np.empty((a.shape[0], topk), dtype=np.int64)
    for r in range(a.shape[0]):
        j = np.arange(a.shape[1])
        order = np.lexsort((j, -a[r]))          # by -a, then by key index
        out[r] = np.sort(order[:topk])
    return out


# ---------------------------------------------------------------------------
# O6/O7/O8  sparse attention, residual, reuse step
# ---------------------------------------------------------------------------
def sparse_attention(q, k, v, perm, kv_idx, n_valid, C, scale, groups=None):
    """Token-sparse attention of each query group over its own KV index set.

    [onedev] "how it is used", component 1: the kernel gathers keys and values
    by index; "what is different": SparseAttn(Q, K, V; G, S).  Reading R6: the
    softmax is renormalised over the selected set S_g only.  Rows of padded
    tokens (>= n_valid) are 0.  Returns [N_pad, d] in token order (only rows of
    the requested groups are filled when `groups` is given).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n_pad = q.shape[0]
    G = n_pad // C
    o = np.zeros((n_pad, v.shape[1]))
    gl = range(G) if groups is None else groups
    for r, g in enumerate(gl):
        mem = np.asarray(perm[g * C:(g + 1) * C])
        sel = np.asarray(kv_idx[g] if groups is None else kv_idx[r])
        s = scale * (q[mem] @ k[sel].T)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        o[mem] = p @ v[sel]
    o[n_valid:] = 0.0
    return o


def residual(o_full, o_sparse, n_valid):
    """R = O_full - O_sparse, recorded at the anchor ([onedev] "what is
    different"); padded rows are 0."""
    r = np.asarray(o_full, np.float64) - np.asarray(o_sparse, np.float64)
    r[n_valid:] = 0.0
    return r


def reuse_step(q, k, v, perm, kv_idx, r, n_valid, C, scale, groups=None):
    """One reuse step: O_t = SparseAttn(Q_t, K_t, V_t; G, S) + R.

    [onedev] "what is different" (the anchor/reuse formula); [aifeeds] "method",
    output: the sparse result plus the cached residual correction.  Reading
    R18: R is added unchanged.
    """
    o = sparse_attention(q, k, v, perm, kv_idx, n_valid, C, scale, groups)
    out = o + np.asarray(r, np.float64)
    if groups is not None:
        mask = np.zeros(q.shape[0], dtype=bool)
        for g in groups:
            mask[np.asarray(perm[g * C:(g + 1) * C])] = True
        out[~mask] = 0.0
    out[n_valid:] = 0.0
    return out


def anchor_pipeline(q, k, v, n_valid, C, topk, scale, power_iters=20):
    """Whole anchor step for one head: dense pass, grouping, exact selection,
    sparse pass and residual ([onedev] "what is different")."""
    o_full, lse = dense_attention(q, k, v, n_valid, scale)
    perm = pddp_groups(q, C, power_iters)
    a = group_scores(q, k, perm, lse, n_valid, C, scale)
    kv_idx = topk_select(a, topk)
    o_sparse = sparse_attention(q, k, v, perm, kv_idx, n_valid, C, scale)
    r = residual(o_full, o_sparse, n_valid)
    return dict(o_full=o_full, lse=lse, perm=perm, scores=a, kv_idx=kv_idx,
                o_sparse=o_sparse, r=r)
