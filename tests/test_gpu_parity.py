"""GPU parity: every C-ABI call against the fp64 oracle on the same bf16 inputs.

Stage-isolated: each oracle stage consumes the GPU's upstream outputs (perm,
kv_idx, O_full), so an allowed tie-band difference upstream cannot cascade.
Shapes span several 64-key tiles, ragged key tails (topk % 64 != 0), padded
tokens (n_valid < n_pad), both head sizes and both group sizes.
"""
import numpy as np
import pytest
import torch

import synthdata as sd
from oracle import mcs_oracle as orc
from tests import parity as par

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def mcs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_diffusion_attn_amd as m
    m.lib()
    return m


def f64(t):
    return par.bf16_to_f64(t)


def random_metadata(n_valid, n_pad, C, topk, heads, seed):
    rng = np.random.default_rng(seed)
    G = n_pad // C
    perm = np.stack([rng.permutation(n_pad) for _ in range(heads)]).astype(np.int32)
    kv = np.stack([np.stack([np.sort(rng.choice(n_valid, topk, replace=False)) for _ in range(G)])
                   for _ in range(heads)]).astype(np.int32)
    return perm[None], kv[None]


SHAPES = [  # (d, C, n_valid, n_pad, topk, heads)
    (64, 64, 1000, 1024, 300, 2),
    (128, 128, 500, 512, 77, 2),
    (128, 64, 700, 704, 129, 1),
    (64, 128, 1024, 1024, 1024, 1),
    (96, 128, 700, 768, 150, 2),
    (96, 64, 900, 960, 201, 1),
    (128, 128, 384, 384, 1, 1),
    (128, 128, 300, 384, 64, 1),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "d%d_C%d_n%d_%d_k%d_h%d" % s)
def test_sparse_attn_random_metadata(mcs, shape):
    d, C, nv, n_pad, topk, H = shape
    cfg = sd.custom(heads=H, n_valid=nv, head_dim=d, group_size=C, n_clusters=8, n_reuse=0)
    assert cfg.n_pad == n_pad
    q, k, v = sd.generate(cfg)[0]
    perm, kv = random_metadata(nv, n_pad, C, topk, H, seed=d + C + topk)
    rng = np.random.default_rng(1)
    r = torch.from_numpy(rng.standard_normal((1, H, n_pad, d)).astype(np.float32) * 0.1).to(torch.bfloat16)
    r[:, :, nv:] = 0
    qd, kd, vd, rd = (t.to(DEV) for t in (q, k, v, r))
    pd, kvd = torch.from_numpy(perm).to(DEV), torch.from_numpy(kv).to(DEV)
    sc = 1.0 / d ** 0.5
    o = mcs.sparse_attn(qd, kd, vd, pd, kvd, rd, nv, C, sc)
    o_nr = mcs.sparse_attn(qd, kd, vd, pd, kvd, None, nv, C, sc)
    torch.cuda.synchronize()
    for h in range(H):
        ref = orc.reuse_step(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), perm[0, h], kv[0, h],
                             f64(r[0, h]), nv, C, sc)
        got = f64(o[0, h])
        if topk == 1:
            # one key: the output is V[j] + R exactly, so the only error is the
            # final rounding to bf16 (half a bf16 ulp, at most 2^-8 relative)
            assert np.all(np.abs(got[:nv] - ref[:nv]) <= 2.0 ** -8 * np.abs(ref[:nv]))
        else:
            par.assert_close(got[:nv], ref[:nv], what=f"sparse+R head {h}")
        assert np.all(got[nv:] == 0)
        ref_nr = orc.sparse_attention(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), perm[0, h], kv[0, h], nv, C, sc)
        if topk == 1:
            assert np.array_equal(f64(o_nr[0, h])[:nv], ref_nr[:nv])  # V rows, exact
        else:
            par.assert_close(f64(o_nr[0, h])[:nv], ref_nr[:nv], what=f"sparse head {h}")


@pytest.mark.parametrize("shape", SHAPES[:6], ids=lambda s: "d%d_C%d_n%d_%d_k%d_h%d" % s)
def test_dense_attn(mcs, shape):
    d, C, nv, n_pad, topk, H = shape
    cfg = sd.custom(heads=H, n_valid=nv, head_dim=d, group_size=C, n_clusters=8, n_reuse=0)
    q, k, v = sd.generate(cfg)[0]
    sc = 1.0 / d ** 0.5
    o, lse = mcs.dense_attn(q.to(DEV), k.to(DEV), v.to(DEV), nv, C, sc)
    torch.cuda.synchronize()
    for h in range(H):
        ref_o, ref_l = orc.dense_attention(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), nv, sc)
        par.assert_close(f64(o[0, h])[:nv], ref_o[:nv], what="dense O")
        l = lse[0, h].double().cpu().numpy()
        assert np.abs(l[:nv] - ref_l[:nv]).max() < 1e-3
        assert np.all(l[nv:] == 0) and np.all(f64(o[0, h])[nv:] == 0)


def run_anchor(mcs, cfg, q, k, v, ws=None):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    perm = mcs.group(qd, cfg.n_valid, cfg.group_size, cfg.power_iters)
    o_full, lse, kv = mcs.anchor_select(qd, kd, vd, perm, cfg.n_valid, cfg.group_size, cfg.topk, cfg.scale,
                                        workspace=ws)
    r = mcs.residual(qd, kd, vd, perm, kv, o_full, cfg.n_valid, cfg.group_size, cfg.scale)
    torch.cuda.synchronize()
    return perm, o_full, lse, kv, r


def all_heads_ws(mcs, cfg, topk=None):
    dims = mcs.make_dims(cfg.batch, cfg.heads, cfg.n_valid, cfg.n_pad, cfg.head_dim, cfg.group_size)
    nbytes = mcs.anchor_select_workspace_bytes(dims, cfg.topk if topk is None else topk)
    return dims, torch.empty(nbytes, dtype=torch.uint8, device=DEV)


TINY_LIKE = [
    sd.CONFIGS["tiny"],
    sd.custom("ragged128", heads=2, n_valid=700, head_dim=128, group_size=128, density_pct=25, n_clusters=8),
    sd.custom("ragged64", heads=1, n_valid=900, head_dim=64, group_size=128, density_pct=15, n_clusters=12),
    sd.custom("c64d128", heads=1, n_valid=1500, head_dim=128, group_size=64, density_pct=20, n_clusters=10),
    sd.custom("d96", heads=2, n_valid=1000, head_dim=96, group_size=128, density_pct=20, n_clusters=10),
    sd.custom("d96c64", heads=1, n_valid=1300, head_dim=96, group_size=64, density_pct=25, n_clusters=12),
]


@pytest.mark.parametrize("cfg", TINY_LIKE, ids=lambda c: c.name)
def test_anchor_and_reuse_pipeline(mcs, cfg):
    steps = sd.generate(cfg)
    q, k, v = steps[0]
    dims, ws = all_heads_ws(mcs, cfg)
    perm, o_full, lse, kv, r = run_anchor(mcs, cfg, q, k, v, ws)
    nv, C, sc, G = cfg.n_valid, cfg.group_size, cfg.scale, cfg.groups
    perm_h, kv_h = perm.cpu().numpy(), kv.cpu().numpy()
    gpu_scores = mcs.anchor_scores(ws, dims).cpu().numpy()
    rules = {"strict": 0, "band": 0}
    for h in range(cfg.heads):
        qh, kh, vh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h])
        # grouping: a valid partition into groups of C, ascending members
        p = perm_h[0, h]
        assert sorted(p.tolist()) == list(range(cfg.n_pad))
        for g in range(G):
            assert np.all(np.diff(p[g * C:(g + 1) * C]) > 0)
        # pass 1
        ref_o, ref_l = orc.dense_attention(qh, kh, vh, nv, sc)
        par.assert_close(f64(o_full[0, h])[:nv], ref_o[:nv], what="O_full")
        assert np.abs(lse[0, h].double().cpu().numpy()[:nv] - ref_l[:nv]).max() < 1e-3
        # pass 2 + top-k, with the GPU's groups: the GPU's fp32 scores within
        # their error bound of the oracle's (with the GPU's lse), the index
        # sets bit-exact against the top-k of those scores, and within the
        # tie-band rule against the fp64 oracle's own scores
        a = orc.group_scores(qh, kh, p, ref_l, nv, C, sc)
        lse_gpu = lse[0, h].double().cpu().numpy()
        a_gl = orc.group_scores(qh, kh, p, lse_gpu, nv, C, sc)
        bh = h  # batch 1
        for g in range(G):
            mem = p[g * C:(g + 1) * C]
            mem = mem[mem < nv]
            par.check_scores(gpu_scores[bh, g], a_gl[g], par.score_error_bound(qh[mem], kh, lse_gpu[mem], sc, nv))
            par.check_selection_exact(kv_h[0, h, g], gpu_scores[bh, g], cfg.topk)
            rules[par.check_selection(kv_h[0, h, g], a[g], cfg.topk)] += 1
        # residual, isolated: the GPU's O_full as input
        o_sp = orc.sparse_attention(qh, kh, vh, p, kv_h[0, h], nv, C, sc)
        par.assert_close(f64(r[0, h])[:nv], (f64(o_full[0, h]) - o_sp)[:nv], what="R")
        # anchor identity: the oracle's O_full minus its sparse output
        par.assert_close(f64(r[0, h])[:nv], (ref_o - o_sp)[:nv], what="R vs oracle O_full")
        assert np.all(f64(r[0, h])[nv:] == 0)
    # reuse steps
    for qt, kt, vt in steps[1:]:
        o = mcs.sparse_attn(qt.to(DEV), kt.to(DEV), vt.to(DEV), perm, kv, r, nv, C, sc)
        torch.cuda.synchronize()
        for h in range(cfg.heads):
            ref = orc.reuse_step(f64(qt[0, h]), f64(kt[0, h]), f64(vt[0, h]), perm_h[0, h], kv_h[0, h],
                                 f64(r[0, h]), nv, C, sc)
            par.assert_close(f64(o[0, h])[:nv], ref[:nv], what="reuse O")
    print(f"{cfg.name}: selection rules {rules}")


@pytest.mark.parametrize("cfg", TINY_LIKE, ids=lambda c: c.name)
def test_group_level_by_level(mcs, cfg):
    q = sd.generate(cfg, steps=1)[0][0]
    qd = q.to(DEV)
    L = cfg.levels
    perms = [np.tile(np.arange(cfg.n_pad), (cfg.heads, 1))]
    for lv in range(1, L + 1):
        perms.append(mcs.group(qd, cfg.n_valid, cfg.group_size, cfg.power_iters, max_levels=lv)[0].cpu().numpy())
    full = mcs.group(qd, cfg.n_valid, cfg.group_size, cfg.power_iters)[0].cpu().numpy()
    assert np.array_equal(full, perms[L])
    swaps = 0
    for h in range(cfg.heads):
        for lv in range(L):
            swaps += par.check_split_level(f64(q[0, h]), perms[lv][h], perms[lv + 1][h], cfg.group_size,
                                           cfg.groups, lv, cfg.power_iters)
    print(f"{cfg.name}: {swaps} band swaps")


@pytest.mark.parametrize("iters", [0, 1, 3])
@pytest.mark.parametrize("d", [64, 96, 128])
def test_group_few_power_iterations(mcs, d, iters):
    """Grouping with 0 (projections on v0 = 1/sqrt(d), node means from the
    row-sum pass), 1 and 3 power iterations, level by level against the
    oracle's splits with the same iteration count."""
    cfg = sd.custom(f"it{iters}d{d}", heads=2, n_valid=900, head_dim=d, group_size=64, n_clusters=7)
    q = sd.generate(cfg, steps=1)[0][0]
    qd = q.to(DEV)
    L = cfg.levels
    perms = [np.tile(np.arange(cfg.n_pad), (cfg.heads, 1))]
    for lv in range(1, L + 1):
        perms.append(mcs.group(qd, cfg.n_valid, cfg.group_size, iters, max_levels=lv)[0].cpu().numpy())
    swaps = 0
    for h in range(cfg.heads):
        for lv in range(L):
            swaps += par.check_split_level(f64(q[0, h]), perms[lv][h], perms[lv + 1][h], cfg.group_size,
                                           cfg.groups, lv, iters)
    print(f"{iters} iterations, d {d}: {swaps} band swaps")


def test_determinism(mcs):
    cfg = TINY_LIKE[1]
    q, k, v = sd.generate(cfg, steps=1)[0]
    a = run_anchor(mcs, cfg, q, k, v)
    b = run_anchor(mcs, cfg, q, k, v)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o1 = mcs.sparse_attn(qd, kd, vd, a[0], a[3], a[4], cfg.n_valid, cfg.group_size, cfg.scale)
    o2 = mcs.sparse_attn(qd, kd, vd, a[0], a[3], a[4], cfg.n_valid, cfg.group_size, cfg.scale)
    assert torch.equal(o1, o2)


def test_small_workspace_head_chunks(mcs):
    cfg = sd.custom("chunks", heads=3, n_valid=640, head_dim=64, group_size=64, density_pct=25, n_clusters=8)
    q, k, v = sd.generate(cfg, steps=1)[0]
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    perm = mcs.group(qd, cfg.n_valid, cfg.group_size)
    dims = mcs.make_dims(1, 3, cfg.n_valid, cfg.n_pad, 64, 64)
    small = torch.empty(mcs.anchor_select_workspace_bytes(dims, cfg.topk, minimum=True), dtype=torch.uint8, device=DEV)
    o1, l1, kv1 = mcs.anchor_select(qd, kd, vd, perm, cfg.n_valid, 64, cfg.topk, cfg.scale)
    o2, l2, kv2 = mcs.anchor_select(qd, kd, vd, perm, cfg.n_valid, 64, cfg.topk, cfg.scale, workspace=small)
    torch.cuda.synchronize()
    assert torch.equal(kv1, kv2) and torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d,C,topk", [(64, 64, 2501), (128, 128, 2403)])
def test_topk_planted_ties_long_rows(mcs, d, C, topk):
    """Rows of 10000 keys (the top-k's histogram passes take their eight-loads-
    in-flight loop twice, then the tail) in which every key row occurs four
    times, so every score is tied four ways and the k-th score's tie run is
    split (topk = 4m + 1 or 4m + 3): the selection must be exactly the top-k of
    the GPU's own scores, ties to the lower key index."""
    nv = 10000
    cfg = sd.custom("ties", heads=1, n_valid=nv, head_dim=d, group_size=C, density_pct=25, n_clusters=8)
    q, k, v = sd.generate(cfg, steps=1)[0]
    base = nv // 4
    k[0, 0, base:nv] = k[0, 0, :base].repeat(3, 1)
    dims, ws = all_heads_ws(mcs, cfg, topk)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    perm = mcs.group(qd, nv, C, cfg.power_iters)
    o_full, lse, kv = mcs.anchor_select(qd, kd, vd, perm, nv, C, topk, cfg.scale, workspace=ws)
    torch.cuda.synchronize()
    sc_gpu = mcs.anchor_scores(ws, dims)[0].cpu().numpy()
    kvh, p = kv[0, 0].cpu().numpy(), perm[0, 0].cpu().numpy()
    # identical key rows got bitwise identical scores
    j = np.arange(nv)
    assert np.array_equal(sc_gpu[:, j], sc_gpu[:, j % base])
    split = 0
    qh, kh = f64(q[0, 0]), f64(k[0, 0])
    lse_gpu = lse[0, 0].double().cpu().numpy()
    for g in range(cfg.groups):
        row = sc_gpu[g]
        par.check_selection_exact(kvh[g], row, topk)
        tau = np.sort(row)[::-1][topk - 1]
        n_eq, n_sel = int((row == tau).sum()), int((row[kvh[g]] == tau).sum())
        assert n_eq >= 4 and 0 < n_sel <= n_eq
        split += n_sel < n_eq
    assert split > cfg.groups // 2, "the k-th score's tie run was rarely split"
    # the scores themselves, on a few groups
    for g in (0, cfg.groups // 2, cfg.groups - 1):
        mem = p[g * C:(g + 1) * C]
        mem = mem[mem < nv]
        a_gl = orc.group_scores(qh, kh, p, lse_gpu, nv, C, cfg.scale, groups=[g])[0]
        par.check_scores(sc_gpu[g], a_gl, par.score_error_bound(qh[mem], kh, lse_gpu[mem], cfg.scale, nv))
    print(f"ties d{d} C{C} k{topk}: tie run split at the k-th score in {split} of {cfg.groups} groups")
