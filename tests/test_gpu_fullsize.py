"""GPU parity at the full layer sizes, in the launch configuration the bench
times (all heads, all groups in one launch per call).  The fp64 oracle checks
sampled outputs: heads {0, H-1}, and in each the first group, the last group
(which holds the padded tokens, if any) and six seeded random groups.  Grouping
is checked level by level on those heads; every head's perm is checked to be a
partition into ascending groups of C.

Selection is checked twice per sampled group: bit-exact on the same inputs
(kv_idx equals the oracle's top-k of the fp32 scores the GPU ranked, read back
from the anchor workspace, whose scores must match the oracle's within the
fp32 error bound of tests/parity.py), and against the fp64 oracle's own scores
under the tie-band rule.
"""
import functools

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


@functools.lru_cache(maxsize=8)
def layer_data(heads, n_valid, head_dim, group_size, n_clusters, sigma, drift, seed):
    cfg = sd.LayerConfig("x", 1, heads, n_valid, head_dim, group_size, 25, n_clusters, sigma, 1, drift, seed=seed)
    return sd.generate(cfg, steps=2)


def data_for(cfg):
    return layer_data(cfg.heads, cfg.n_valid, cfg.head_dim, cfg.group_size, cfg.n_clusters, cfg.sigma,
                      cfg.drift, cfg.seed)


FULL = ["480p", "3d", "wan720p", "hunyuan720p_15", "hunyuan720p_25", "480p_c64", "480p_d96"]
# the 480p layer with groups of 64 queries (the split-key-tile attention path)
EXTRA = {"480p_c64": sd.custom("480p_c64", heads=24, n_valid=32760, head_dim=128, group_size=64,
                               density_pct=25, n_clusters=64)}


def config(name):
    return EXTRA[name] if name in EXTRA else sd.CONFIGS[name]


@pytest.mark.parametrize("name", FULL)
def test_fullsize_pipeline_sampled(mcs, name):
    cfg = config(name)
    print(f"\n[{name}] H{cfg.heads} N{cfg.n_valid}->{cfg.n_pad} d{cfg.head_dim} C{cfg.group_size} k{cfg.topk}",
          flush=True)
    (q, k, v), (qt, kt, vt) = data_for(cfg)
    nv, C, sc, G, H = cfg.n_valid, cfg.group_size, cfg.scale, cfg.groups, cfg.heads
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    perm = mcs.group(qd, nv, C, cfg.power_iters)
    # an all-heads workspace keeps the fp32 scores the top-k ranked
    dims = mcs.make_dims(1, H, nv, cfg.n_pad, cfg.head_dim, C)
    ws = torch.empty(mcs.anchor_select_workspace_bytes(dims, cfg.topk), dtype=torch.uint8, device=DEV)
    o_full, lse, kv = mcs.anchor_select(qd, kd, vd, perm, nv, C, cfg.topk, sc, workspace=ws)
    r = mcs.residual(qd, kd, vd, perm, kv, o_full, nv, C, sc)
    del qd, kd, vd
    o = mcs.sparse_attn(qt.to(DEV), kt.to(DEV), vt.to(DEV), perm, kv, r, nv, C, sc)
    torch.cuda.synchronize()

    # every head: a partition of [0, n_pad) into ascending groups of C
    ps, _ = torch.sort(perm[0].long(), dim=1)
    assert torch.equal(ps, torch.arange(cfg.n_pad, device=DEV).expand(H, -1))
    pg = perm[0].view(H, G, C)
    assert bool((pg[:, :, 1:] > pg[:, :, :-1]).all())
    kvs = kv[0]
    assert bool((kvs[:, :, 1:] > kvs[:, :, :-1]).all()) and int(kvs.max()) < nv and int(kvs.min()) >= 0
    assert torch.isfinite(o.float()).all()

    groups = sd.sample_groups(cfg)
    rules = {"strict": 0, "band": 0}
    worst_rel, worst_frac = 0.0, 0.0
    perm_h_all, kv_h_all = perm.cpu().numpy(), kv.cpu().numpy()
    gpu_scores = mcs.anchor_scores(ws, dims)
    for h in (0, H - 1):
        f = par.bf16_to_f64
        qh, kh, vh = f(q[0, h]), f(k[0, h]), f(v[0, h])
        ph, kvh = perm_h_all[0, h], kv_h_all[0, h]
        rows = np.concatenate([ph[g * C:(g + 1) * C] for g in groups])
        ref_o, ref_l = orc.dense_attention(qh, kh, vh, nv, sc, rows=rows)
        par.assert_close(f(o_full[0, h])[rows], ref_o, rows=rows < nv, what=f"{name} O_full h{h}")
        lse_gpu = lse[0, h].double().cpu().numpy()
        assert np.abs(lse_gpu[rows] - ref_l)[rows < nv].max() < 1e-3
        lse_full = np.zeros(cfg.n_pad)
        lse_full[rows] = ref_l
        a = orc.group_scores(qh, kh, ph, lse_full, nv, C, sc, groups=groups)
        # the scores the GPU ranked, against the oracle's with the GPU's lse
        a_gl = orc.group_scores(qh, kh, ph, lse_gpu, nv, C, sc, groups=groups)
        for i, g in enumerate(groups):
            ga = gpu_scores[h, g].cpu().numpy()
            mem = ph[g * C:(g + 1) * C]
            mem = mem[mem < nv]
            bound = par.score_error_bound(qh[mem], kh, lse_gpu[mem], sc, nv)
            rel, frac = par.check_scores(ga, a_gl[i], bound)
            worst_rel, worst_frac = max(worst_rel, rel), max(worst_frac, frac)
            # index work bit-exact on the same inputs
            par.check_selection_exact(kvh[g], ga, cfg.topk)
            # and against the fp64 oracle's own scores (R5 rule)
            rule = par.check_selection(kvh[g], a[i], cfg.topk)
            rules[rule] += 1
            band, agree = par.selection_stats(kvh[g], a[i], cfg.topk)
            print(f"[{name}] h{h} g{g}: rule {rule}, tie band holds {band} keys, "
                  f"{agree:.5f} of the set shared with the fp64 top-k, scores max rel err {rel:.2e}",
                  flush=True)
        o_sp = orc.sparse_attention(qh, kh, vh, ph, kvh[groups], nv, C, sc, groups=groups)
        valid = rows < nv
        par.assert_close(f(r[0, h])[rows], (f(o_full[0, h]) - o_sp)[rows], rows=valid, what=f"{name} R h{h}")
        ref = orc.reuse_step(f(qt[0, h]), f(kt[0, h]), f(vt[0, h]), ph, kvh[groups], f(r[0, h]), nv, C, sc,
                             groups=groups)
        par.assert_close(f(o[0, h])[rows], ref[rows], rows=valid, what=f"{name} reuse O h{h}")
        assert np.all(f(o[0, h])[rows[~valid]] == 0)
    print(f"[{name}] selection rules on sampled groups: {rules}; kv_idx equal to the top-k of the GPU's "
          f"scores in all {sum(rules.values())}; scores max rel err {worst_rel:.2e}, "
          f"max err / bound {worst_frac:.3f}", flush=True)


@pytest.mark.parametrize("name", ["480p", "3d", "hunyuan720p_15", "480p_d96"])
def test_fullsize_group_levels(mcs, name):
    cfg = sd.CONFIGS[name]
    (q, _, _), _ = data_for(cfg)
    qd = q.to(DEV)
    H, L = cfg.heads, cfg.levels
    heads = (0, H - 1)
    perms = [np.tile(np.arange(cfg.n_pad), (len(heads), 1))]
    for lv in range(1, L + 1):
        p = mcs.group(qd, cfg.n_valid, cfg.group_size, cfg.power_iters, max_levels=lv)
        perms.append(p[0, list(heads)].cpu().numpy())
    swaps = 0
    for i, h in enumerate(heads):
        qh = par.bf16_to_f64(q[0, h])
        for lv in range(L):
            swaps += par.check_split_level(qh, perms[lv][i], perms[lv + 1][i], cfg.group_size, cfg.groups, lv,
                                           cfg.power_iters)
    print(f"[{name}] PDDP levels checked on heads {heads}: {swaps} band swaps", flush=True)
