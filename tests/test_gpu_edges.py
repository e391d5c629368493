"""GPU edge cases of the C-ABI calls against the fp64 oracle: full density,
a single valid token, batch > 1, a single selected key, a non-default softmax
scale and padded tokens spread over several groups."""
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


f64 = par.bf16_to_f64


def test_full_density_selects_everything_and_matches_dense(mcs):
    cfg = sd.custom("full", heads=2, n_valid=500, head_dim=128, group_size=128, density_pct=100, n_clusters=6)
    assert cfg.topk == cfg.n_valid
    q, k, v = (t.to(DEV) for t in sd.generate(cfg, steps=1)[0])
    perm = mcs.group(q, cfg.n_valid, cfg.group_size)
    o_full, lse, kv = mcs.anchor_select(q, k, v, perm, cfg.n_valid, cfg.group_size, cfg.topk, cfg.scale)
    r = mcs.residual(q, k, v, perm, kv, o_full, cfg.n_valid, cfg.group_size, cfg.scale)
    o = mcs.sparse_attn(q, k, v, perm, kv, None, cfg.n_valid, cfg.group_size, cfg.scale)
    torch.cuda.synchronize()
    want = torch.arange(cfg.n_valid, device=DEV, dtype=torch.int32)
    assert torch.equal(kv, want.expand_as(kv))
    for h in range(cfg.heads):
        ref, _ = orc.dense_attention(f64(q[0, h].cpu()), f64(k[0, h].cpu()), f64(v[0, h].cpu()),
                                     cfg.n_valid, cfg.scale)
        par.assert_close(f64(o[0, h].cpu())[:cfg.n_valid], ref[:cfg.n_valid], what="full-density sparse")
        # R = O_full - O_sparse is only rounding noise at full density
        assert float(r[0, h].abs().max()) < 2e-2


def test_single_valid_token(mcs):
    cfg = sd.custom("one", heads=1, n_valid=1, head_dim=64, group_size=64, density_pct=100, n_clusters=1)
    q, k, v = (t.to(DEV) for t in sd.generate(cfg, steps=1)[0])
    perm = mcs.group(q, 1, 64)
    o_full, lse, kv = mcs.anchor_select(q, k, v, perm, 1, 64, 1, cfg.scale)
    o = mcs.sparse_attn(q, k, v, perm, kv, None, 1, 64, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(kv, torch.zeros_like(kv))
    assert torch.equal(o_full[0, 0, 0], v[0, 0, 0]) and torch.equal(o[0, 0, 0], v[0, 0, 0])
    assert bool((o_full[0, 0, 1:] == 0).all()) and bool((o[0, 0, 1:] == 0).all())
    assert float(lse[0, 0, 0]) == pytest.approx(float(q[0, 0, 0].float() @ k[0, 0, 0].float()) * cfg.scale, abs=1e-3)


def test_batch_of_two(mcs):
    cfg = sd.LayerConfig("b2", 2, 2, 700, 128, 128, 20, 8, 0.3, 1, 0.05)
    (q, k, v), (qt, kt, vt) = sd.generate(cfg)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    nv, C, sc = cfg.n_valid, cfg.group_size, cfg.scale
    perm = mcs.group(qd, nv, C)
    o_full, lse, kv = mcs.anchor_select(qd, kd, vd, perm, nv, C, cfg.topk, sc)
    r = mcs.residual(qd, kd, vd, perm, kv, o_full, nv, C, sc)
    o = mcs.sparse_attn(qt.to(DEV), kt.to(DEV), vt.to(DEV), perm, kv, r, nv, C, sc)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(2):
            qh, kh, vh = f64(q[b, h]), f64(k[b, h]), f64(v[b, h])
            p, kvh = perm[b, h].cpu().numpy(), kv[b, h].cpu().numpy()
            ref_o, ref_l = orc.dense_attention(qh, kh, vh, nv, sc)
            par.assert_close(f64(o_full[b, h].cpu())[:nv], ref_o[:nv], what=f"O_full b{b} h{h}")
            a = orc.group_scores(qh, kh, p, ref_l, nv, C, sc)
            for g in range(cfg.groups):
                par.check_selection(kvh[g], a[g], cfg.topk)
            ref = orc.reuse_step(f64(qt[b, h]), f64(kt[b, h]), f64(vt[b, h]), p, kvh, f64(r[b, h].cpu()), nv, C, sc)
            par.assert_close(f64(o[b, h].cpu())[:nv], ref[:nv], what=f"reuse b{b} h{h}")


def test_nondefault_scale(mcs):
    cfg = sd.custom("scale", heads=1, n_valid=640, head_dim=64, group_size=64, n_clusters=5)
    q, k, v = sd.generate(cfg, steps=1)[0]
    for sc in (0.02, 0.4):
        o, lse = mcs.dense_attn(q.to(DEV), k.to(DEV), v.to(DEV), 640, 64, sc)
        torch.cuda.synchronize()
        ref_o, ref_l = orc.dense_attention(f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0]), 640, sc)
        par.assert_close(f64(o[0, 0].cpu()), ref_o, what=f"dense scale {sc}")
        assert np.abs(lse[0, 0].double().cpu().numpy() - ref_l).max() < 1e-3


def test_padded_tokens_in_three_groups(mcs):
    # n_valid = 130 with C = 64: 62 padded (all-zero) tokens among three groups
    cfg = sd.custom("padgroups", heads=1, n_valid=130, head_dim=128, group_size=64, density_pct=50, n_clusters=3)
    assert cfg.n_pad == 192
    q, k, v = (t.to(DEV) for t in sd.generate(cfg, steps=1)[0])
    nv, C, sc = cfg.n_valid, cfg.group_size, cfg.scale
    perm = mcs.group(q, nv, C)
    o_full, lse, kv = mcs.anchor_select(q, k, v, perm, nv, C, cfg.topk, sc)
    r = mcs.residual(q, k, v, perm, kv, o_full, nv, C, sc)
    o = mcs.sparse_attn(q, k, v, perm, kv, r, nv, C, sc)
    torch.cuda.synchronize()
    p = perm[0, 0].cpu().numpy()
    kvh = kv[0, 0].cpu().numpy()
    assert kvh.max() < nv
    for g in range(cfg.groups):
        assert np.all(np.diff(kvh[g]) > 0)
    assert bool((o[0, 0, nv:] == 0).all()) and bool((r[0, 0, nv:] == 0).all())
    ref = orc.reuse_step(f64(q[0, 0].cpu()), f64(k[0, 0].cpu()), f64(v[0, 0].cpu()), p, kvh, f64(r[0, 0].cpu()),
                         nv, C, sc)
    par.assert_close(f64(o[0, 0].cpu())[:nv], ref[:nv], what="padding groups")
