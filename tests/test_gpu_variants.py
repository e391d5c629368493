"""GPU parity of the oracle-analysis selection variants (onedev.kr summary,
"how it works") against the fp64 oracle: block oracle and mean-pooled vanilla
BSA block selection (mcs_block_select), their token expansion, and attention,
residual and reuse over index rows with per-group counts
(mcs_sparse_attn_counts, mcs_residual_counts)."""
import numpy as np
import pytest
import torch

import synthdata as sd
from oracle import mcs_oracle as orc
from oracle import variants as var
from tests import parity as par

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
f64 = par.bf16_to_f64

# (name, heads, n_valid, n_pad, d, C, block, nblocks)
CASES = [
    ("d128_C64_b64", 2, 500, 512, 128, 64, 64, 2),
    ("d64_C128_b32", 1, 1000, 1024, 64, 128, 32, 8),
    ("d128_C128_b48_tail", 1, 700, 768, 128, 128, 48, 4),
]


@pytest.fixture(scope="module")
def mcs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_diffusion_attn_amd as m
    m.lib()
    return m


def make(case, steps=2):
    name, H, nv, n_pad, d, C, B, nb = case
    cfg = sd.custom(name, heads=H, n_valid=nv, head_dim=d, group_size=C, n_clusters=8)
    assert cfg.n_pad == n_pad
    return cfg, sd.generate(cfg, steps=steps)


def gpu_blocks(kv_row, count, B):
    toks = kv_row[:count]
    return np.unique(toks // B)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("mode", ["exact", "meanpool"])
def test_block_select(mcs, case, mode):
    cfg, steps = make(case, steps=1)
    _, H, nv, n_pad, d, C, B, nb = case
    q, k, v = steps[0]
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    perm = mcs.identity_perm(1, H, n_pad, DEV)
    sc = cfg.scale
    _, lse = mcs.dense_attn(qd, kd, vd, nv, C, sc)
    m = mcs.BLOCK_EXACT if mode == "exact" else mcs.BLOCK_MEANPOOL
    kv, cnt = mcs.block_select(qd, kd, perm, lse if mode == "exact" else None, m, B, nb, nv, C, sc)
    torch.cuda.synchronize()
    kv, cnt = kv.cpu().numpy(), cnt.cpu().numpy()
    rules = {"strict": 0, "band": 0}
    for h in range(H):
        qh, kh, vh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h])
        pid = var.identity_perm(n_pad)
        if mode == "exact":
            _, lse_ref = orc.dense_attention(qh, kh, vh, nv, sc)
            scores = var.block_oracle_scores(orc.group_scores(qh, kh, pid, lse_ref, nv, C, sc), nv, B)
        else:
            scores = var.meanpool_scores(qh, kh, pid, nv, C, B, sc)
        for g in range(n_pad // C):
            blk = gpu_blocks(kv[0, h, g], cnt[0, h, g], B)
            rules[par.check_block_selection(blk, scores[g], nb)] += 1
            # expansion: the blocks' tokens, ascending, then -1
            want = np.concatenate(var.expand_blocks([blk], nv, B))
            assert cnt[0, h, g] == len(want)
            np.testing.assert_array_equal(kv[0, h, g, :len(want)], want)
            assert np.all(kv[0, h, g, len(want):] == -1)
    print(f"{case[0]} {mode}: {rules}")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_counts_attention_residual_and_reuse(mcs, case):
    """Anchor: block-oracle rows -> residual; reuse step on drifted inputs; both
    against the oracle on the GPU's own rows."""
    cfg, steps = make(case)
    _, H, nv, n_pad, d, C, B, nb = case
    (q, k, v), (qt, kt, vt) = steps
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    perm = mcs.identity_perm(1, H, n_pad, DEV)
    sc = cfg.scale
    o_full, lse = mcs.dense_attn(qd, kd, vd, nv, C, sc)
    kv, cnt = mcs.block_select(qd, kd, perm, lse, mcs.BLOCK_EXACT, B, nb, nv, C, sc)
    r = mcs.residual_counts(qd, kd, vd, perm, kv, cnt, o_full, nv, C, sc)
    o_nr = mcs.sparse_attn_counts(qt.to(DEV), kt.to(DEV), vt.to(DEV), perm, kv, cnt, None, nv, C, sc)
    o = mcs.sparse_attn_counts(qt.to(DEV), kt.to(DEV), vt.to(DEV), perm, kv, cnt, r, nv, C, sc)
    torch.cuda.synchronize()
    kvn, cntn = kv.cpu().numpy(), cnt.cpu().numpy()
    pid = var.identity_perm(n_pad)
    for h in range(H):
        sets = [kvn[0, h, g, :cntn[0, h, g]] for g in range(n_pad // C)]
        ofull_ref, _ = orc.dense_attention(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), nv, sc)
        osp = orc.sparse_attention(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), pid, sets, nv, C, sc)
        par.assert_close(f64(r[0, h].cpu())[:nv], (f64(o_full[0, h].cpu()) - osp)[:nv], what=f"R h{h}")
        ref_nr = orc.sparse_attention(f64(qt[0, h]), f64(kt[0, h]), f64(vt[0, h]), pid, sets, nv, C, sc)
        par.assert_close(f64(o_nr[0, h].cpu())[:nv], ref_nr[:nv], what=f"sparse counts h{h}")
        ref = orc.reuse_step(f64(qt[0, h]), f64(kt[0, h]), f64(vt[0, h]), pid, sets, f64(r[0, h].cpu()),
                             nv, C, sc)
        par.assert_close(f64(o[0, h].cpu())[:nv], ref[:nv], what=f"reuse counts h{h}")
        assert bool((o[0, h, nv:] == 0).all()) and bool((r[0, h, nv:] == 0).all())


def test_all_blocks_equal_dense(mcs):
    _, H, nv, n_pad, d, C, B, _ = CASES[0]
    cfg, steps = make(CASES[0], steps=1)
    qd, kd, vd = (t.to(DEV) for t in steps[0])
    perm = mcs.identity_perm(1, H, n_pad, DEV)
    nb_all = (nv + B - 1) // B
    o_d, lse = mcs.dense_attn(qd, kd, vd, nv, C, cfg.scale)
    for m in (mcs.BLOCK_EXACT, mcs.BLOCK_MEANPOOL):
        kv, cnt = mcs.block_select(qd, kd, perm, lse, m, B, nb_all, nv, C, cfg.scale)
        o = mcs.sparse_attn_counts(qd, kd, vd, perm, kv, cnt, None, nv, C, cfg.scale)
        torch.cuda.synchronize()
        assert bool((cnt == nv).all())
        assert float((o.float() - o_d.float())[:, :, :nv].abs().max()) < 2e-2


def test_unit_blocks_match_the_token_selection(mcs):
    """Exact blocks of one key are the token oracle: the same index sets as
    mcs_anchor_select on the same partition (outside ties)."""
    cfg = sd.custom("unit", heads=1, n_valid=480, head_dim=64, group_size=64, n_clusters=5)
    q, k, v = (t.to(DEV) for t in sd.generate(cfg, steps=1)[0])
    perm = mcs.identity_perm(1, 1, cfg.n_pad, DEV)
    topk = 96
    _, lse, kv_tok = mcs.anchor_select(q, k, v, perm, cfg.n_valid, 64, topk, cfg.scale)
    kv, cnt = mcs.block_select(q, k, perm, lse, mcs.BLOCK_EXACT, 1, topk, cfg.n_valid, 64, cfg.scale)
    torch.cuda.synchronize()
    assert bool((cnt == topk).all())
    same = (kv == kv_tok).all(dim=-1).float().mean().item()
    assert same == 1.0, f"{same:.3f} of the groups agree"


def test_counts_are_clamped(mcs):
    """A count above the row stride uses the whole row; a count below 1 uses
    one key (no out-of-row reads)."""
    cfg = sd.custom("clamp", heads=1, n_valid=256, head_dim=64, group_size=64)
    q, k, v = (t.to(DEV) for t in sd.generate(cfg, steps=1)[0])
    perm = mcs.identity_perm(1, 1, 256, DEV)
    G = 4
    kv = torch.arange(32, dtype=torch.int32, device=DEV).expand(1, 1, G, 32).contiguous()
    big = torch.full((1, 1, G), 1000, dtype=torch.int32, device=DEV)
    full = torch.full((1, 1, G), 32, dtype=torch.int32, device=DEV)
    zero = torch.zeros((1, 1, G), dtype=torch.int32, device=DEV)
    one = torch.ones((1, 1, G), dtype=torch.int32, device=DEV)
    a = mcs.sparse_attn_counts(q, k, v, perm, kv, big, None, 256, 64)
    b = mcs.sparse_attn_counts(q, k, v, perm, kv, full, None, 256, 64)
    c = mcs.sparse_attn_counts(q, k, v, perm, kv, zero, None, 256, 64)
    e = mcs.sparse_attn_counts(q, k, v, perm, kv, one, None, 256, 64)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, e)
    # one key: every valid row is that key's value row
    assert torch.equal(e[0, 0, :256], v[0, 0, 0].expand(256, -1))
