"""Strided inputs and outputs (the `_strided` calls of the C ABI).

A DiT block produces Q, K and V as [batch, tokens, heads, head_dim] (BNHD),
often as slices of one fused QKV projection [B, N, 3, H, d].  The strided
calls read those views in place and write the layer output in the caller's
layout.  The arithmetic does not depend on where a row lives, so every output
must be bitwise equal to the contiguous path on contiguous copies of the same
values (the contiguous path is itself checked against the fp64 oracle in the
parity tests); one case is also checked against the oracle directly.
"""
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


def bnhd_view(x):
    """x [B,H,N,d] contiguous -> the same values as a [B,H,N,d] view of a
    contiguous [B,N,H,d] tensor."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


def fused_views(q, k, v):
    """q, k, v [B,H,N,d] -> views into one [B,N,3,H,d] tensor."""
    qkv = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous()
    return tuple(qkv[:, :, i].transpose(1, 2) for i in range(3))


def run_path(mcs, cfg, q, k, v, o_like=None):
    C, nv, tk, sc = cfg.group_size, cfg.n_valid, cfg.topk, cfg.scale
    perm = mcs.group(q, nv, C, cfg.power_iters)
    o_full = None if o_like is None else torch.empty_like(o_like)
    o_full, lse, kv = mcs.anchor_select(q, k, v, perm, nv, C, tk, sc, o_full=o_full)
    r = mcs.residual(q, k, v, perm, kv, o_full, nv, C, sc)
    o = None if o_like is None else torch.empty_like(o_like)
    o = mcs.sparse_attn(q, k, v, perm, kv, r, nv, C, sc, o=o)
    od = None if o_like is None else torch.empty_like(o_like)
    od, _ = mcs.dense_attn(q, k, v, nv, C, sc, o=od, want_lse=False)
    torch.cuda.synchronize()
    return dict(perm=perm, o_full=o_full, lse=lse, kv=kv, r=r, o=o, dense=od)


CASES = [
    sd.custom("bnhd-d128", batch=2, heads=3, n_valid=700, head_dim=128, group_size=128,
              density_pct=20, n_clusters=8),
    sd.custom("bnhd-d64", batch=1, heads=4, n_valid=1000, head_dim=64, group_size=64,
              density_pct=15, n_clusters=10, seed=3),
    sd.custom("bnhd-mixed", batch=2, heads=2, n_valid=640, head_dim=64, group_size=128,
              density_pct=30, n_clusters=5, seed=5),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("layout", ["bnhd", "fused_qkv"])
def test_strided_path_is_bitwise_the_contiguous_path(mcs, cfg, layout):
    print(f"strided {layout} {cfg}", flush=True)
    q, k, v = (t.to(DEV) for t in sd.generate(cfg, steps=1)[0])
    ref = run_path(mcs, cfg, q, k, v)
    if layout == "bnhd":
        qs, ks, vs = bnhd_view(q), bnhd_view(k), bnhd_view(v)
        o_like = qs                     # outputs in the same BNHD layout
    else:
        qs, ks, vs = fused_views(q, k, v)
        o_like = bnhd_view(q)           # outputs as a separate BNHD tensor
    assert not qs.is_contiguous() or cfg.heads == 1
    got = run_path(mcs, cfg, qs, ks, vs, o_like=o_like)
    for name in ("o_full", "o", "dense"):
        assert got[name].stride() == o_like.stride(), name
    assert got["r"].is_contiguous()
    for name, want in ref.items():
        assert torch.equal(got[name].contiguous(), want), name


def test_strided_sparse_output_matches_oracle(mcs):
    """One strided reuse step against the fp64 oracle, on the selection the
    GPU made (parity of the selection itself is covered elsewhere)."""
    cfg = CASES[0]
    steps = [tuple(t.to(DEV) for t in s) for s in sd.generate(cfg, steps=2)]
    (q0, k0, v0), (q1, k1, v1) = steps
    C, nv, tk, sc = cfg.group_size, cfg.n_valid, cfg.topk, cfg.scale
    qs, ks, vs = fused_views(q0, k0, v0)
    perm = mcs.group(qs, nv, C, cfg.power_iters)
    o_full, lse, kv = mcs.anchor_select(qs, ks, vs, perm, nv, C, tk, sc)
    r = mcs.residual(qs, ks, vs, perm, kv, o_full, nv, C, sc)
    q1s, k1s, v1s = fused_views(q1, k1, v1)
    o = mcs.sparse_attn(q1s, k1s, v1s, perm, kv, r, nv, C, sc, o=torch.empty_like(bnhd_view(q1)))
    torch.cuda.synchronize()
    f64 = par.bf16_to_f64
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            want = orc.reuse_step(f64(q1[b, h].cpu()), f64(k1[b, h].cpu()), f64(v1[b, h].cpu()),
                                  perm[b, h].cpu().numpy(), kv[b, h].cpu().numpy(),
                                  f64(r[b, h].cpu()), nv, C, sc)
            par.assert_close(f64(o[b, h].cpu())[:nv], want[:nv], what=f"strided reuse b{b} h{h}")
