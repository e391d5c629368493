"""Attention on logits with a large, rising range: the lazily raised running max.

The kernels keep a running row max that is raised only when a tile's max
exceeds it by more than 8 in log2 units; only then are O and the row sum
rescaled.  Clustered synthetic data hardly ever triggers that.  Here the keys
grow along one direction u, key j as (j/64)·u plus noise, so for a query near
+u each 64-key tile's max beats the last by 11 to 16 log2 units and every
tile rescales.  For a query near -u the first tile holds the max and no tile
rescales.  Even and odd rows alternate between the two, so the lanes of every
wavefront disagree on whether to raise.  Logits reach 140 to 190 in log2 units.
Dense attention (O and the log-sum-exp), the anchor's score pass and top-k,
the reuse step and the residual are checked against the fp64 oracle on the
same bf16 inputs.
"""
import numpy as np
import pytest
import torch

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


def rising_inputs(d, n_valid, n_pad, seed):
    rng = np.random.default_rng(seed)
    u = rng.choice([-1.0, 1.0], size=d)
    ramp = np.arange(n_pad) / 64.0
    k = ramp[:, None] * u[None, :] + 0.5 * rng.standard_normal((n_pad, d))
    sign = np.where(np.arange(n_pad) % 2 == 0, 1.0, -1.0)
    q = sign[:, None] * u[None, :] + 0.3 * rng.standard_normal((n_pad, d))
    v = rng.standard_normal((n_pad, d))
    out = []
    for x in (q, k, v):
        x[n_valid:] = 0.0
        out.append(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).reshape(1, 1, n_pad, d))
    return out


@pytest.mark.parametrize("d,C", [(128, 128), (64, 64)])
def test_rising_logits_dense_sparse_residual(mcs, d, C):
    n_valid, n_pad = 700, 768            # 11 key tiles, the last one ragged (60 keys)
    print(f"rising logits d{d} C{C}", flush=True)
    q, k, v = rising_inputs(d, n_valid, n_pad, seed=d + C)
    sc = 1.0 / np.sqrt(d)
    qf, kf, vf = (par.bf16_to_f64(t[0, 0]) for t in (q, k, v))
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))

    # dense: the online softmax runs over all 11 tiles in key order
    o, lse = mcs.dense_attn(qd, kd, vd, n_valid, C, sc)
    torch.cuda.synchronize()
    ref_o, ref_l = orc.dense_attention(qf, kf, vf, n_valid, sc)
    s_max = float(np.max(qf[:n_valid] @ kf[:n_valid].T)) * sc * np.log2(np.e)
    assert s_max > 120.0, "the inputs do not reach the intended logit range"
    par.assert_close(par.bf16_to_f64(o[0, 0].cpu())[:n_valid], ref_o[:n_valid], what="dense O")
    got_l = lse[0, 0].double().cpu().numpy()[:n_valid]
    assert np.abs(got_l - ref_l[:n_valid]).max() <= 1e-4 * np.abs(ref_l[:n_valid]).max()

    # reuse step and residual on random ascending index sets (ascending keys
    # keep the rising order inside the sparse tile sequence)
    rng = np.random.default_rng(7)
    G, topk = n_pad // C, 333
    perm = np.concatenate([rng.permutation(n_valid), np.arange(n_valid, n_pad)]).astype(np.int32)
    kv = np.stack([np.sort(rng.choice(n_valid, topk, replace=False)) for _ in range(G)]).astype(np.int32)
    r = torch.from_numpy(0.05 * rng.standard_normal((1, 1, n_pad, d)).astype(np.float32)).to(torch.bfloat16)
    r[:, :, n_valid:] = 0
    pd = torch.from_numpy(perm).reshape(1, 1, n_pad).to(DEV)
    kvd = torch.from_numpy(kv).reshape(1, 1, G, topk).to(DEV)
    os_ = mcs.sparse_attn(qd, kd, vd, pd, kvd, r.to(DEV), n_valid, C, sc)
    res = mcs.residual(qd, kd, vd, pd, kvd, o, n_valid, C, sc)
    torch.cuda.synchronize()
    ref_s = orc.reuse_step(qf, kf, vf, perm, kv, par.bf16_to_f64(r[0, 0]), n_valid, C, sc)
    par.assert_close(par.bf16_to_f64(os_[0, 0].cpu())[:n_valid], ref_s[:n_valid], what="reuse step")
    sparse_only = orc.sparse_attention(qf, kf, vf, perm, kv, n_valid, C, sc)
    ref_r = orc.residual(par.bf16_to_f64(o[0, 0].cpu()), sparse_only, n_valid)
    par.assert_close(par.bf16_to_f64(res[0, 0].cpu())[:n_valid], ref_r[:n_valid], what="residual")

    # anchor selection on the same groups: the score pass weighs every key by
    # exp(s - lse), which spans hundreds of binary orders of magnitude here
    _, lse_a, kv_a = mcs.anchor_select(qd, kd, vd, pd, n_valid, C, topk, sc)
    torch.cuda.synchronize()
    a = orc.group_scores(qf, kf, perm, ref_l, n_valid, C, sc)
    kv_h = kv_a[0, 0].cpu().numpy()
    for g in range(G):
        par.check_selection(kv_h[g], a[g], topk)
