"""Attention on logits of a large range: both softmax passes.

The attention kernel first runs with no offset at all (p = exp2 of the scaled
logit, no row max) and accepts that pass when every row's probability sum
stays in [2^-60, 2^64] and O is finite; otherwise the workgroup redoes the
group with a running row max that is raised only when a tile's max exceeds it
by more than 8 in log2 units.  Clustered synthetic data stays in the first
pass.  Here the keys grow along one direction u, key j as (slope·j/64)·u plus
noise, so for a query near +u each 64-key tile's max beats the last by a fixed
step; for a query near -u the first tile holds the max; even and odd rows
alternate between the two.
- "rising" (slope 1): steps of 11 to 16 log2 units, logits reach 140 to 190,
  the first pass overflows its range and the redo raises the running max on
  every tile.
- "gentle" (slope 1/4): steps of 3 to 4 units, logits stay below about 50, and
  the first pass is accepted with probabilities up to about 2^48.
- "negative": every logit below -80 in log2 units, so the first pass
  underflows its range and the redo takes over from below.
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


def rising_inputs(d, n_valid, n_pad, seed, slope=1.0):
    rng = np.random.default_rng(seed)
    u = rng.choice([-1.0, 1.0], size=d)
    ramp = slope * np.arange(n_pad) / 64.0
    k = ramp[:, None] * u[None, :] + 0.5 * rng.standard_normal((n_pad, d))
    sign = np.where(np.arange(n_pad) % 2 == 0, 1.0, -1.0)
    q = sign[:, None] * u[None, :] + 0.3 * rng.standard_normal((n_pad, d))
    v = rng.standard_normal((n_pad, d))
    out = []
    for x in (q, k, v):
        x[n_valid:] = 0.0
        out.append(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).reshape(1, 1, n_pad, d))
    return out


def negative_inputs(d, n_valid, n_pad, seed):
    """Every logit far below -60 in log2 units (about -110, a spread of about 1
    across the keys of a row, so attention is diffuse)."""
    rng = np.random.default_rng(seed)
    u = rng.choice([-1.0, 1.0], size=d)
    beta = 110.0 / (np.sqrt(d) * np.log2(np.e))
    k = u[None, :] + 0.1 * rng.standard_normal((n_pad, d))
    q = -beta * u[None, :] + 0.3 * rng.standard_normal((n_pad, d))
    v = rng.standard_normal((n_pad, d))
    out = []
    for x in (q, k, v):
        x[n_valid:] = 0.0
        out.append(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).reshape(1, 1, n_pad, d))
    return out


@pytest.mark.parametrize("case", ["rising", "gentle", "negative"])
@pytest.mark.parametrize("d,C", [(128, 128), (64, 64)])
def test_logit_range_dense_sparse_residual(mcs, d, C, case):
    n_valid, n_pad = 700, 768            # 11 key tiles, the last one ragged (60 keys)
    print(f"logit range {case} d{d} C{C}", flush=True)
    if case == "negative":
        q, k, v = negative_inputs(d, n_valid, n_pad, seed=d + C)
    else:
        q, k, v = rising_inputs(d, n_valid, n_pad, seed=d + C, slope=1.0 if case == "rising" else 0.25)
    sc = 1.0 / np.sqrt(d)
    qf, kf, vf = (par.bf16_to_f64(t[0, 0]) for t in (q, k, v))
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))

    # dense: the online softmax runs over all 11 tiles in key order
    o, lse = mcs.dense_attn(qd, kd, vd, n_valid, C, sc)
    torch.cuda.synchronize()
    ref_o, ref_l = orc.dense_attention(qf, kf, vf, n_valid, sc)
    logits = (qf[:n_valid] @ kf[:n_valid].T) * sc * np.log2(np.e)
    s_max = float(logits.max())
    if case == "rising":
        assert s_max > 120.0, "the inputs do not reach the intended logit range"
    elif case == "gentle":
        # every row's sum stays inside the zero-offset pass's [2^-60, 2^64]
        assert 25.0 < s_max < 55.0 and float(logits.max(axis=1).min()) > -50.0, "logits outside the intended range"
    else:
        assert s_max < -70.0, "the inputs do not reach the intended logit range"
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


@pytest.mark.parametrize("d,C", [(128, 128), (64, 64)])
def test_redo_in_some_groups_of_one_launch(mcs, d, C):
    """One reuse-step launch in which some groups take the redo and the others
    keep the first pass: with the rising inputs, rows near +u overflow the
    first pass's range and rows near -u do not; a perm that lists the +u rows
    first gives groups of only +u rows, one mixed group, and groups of only -u
    rows.  Both kinds are checked against the oracle in the same launch."""
    n_valid, n_pad = 700, 768
    print(f"redo in some groups d{d} C{C}", flush=True)
    q, k, v = rising_inputs(d, n_valid, n_pad, seed=3 * d + C)
    sc = 1.0 / np.sqrt(d)
    qf, kf, vf = (par.bf16_to_f64(t[0, 0]) for t in (q, k, v))
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    G, topk = n_pad // C, 333
    rows = np.arange(n_valid)
    perm = np.concatenate([rows[rows % 2 == 0], rows[rows % 2 == 1], np.arange(n_valid, n_pad)]).astype(np.int32)
    rng = np.random.default_rng(11)
    kv = np.stack([np.sort(rng.choice(n_valid, topk, replace=False)) for _ in range(G)]).astype(np.int32)
    # each group's largest row sum of 2^(scaled logit) over its keys, in log2
    # units: beyond 64 the first pass is rejected, inside [-60, 64] it is kept
    log2sum = []
    for g in range(G):
        members = [int(i) for i in perm[g * C:(g + 1) * C] if i < n_valid]
        if not members:                  # a group of padding rows only
            continue
        lg = (qf[members] @ kf[kv[g]].T) * sc * np.log2(np.e)
        m = lg.max(axis=1, keepdims=True)
        log2sum.append(float((m[:, 0] + np.log2(np.exp2(lg - m).sum(axis=1))).max()))
    redo = [x > 64.0 for x in log2sum]
    assert any(redo) and not all(redo), f"the launch is not mixed: {log2sum}"
    assert all(x > -60.0 for x in log2sum)
    r = torch.from_numpy(0.05 * rng.standard_normal((1, 1, n_pad, d)).astype(np.float32)).to(torch.bfloat16)
    r[:, :, n_valid:] = 0
    pd = torch.from_numpy(perm).reshape(1, 1, n_pad).to(DEV)
    kvd = torch.from_numpy(kv).reshape(1, 1, G, topk).to(DEV)
    os_ = mcs.sparse_attn(qd, kd, vd, pd, kvd, r.to(DEV), n_valid, C, sc)
    torch.cuda.synchronize()
    ref_s = orc.reuse_step(qf, kf, vf, perm, kv, par.bf16_to_f64(r[0, 0]), n_valid, C, sc)
    par.assert_close(par.bf16_to_f64(os_[0, 0].cpu())[:n_valid], ref_s[:n_valid], what="reuse step")
