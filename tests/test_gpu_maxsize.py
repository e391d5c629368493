"""The largest supported sequence: n_pad = 2^24 - 128 tokens (one head, d = 128,
C = 128, 131071 groups), where a head's K/V rows span just under the 4 GiB
reach of the 32-bit buffer offsets.

Inputs are drawn on the device from a seeded generator (4.3 GB per tensor is
too much to draw on the host); the oracle then checks sampled groups from the
bytes the GPU used.  The reuse step runs on random ascending index sets that
include the last tokens; the grouping runs all 17 levels and is checked for
its invariants (a partition of the tokens into ascending groups of C).
"""
import numpy as np
import pytest
import torch

from oracle import mcs_oracle as orc
from tests import parity as par

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_PAD = (1 << 24) - 128
N_VALID = N_PAD - 77
D, C, K = 128, 128, 64


@pytest.fixture(scope="module")
def mcs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_diffusion_attn_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def qkv():
    g = torch.Generator(device=DEV)
    g.manual_seed(1234)
    out = []
    for _ in range(3):
        t = torch.randn((1, 1, N_PAD, D), generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
        t[:, :, N_VALID:] = 0
        out.append(t)
    torch.cuda.synchronize()
    yield out
    del out
    torch.cuda.empty_cache()


def test_max_size_sparse_attention(mcs, qkv):
    q, k, v = qkv
    print(f"max size sparse: n_pad {N_PAD}, groups {N_PAD // C}", flush=True)
    G = N_PAD // C
    g = torch.Generator(device=DEV)
    g.manual_seed(99)
    # k ascending distinct keys per group: sorted random draws, made distinct by
    # spreading them over k equal strata of the valid range; the last group
    # takes the last k valid tokens
    stride = N_VALID // K
    base = torch.arange(K, device=DEV, dtype=torch.int64) * stride
    off = torch.randint(0, stride, (G, K), generator=g, device=DEV)
    kv = (base[None, :] + off).to(torch.int32)
    kv[-1] = torch.arange(N_VALID - K, N_VALID, device=DEV, dtype=torch.int32)
    kv = kv.reshape(1, 1, G, K).contiguous()
    perm = torch.arange(N_PAD, device=DEV, dtype=torch.int32).reshape(1, 1, N_PAD)
    r = (0.01 * torch.randn((1, 1, N_PAD, D), generator=g, device=DEV)).to(torch.bfloat16)
    r[:, :, N_VALID:] = 0
    sc = 1.0 / np.sqrt(D)
    o = mcs.sparse_attn(q, k, v, perm, kv, r, N_VALID, C, sc)
    torch.cuda.synchronize()
    assert bool((o[0, 0, N_VALID:] == 0).all())
    for grp in (0, 1, G // 2, G - 2, G - 1):
        rows = np.arange(grp * C, (grp + 1) * C)
        sel = kv[0, 0, grp].cpu().numpy()
        qg = par.bf16_to_f64(q[0, 0, grp * C:(grp + 1) * C].cpu())
        kg = par.bf16_to_f64(k[0, 0].index_select(0, kv[0, 0, grp].long()).cpu())
        vg = par.bf16_to_f64(v[0, 0].index_select(0, kv[0, 0, grp].long()).cpu())
        rg = par.bf16_to_f64(r[0, 0, grp * C:(grp + 1) * C].cpu())
        # the oracle on a compacted slice: the group's own rows and its keys
        nv_local = int(np.sum(rows < N_VALID))
        want = orc.reuse_step(qg, kg, vg, np.arange(C), np.arange(K)[None, :], rg, nv_local, C, sc)
        got = par.bf16_to_f64(o[0, 0, grp * C:(grp + 1) * C].cpu())
        assert sel.max() < N_VALID
        par.assert_close(got[:nv_local], want[:nv_local], what=f"max-size group {grp}")


def test_max_size_grouping_invariants(mcs, qkv):
    q = qkv[0]
    print("max size grouping", flush=True)
    perm = mcs.group(q, N_VALID, C, 20)
    torch.cuda.synchronize()
    p = perm[0, 0]
    assert torch.equal(torch.sort(p)[0], torch.arange(N_PAD, device=DEV, dtype=torch.int32))
    pg = p.reshape(N_PAD // C, C)
    assert bool((pg[:, 1:] > pg[:, :-1]).all()), "group members are not ascending"
