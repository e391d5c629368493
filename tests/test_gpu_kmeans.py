"""GPU parity of the size-balanced k-means grouping (mcs_group_kmeans), the
comparator of Fast PDDP, iteration by iteration against the fp64 oracle
(tests/parity.check_kmeans_step), plus output invariants and determinism."""
import numpy as np
import pytest
import torch

import synthdata as sd
from oracle import kmeans as okm
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


CASES = [
    sd.custom("km-d128", batch=1, heads=2, n_valid=1000, head_dim=128, group_size=128, n_clusters=8),
    sd.custom("km-d64-b2", batch=2, heads=2, n_valid=2000, head_dim=64, group_size=64, n_clusters=12,
              seed=4),
    # more tokens than one balancing tile (1024), a ragged last tile, padding rows
    sd.custom("km-tiles", batch=1, heads=1, n_valid=3000, head_dim=128, group_size=64, n_clusters=20,
              seed=7),
]


def is_partition(perm, n_pad):
    return np.array_equal(np.sort(perm), np.arange(n_pad))


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_kmeans_iterations_match_oracle(mcs, cfg):
    print(f"kmeans {cfg}", flush=True)
    q = sd.generate(cfg, steps=1)[0][0].to(DEV)
    C, nv = cfg.group_size, cfg.n_valid
    p0 = mcs.group_kmeans(q, nv, C, iters=0)
    torch.cuda.synchronize()
    ident = np.arange(cfg.n_pad)
    assert all(np.array_equal(p0[b, h].cpu().numpy(), ident)
               for b in range(cfg.batch) for h in range(cfg.heads))
    prev = p0
    diffs = 0
    for it in range(1, 5):
        perm, lab = mcs.group_kmeans(q, nv, C, iters=it, want_labels=True)
        torch.cuda.synchronize()
        for b in range(cfg.batch):
            for h in range(cfg.heads):
                x = par.bf16_to_f64(q[b, h].cpu())
                diffs += par.check_kmeans_step(x, prev[b, h].cpu().numpy(), lab[b, h].cpu().numpy(),
                                               perm[b, h].cpu().numpy(), C)
        prev = perm
    print(f"labels inside the rounding margin that differ: {diffs}")


def test_kmeans_full_size_last_iteration(mcs):
    """480p layer (24 heads x 32768 tokens, 256 groups): the last of 10
    iterations checked on three heads; every head's output is a partition."""
    cfg = sd.CONFIGS["480p"]
    q = sd.generate(cfg, steps=1)[0][0].to(DEV)
    C, nv = cfg.group_size, cfg.n_valid
    p9 = mcs.group_kmeans(q, nv, C, iters=9)
    p10, lab = mcs.group_kmeans(q, nv, C, iters=10, want_labels=True)
    torch.cuda.synchronize()
    for h in range(cfg.heads):
        assert is_partition(p10[0, h].cpu().numpy(), cfg.n_pad)
    for h in (0, 11, 23):
        x = par.bf16_to_f64(q[0, h].cpu())
        par.check_kmeans_step(x, p9[0, h].cpu().numpy(), lab[0, h].cpu().numpy(),
                              p10[0, h].cpu().numpy(), C)


def test_kmeans_is_deterministic_and_separated_clusters_recovered(mcs):
    torch.manual_seed(0)
    G, C, d = 16, 64, 128
    centres = 8.0 * torch.randn(G, d)
    truth = torch.arange(G).repeat_interleave(C)
    order = torch.arange(G * C)
    for g in range(G):  # one point exchanged with each neighbouring block (cyclic)
        a, b = g * C + C - 1, ((g + 1) % G) * C
        order[a], order[b] = order[b].clone(), order[a].clone()
    x = (centres[truth] + 0.05 * torch.randn(G * C, d))[order]
    q = x.to(torch.bfloat16).reshape(1, 1, G * C, d).to(DEV)
    p1 = mcs.group_kmeans(q, G * C, C, iters=3)
    p2 = mcs.group_kmeans(q, G * C, C, iters=3)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)
    lab_true = truth[order].numpy()
    perm = p1[0, 0].cpu().numpy()
    for g in range(G):
        assert set(lab_true[perm[g * C:(g + 1) * C]]) == {g}
    xo = par.bf16_to_f64(q[0, 0].cpu())
    assert np.array_equal(perm, okm.balanced_kmeans(xo, C, 3))
