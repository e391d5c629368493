"""mcs_anchor_select_noalloc (the anchor selection with the library's fixed
device scratch as its workspace) gives bitwise the results of
mcs_anchor_select with a caller workspace, on two calls in a row, the second
on a smaller layer (the scratch keeps the first call's contents)."""
import pytest
import torch

import synthdata as sd

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def mcs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_diffusion_attn_amd as m
    m.lib()
    return m


def _check(mcs, cfg):
    q, k, v = (t.to(DEV) for t in sd.generate(cfg, steps=1)[0])
    nv, C, sc = cfg.n_valid, cfg.group_size, cfg.scale
    perm = mcs.group(q, nv, C, cfg.power_iters)
    ref = mcs.anchor_select(q, k, v, perm, nv, C, cfg.topk, sc)
    got = mcs.anchor_select_noalloc(q, k, v, perm, nv, C, cfg.topk, sc)
    torch.cuda.synchronize()
    for name, a, b in zip(("o_full", "lse", "kv_idx"), ref, got):
        assert torch.equal(a, b), f"{cfg.name}: {name} differs"


def test_noalloc_matches_workspace_call_twice(mcs):
    # first call: 12 heads of 30000 tokens (about 28 MB of scores per head,
    # six heads per scratch chunk), then a smaller layer with d = 64, C = 64
    big = sd.custom("noalloc_big", heads=12, n_valid=30000, head_dim=128, group_size=128,
                    density_pct=25, n_clusters=32)
    small = sd.custom("noalloc_small", heads=2, n_valid=3000, head_dim=64, group_size=64,
                      density_pct=15, n_clusters=8)
    dims = mcs.make_dims(1, big.heads, big.n_valid, big.n_pad, big.head_dim, big.group_size)
    per_head = mcs.anchor_select_workspace_bytes(dims, big.topk, minimum=True)
    assert 1 < mcs.NOALLOC_SCRATCH_BYTES // per_head < big.heads  # several chunks
    _check(mcs, big)
    _check(mcs, small)


def test_noalloc_rejects_heads_beyond_the_scratch(mcs):
    # one head of the Hunyuan 720p layer needs about 445 MB of scores
    cfg = sd.CONFIGS["hunyuan720p_25"]
    q = torch.zeros((1, 1, cfg.n_pad, 128), dtype=torch.bfloat16, device=DEV)
    perm = torch.zeros((1, 1, cfg.n_pad), dtype=torch.int32, device=DEV)
    with pytest.raises(mcs.MCSError) as e:
        mcs.anchor_select_noalloc(q, q, q, perm, cfg.n_valid, cfg.group_size, cfg.topk, cfg.scale)
    assert e.value.status == mcs.MCS_ERR_UNSUPPORTED and "scratch" in str(e.value)
