"""The C-ABI calls under HIP graph capture.

Every call only enqueues kernels on the caller's stream: no allocation, no
synchronisation, no memset.  So a whole anchor step (grouping, two-pass
selection, residual) and a reuse step can be captured once and replayed, as a
serving loop would.  Each replay, with eager work and synchronisations between
the replays, must reproduce the eager outputs bit for bit.
"""
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


@pytest.mark.parametrize("name", ["tiny", "b2"])
def test_anchor_and_reuse_steps_replay_from_a_graph(mcs, name):
    if name == "tiny":
        cfg = sd.CONFIGS["tiny"]
    else:
        cfg = sd.custom("b2", batch=2, heads=3, n_valid=900, head_dim=128, group_size=128,
                        density_pct=20, n_clusters=6)
    print(f"graph {cfg}", flush=True)
    (q0, k0, v0), (q1, k1, v1) = [tuple(t.to(DEV) for t in s) for s in sd.generate(cfg, steps=2)]
    nv, C, tk, sc = cfg.n_valid, cfg.group_size, cfg.topk, cfg.scale
    B, H, n_pad, d = q0.shape
    G = n_pad // C
    dims = mcs._dims_of(q0, nv, C)
    ws_g = torch.empty(mcs.group_workspace_bytes(dims), dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(mcs.anchor_select_workspace_bytes(dims, tk), dtype=torch.uint8, device=DEV)
    perm = torch.empty((B, H, n_pad), dtype=torch.int32, device=DEV)
    o_full = torch.empty_like(q0)
    lse = torch.empty((B, H, n_pad), dtype=torch.float32, device=DEV)
    kv = torch.empty((B, H, G, tk), dtype=torch.int32, device=DEV)
    r = torch.empty_like(q0)
    o = torch.empty_like(q0)

    def anchor():
        mcs.group(q0, nv, C, cfg.power_iters, perm=perm, workspace=ws_g)
        mcs.anchor_select(q0, k0, v0, perm, nv, C, tk, sc, o_full=o_full, lse=lse, kv_idx=kv,
                          workspace=ws_a)
        mcs.residual(q0, k0, v0, perm, kv, o_full, nv, C, sc, r=r)

    def reuse():
        mcs.sparse_attn(q1, k1, v1, perm, kv, r, nv, C, sc, o=o)

    anchor()
    reuse()
    torch.cuda.synchronize()
    want = [t.clone() for t in (perm, o_full, lse, kv, r, o)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm-up on the capture stream's side
        anchor()
        reuse()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_anchor, g_reuse = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_anchor):
        anchor()
    with torch.cuda.graph(g_reuse):
        reuse()
    for rep in range(3):
        for t in (perm, o_full, lse, kv, r, o):
            t.zero_()
        torch.cuda.synchronize()
        g_anchor.replay()
        g_reuse.replay()
        torch.cuda.synchronize()
        got = (perm, o_full, lse, kv, r, o)
        for name_, a, b in zip(("perm", "o_full", "lse", "kv_idx", "r", "o"), got, want):
            assert torch.equal(a, b), f"replay {rep}: {name_}"
        # eager work between the replays
        mcs.dense_attn(q1, k1, v1, nv, C, sc, want_lse=False)
        torch.cuda.synchronize()
