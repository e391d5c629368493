"""The multi-layer driver gives bitwise the same outputs with metadata offloaded
to pinned host memory (two device slots, prefetch one layer ahead on a copy
stream) as with every layer resident, over a schedule with dense warm-up,
anchors and reuse steps."""
import pytest
import torch

import synthdata as sd

pytestmark = pytest.mark.gpu


def test_offload_matches_resident():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_diffusion_attn_amd.driver import LayerShape, Schedule, Stack
    dev = "cuda:0"
    n_layers, n_steps = 5, 8
    cfgs = [sd.custom(f"drv{l}", heads=2, n_valid=1000, head_dim=128, group_size=128, n_clusters=6,
                      n_reuse=n_steps - 1, seed=l) for l in range(n_layers)]
    data = [[tuple(t.to(dev) for t in s) for s in sd.generate(c)] for c in cfgs]
    c = cfgs[0]
    shape = LayerShape(c.batch, c.heads, c.n_valid, c.n_pad, c.head_dim, c.group_size, c.topk)
    inputs = lambda layer, step: data[layer][step]  # noqa: E731
    sched = Schedule(n_steps, warmup=2, refresh=3)
    assert sched.kinds() == ["dense", "anchor", "reuse", "reuse", "anchor", "reuse", "reuse", "anchor"]
    results = {}
    for offload in (False, True):
        outs = [[torch.empty_like(data[0][0][0]) for _ in range(n_layers)] for _ in range(n_steps)]
        Stack(n_layers, shape, inputs, offload, c.scale, device=dev).run(sched, outs)
        torch.cuda.synchronize()
        results[offload] = outs
    for s in range(n_steps):
        for l in range(n_layers):
            assert torch.equal(results[False][s][l], results[True][s][l]), f"step {s} layer {l}"
