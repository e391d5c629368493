"""The ablation ladder module runs end to end on the GPU path (all rungs in
the library's kernels) on a small grid-label layer, and the residual rung
improves on the grouped rung after one step of drift.  At 10% density the
grouped rung keeps a sparse error well above the bf16 rounding floor of the
outputs (about 0.004 relative L2), which the residual removes; at that floor
the two rungs are indistinguishable."""
import dataclasses

import pytest
import torch

import synthdata as sd

pytestmark = pytest.mark.gpu


def test_ladder_runs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_diffusion_attn_amd import ablation
    cfg = dataclasses.replace(sd.custom("abl", heads=2, n_valid=4000, head_dim=128, group_size=128,
                                        density_pct=10, n_clusters=16),
                              grid=(4, 25, 40), layout="grid")
    res = ablation.ladder(cfg, 1)
    e = list(res["rel_l2"].values())
    print(res)
    assert len(e) == 5 and all(0.0 < x < 10.0 for x in e)
    assert e[4] < max(e[3], 0.005)
