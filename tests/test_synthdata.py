"""The seeded input generator: shapes, padding, derived sizes and determinism."""
import torch

import synthdata as sd


def test_derived_sizes_of_the_layer_configs():
    want = {  # (N_pad, G, k, levels)
        "tiny": (1024, 16, 256, 4), "480p": (32768, 256, 8190, 8),
        "wan720p": (75648, 591, 11340, 10), "hunyuan720p_15": (118912, 929, 17820, 10),
        "hunyuan720p_25": (118912, 929, 29700, 10), "3d": (65536, 512, 9831, 9),
    }
    for name, (n_pad, G, k, L) in want.items():
        c = sd.CONFIGS[name]
        assert (c.n_pad, c.groups, c.topk, c.levels) == (n_pad, G, k, L), name


def test_generate_shapes_padding_determinism_and_head_subset():
    cfg = sd.custom(heads=3, n_valid=200, head_dim=16, group_size=64, n_reuse=2)
    a = sd.generate(cfg)
    b = sd.generate(cfg)
    assert len(a) == 3
    for (q, k, v), (q2, k2, v2) in zip(a, b):
        assert q.shape == (1, 3, 256, 16) and q.dtype == torch.bfloat16
        assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
        assert torch.all(q[:, :, 200:] == 0) and torch.all(v[:, :, 200:] == 0)
    assert not torch.equal(a[0][0], a[1][0])
    sub = sd.generate(cfg, heads=[2])
    for s in range(3):
        for t in range(3):
            assert torch.equal(sub[s][t][:, 0], a[s][t][:, 2])


def test_sample_groups():
    g = sd.sample_groups(sd.CONFIGS["480p"])
    assert g[0] == 0 and g[-1] == 255 and len(g) == 8 and g == sorted(set(g))
