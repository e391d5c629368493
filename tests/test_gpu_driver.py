"""The multi-layer driver over a schedule with dense warm-up, a first anchor,
reuse steps and refresh anchors (the onedev.kr summary, "what is different":
an anchor is the last warm-up step or the last step of a refresh interval;
"how it is used", last paragraph: inactive cache entries offloaded to the host
and prefetched one layer ahead).

test_offload_matches_resident: offloaded metadata (pinned host memory, two
device slots, prefetch on a copy stream) gives bitwise the resident outputs.

test_schedule_against_oracle: with offload on, every (step, layer) output is
checked against the fp64 oracle: dense and anchor steps against dense
attention; each anchor's metadata, read back from its pinned host copy, against
the oracle's selection and residual rules; each reuse step against the oracle's
reuse step on the metadata of the latest anchor, as it came back from the host.
Every anchor epoch draws fresh inputs, so metadata of an earlier anchor would
give a far larger error than the tolerance (asserted for the steps after each
refresh).
"""
import numpy as np
import pytest
import torch

import synthdata as sd
from oracle import mcs_oracle as orc
from tests import parity as par

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
f64 = par.bf16_to_f64


def _setup(n_layers, n_steps, per_epoch_data):
    from sparse_attention_diffusion_attn_amd.driver import LayerShape, Schedule
    sched = Schedule(n_steps, warmup=2, refresh=3)
    kinds = sched.kinds()
    assert kinds == ["dense", "anchor", "reuse", "reuse", "anchor", "reuse", "reuse", "anchor"]
    # first step of the epoch each step belongs to (dense step, or its anchor)
    epoch = [max(e for e in range(s + 1) if e == 0 or kinds[e] == "anchor") for s in range(n_steps)]
    base = dict(heads=2, n_valid=1000, head_dim=128, group_size=128, n_clusters=6, n_reuse=n_steps - 1)
    cpu = []
    for layer in range(n_layers):
        if per_epoch_data:
            runs = {e: sd.generate(sd.custom(f"drv{layer}_{e}", seed=100 * layer + e, **base))
                    for e in sorted(set(epoch))}
            cpu.append([runs[epoch[s]][s - epoch[s]] for s in range(n_steps)])
        else:
            cpu.append(sd.generate(sd.custom(f"drv{layer}", seed=layer, **base)))
    c = sd.custom("shape", **base)
    shape = LayerShape(c.batch, c.heads, c.n_valid, c.n_pad, c.head_dim, c.group_size, c.topk)
    return sched, kinds, epoch, cpu, shape, c


def test_offload_matches_resident():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_diffusion_attn_amd.driver import Stack
    n_layers, n_steps = 5, 8
    sched, _, _, cpu, shape, c = _setup(n_layers, n_steps, per_epoch_data=False)
    data = [[tuple(t.to(DEV) for t in s) for s in layer] for layer in cpu]
    inputs = lambda layer, step: data[layer][step]  # noqa: E731
    results = {}
    for offload in (False, True):
        outs = [[torch.empty_like(data[0][0][0]) for _ in range(n_layers)] for _ in range(n_steps)]
        Stack(n_layers, shape, inputs, offload, c.scale, device=DEV).run(sched, outs)
        torch.cuda.synchronize()
        results[offload] = outs
    for s in range(n_steps):
        for l in range(n_layers):
            assert torch.equal(results[False][s][l], results[True][s][l]), f"step {s} layer {l}"


def test_schedule_against_oracle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_diffusion_attn_amd.driver import Stack
    n_layers, n_steps = 5, 8
    sched, kinds, epoch, cpu, shape, c = _setup(n_layers, n_steps, per_epoch_data=True)
    data = [[tuple(t.to(DEV) for t in s) for s in layer] for layer in cpu]
    inputs = lambda layer, step: data[layer][step]  # noqa: E731
    stack = Stack(n_layers, shape, inputs, True, c.scale, device=DEV)
    outs = [[torch.empty_like(data[0][0][0]) for _ in range(n_layers)] for _ in range(n_steps)]
    meta = {}   # (anchor step, layer) -> (perm, kv_idx, R) as they came back to the host
    for s, kind in enumerate(kinds):
        stack.step(s, kind, outs[s])
        torch.cuda.synchronize()
        if kind == "anchor":
            for l in range(n_layers):
                meta[(s, l)] = tuple(t.clone() for t in stack.store.host[l])
    nv, C, sc, G, k = c.n_valid, c.group_size, c.scale, c.groups, c.topk
    stale_gap = []
    for s, kind in enumerate(kinds):
        for l in range(n_layers):
            q, kk, v = (f64(t[0]) for t in cpu[l][s])
            got = f64(outs[s][l][0])
            for h in range(c.heads):
                if kind in ("dense", "anchor"):
                    ref, lse = orc.dense_attention(q[h], kk[h], v[h], nv, sc)
                    par.assert_close(got[h][:nv], ref[:nv], what=f"{kind} step {s} layer {l} head {h}")
                    assert np.all(got[h][nv:] == 0)
                if kind == "anchor":
                    perm, kv = (t[0, h].numpy() for t in meta[(s, l)][:2])
                    r = f64(meta[(s, l)][2][0, h])
                    assert sorted(perm.tolist()) == list(range(c.n_pad))
                    a = orc.group_scores(q[h], kk[h], perm, lse, nv, C, sc)
                    for g in range(G):
                        par.check_selection(kv[g], a[g], k)
                    o_sp = orc.sparse_attention(q[h], kk[h], v[h], perm, kv, nv, C, sc)
                    par.assert_close(r[:nv], (got[h] - o_sp)[:nv], what=f"R of anchor {s} layer {l} head {h}")
                if kind == "reuse":
                    e = epoch[s]
                    perm, kv = (t[0, h].numpy() for t in meta[(e, l)][:2])
                    r = f64(meta[(e, l)][2][0, h])
                    ref = orc.reuse_step(q[h], kk[h], v[h], perm, kv, r, nv, C, sc)
                    par.assert_close(got[h][:nv], ref[:nv], what=f"reuse step {s} layer {l} head {h}")
                    assert np.all(got[h][nv:] == 0)
                    earlier = [a for (a, ll) in meta if ll == l and a < e]
                    if earlier:
                        a0 = max(earlier)
                        p0, kv0 = (t[0, h].numpy() for t in meta[(a0, l)][:2])
                        stale = orc.reuse_step(q[h], kk[h], v[h], p0, kv0, f64(meta[(a0, l)][2][0, h]), nv, C, sc)
                        stale_gap.append(float(np.abs(got[h][:nv] - stale[:nv]).mean()))
    # outputs built on the previous anchor's metadata would fail the check
    assert stale_gap and min(stale_gap) > 20 * par.MEAN_ABS, min(stale_gap)
    print(f"schedule {kinds}: {n_layers} layers checked; stale-metadata gap >= {min(stale_gap):.3f}")
