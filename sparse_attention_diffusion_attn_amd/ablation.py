"""Synthetic ablation ladder of MC-Sparse's design choices on the GPU path.

The onedev.kr summary ("how it works" and the system/ablation paragraph)
builds MC-Sparse from vanilla block-sparse attention (BSA) by adding, in turn:
exact KV selection with cross-step reuse, token-level KV granularity, query
grouping and residual compensation, and reports that each step improves
fidelity at every density.  The pages measure fidelity on generated videos;
here the measure is the error of one attention layer's reuse-step output
against dense attention at the same step, on the seeded synthetic layers.

Rungs (all at one density: k = ceil(density * N) tokens, or the nearest whole
number of KV blocks of C keys):
  1  vanilla BSA            contiguous query blocks, KV blocks ranked by
                            mean-pooled q . k computed at the current step
  2  + exact, reused        blocks chosen at the anchor by exact probability
                            mass (block oracle), reused at the reuse step
  3  + token granularity    individual KV tokens chosen at the anchor by exact
                            probability (token oracle), reused
  4  + query grouping       Fast PDDP groups instead of contiguous blocks
  5  + residual             R = O_full - O_sparse from the anchor added
                            (MC-Sparse)

Every rung runs in the library's kernels (mcs_block_select,
mcs_anchor_select, mcs_group, mcs_residual(_counts),
mcs_sparse_attn(_counts), mcs_dense_attn).

The synthetic layers are run with both label layouts of synthdata: "random"
(a cluster's tokens scattered over the sequence, the adversarial case for
contiguous blocks) and "grid" (clusters are spatial cells of the latent grid,
so contiguous blocks see a handful of clusters).

Usage: python -m sparse_attention_diffusion_attn_amd.ablation [--config 480p]
       [--densities 15,25] [--layouts random,grid] [--drift-steps 1]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import sparse_attention_diffusion_attn_amd as mcs  # noqa: E402
import synthdata as sd  # noqa: E402

RUNGS = ["vanilla BSA", "+ exact selection, reused", "+ token granularity",
         "+ query grouping", "+ residual (MC-Sparse)"]


def rel_err(o, ref, nv):
    a = o[:, :, :nv].float()
    b = ref[:, :, :nv].float()
    return float((a - b).norm() / b.norm())


def ladder(cfg, drift_steps=1):
    """Errors of the five rungs at reuse step `drift_steps` after the anchor."""
    dev = "cuda:0"
    steps = [tuple(t.to(dev) for t in s) for s in sd.generate(cfg, steps=1 + drift_steps)]
    (q0, k0, v0), (qt, kt, vt) = steps[0], steps[-1]
    B, H, nv, n_pad, d, C, k = cfg.batch, cfg.heads, cfg.n_valid, cfg.n_pad, cfg.head_dim, cfg.group_size, cfg.topk
    sc = cfg.scale
    nb_all = (nv + C - 1) // C
    n_b = min(nb_all, max(1, (k + C // 2) // C))
    ident = mcs.identity_perm(B, H, n_pad, dev)

    o_dense_t, _ = mcs.dense_attn(qt, kt, vt, nv, C, sc, want_lse=False)
    o_full0, lse0 = mcs.dense_attn(q0, k0, v0, nv, C, sc)
    out = {}
    # 1: vanilla BSA at the current step
    kv, cnt = mcs.block_select(qt, kt, ident, None, mcs.BLOCK_MEANPOOL, C, n_b, nv, C, sc)
    out[RUNGS[0]] = rel_err(mcs.sparse_attn_counts(qt, kt, vt, ident, kv, cnt, None, nv, C, sc), o_dense_t, nv)
    # 2: block oracle at the anchor, reused
    kv, cnt = mcs.block_select(q0, k0, ident, lse0, mcs.BLOCK_EXACT, C, n_b, nv, C, sc)
    out[RUNGS[1]] = rel_err(mcs.sparse_attn_counts(qt, kt, vt, ident, kv, cnt, None, nv, C, sc), o_dense_t, nv)
    # 3: token oracle at the anchor (contiguous query blocks), reused
    _, _, kv_tok = mcs.anchor_select(q0, k0, v0, ident, nv, C, k, sc)
    out[RUNGS[2]] = rel_err(mcs.sparse_attn(qt, kt, vt, ident, kv_tok, None, nv, C, sc), o_dense_t, nv)
    # 4: PDDP groups + token oracle, reused
    perm = mcs.group(q0, nv, C, cfg.power_iters)
    o_full, _, kv_g = mcs.anchor_select(q0, k0, v0, perm, nv, C, k, sc)
    out[RUNGS[3]] = rel_err(mcs.sparse_attn(qt, kt, vt, perm, kv_g, None, nv, C, sc), o_dense_t, nv)
    # 5: + residual
    r = mcs.residual(q0, k0, v0, perm, kv_g, o_full, nv, C, sc)
    out[RUNGS[4]] = rel_err(mcs.sparse_attn(qt, kt, vt, perm, kv_g, r, nv, C, sc), o_dense_t, nv)
    torch.cuda.synchronize()
    return {"tokens": k, "blocks": n_b, "block_tokens": n_b * C, "rel_l2": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="480p")
    ap.add_argument("--densities", default="15,25")
    ap.add_argument("--drift-steps", type=int, default=1)
    ap.add_argument("--layouts", default="random,grid")
    args = ap.parse_args()
    assert torch.cuda.is_available(), "the ablation runs on the GPU"
    mcs.lib()
    base = sd.CONFIGS[args.config]
    rows = []
    for layout in args.layouts.split(","):
        for dens in (int(x) for x in args.densities.split(",")):
            cfg = dataclasses.replace(base, density_pct=dens, n_reuse=args.drift_steps, layout=layout)
            res = ladder(cfg, args.drift_steps)
            res.update({"config": args.config, "layout": layout, "density_pct": dens,
                        "drift_steps": args.drift_steps})
            rows.append(res)
            print(f"# {args.config} {layout} labels, density {dens}% (k={res['tokens']} tokens, "
                  f"{res['blocks']} blocks = {res['block_tokens']} tokens), reuse step "
                  f"{args.drift_steps}: relative L2 error of the layer output vs dense attention",
                  file=sys.stderr)
            for name, e in res["rel_l2"].items():
                print(f"#   {name:28s} {e:.5f}", file=sys.stderr)
    print(json.dumps({"ablation": rows}))


if __name__ == "__main__":
    main()
