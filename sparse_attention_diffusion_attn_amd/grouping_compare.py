"""Fast PDDP against the size-balanced k-means comparator on the GPU.

The onedev.kr summary ("how it is used", component 2, and the system
paragraph) picks PDDP median splits over k-means because the query tile needs
groups of exactly C, and reports Fast PDDP's grouping cost against
Flash-KMeans.  This measures, on the seeded synthetic layers, both groupings
as built here (mcs_group and mcs_group_kmeans), each producing tile-aligned
groups:

  time      per call (HIP events, median of repeats); for k-means also the
            cost of one iteration
  spread    within-group sum of squared distances to the group mean, as a
            fraction of the head's total (fp64, all heads)
  accuracy  relative L2 error of the reuse-step output against dense attention
            one drift step after the anchor, with and without the residual,
            when the groups feed the same selection and sparse kernels

Usage: python -m sparse_attention_diffusion_attn_amd.grouping_compare
       [--configs 480p,wan720p] [--layout random] [--iters 1,5,10,20]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import statistics
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import sparse_attention_diffusion_attn_amd as mcs  # noqa: E402
import synthdata as sd  # noqa: E402


def timed(fn, reps):
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return statistics.median(ts)


def spread(q, perm, C):
    """Within-group SSE / total SSE about the head mean, over all heads."""
    within = total = 0.0
    B, H, n_pad, d = q.shape
    for b in range(B):
        for h in range(H):
            x = q[b, h].double()
            xg = x[perm[b, h].long()].reshape(n_pad // C, C, d)
            within += float(((xg - xg.mean(dim=1, keepdim=True)) ** 2).sum())
            total += float(((x - x.mean(dim=0, keepdim=True)) ** 2).sum())
    return within / total


def reuse_error(cfg, steps, perm):
    (q0, k0, v0), (qt, kt, vt) = steps
    nv, C, k, sc = cfg.n_valid, cfg.group_size, cfg.topk, cfg.scale
    o_ref, _ = mcs.dense_attn(qt, kt, vt, nv, C, sc, want_lse=False)
    o_full, _, kv = mcs.anchor_select(q0, k0, v0, perm, nv, C, k, sc)
    r = mcs.residual(q0, k0, v0, perm, kv, o_full, nv, C, sc)
    out = {}
    for name, res in (("no_residual", None), ("residual", r)):
        o = mcs.sparse_attn(qt, kt, vt, perm, kv, res, nv, C, sc)
        a = o[:, :, :nv].float()
        ref = o_ref[:, :, :nv].float()
        out[name] = float((a - ref).norm() / ref.norm())
    return out


def compare(cfg, iters_list, reps=3):
    dev = "cuda:0"
    steps = [tuple(t.to(dev) for t in s) for s in sd.generate(cfg, steps=2)]
    q = steps[0][0]
    nv, C = cfg.n_valid, cfg.group_size
    ws_p = torch.empty(mcs.group_workspace_bytes(mcs._dims_of(q, nv, C)), dtype=torch.uint8, device=dev)
    dims = mcs._dims_of(q, nv, C)
    import ctypes
    ws_k = torch.empty(int(mcs.lib().mcs_group_kmeans_workspace_bytes(ctypes.byref(dims))),
                       dtype=torch.uint8, device=dev)
    perm = mcs.group(q, nv, C, cfg.power_iters, workspace=ws_p)
    torch.cuda.synchronize()
    res = {"config": cfg.name, "layout": cfg.layout, "heads": cfg.batch * cfg.heads,
           "n_pad": cfg.n_pad, "groups": cfg.groups}
    res["pddp"] = {"ms": timed(lambda: mcs.group(q, nv, C, cfg.power_iters, perm=perm, workspace=ws_p), reps),
                   "spread": spread(q, perm, C), "error": reuse_error(cfg, steps, perm)}
    res["contiguous"] = {"spread": spread(q, mcs.identity_perm(cfg.batch, cfg.heads, cfg.n_pad, dev), C)}
    km = {}
    pk = torch.empty_like(perm)
    for it in iters_list:
        ms = timed(lambda: mcs.group_kmeans(q, nv, C, it, perm=pk, workspace=ws_k), reps)
        km[it] = {"ms": ms, "spread": spread(q, pk, C)}
        if it == max(iters_list):
            km[it]["error"] = reuse_error(cfg, steps, pk)
    res["kmeans"] = km
    lo, hi = min(iters_list), max(iters_list)
    res["kmeans_ms_per_iter"] = (km[hi]["ms"] - km[lo]["ms"]) / (hi - lo) if hi > lo else None
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--configs", default="480p,wan720p,hunyuan720p_15,3d")
    ap.add_argument("--layout", default="random")
    ap.add_argument("--iters", default="1,5,10,20")
    args = ap.parse_args()
    assert torch.cuda.is_available(), "the comparison runs on the GPU"
    mcs.lib()
    iters = [int(x) for x in args.iters.split(",")]
    rows = []
    for name in args.configs.split(","):
        cfg = dataclasses.replace(sd.CONFIGS[name], layout=args.layout)
        r = compare(cfg, iters)
        rows.append(r)
        p = r["pddp"]
        print(f"# {name} ({args.layout} labels, {r['heads']} heads x {r['n_pad']} tokens, "
              f"{r['groups']} groups): PDDP {p['ms']:.2f} ms spread {p['spread']:.4f} "
              f"err {p['error']['no_residual']:.4f}/{p['error']['residual']:.4f}; "
              f"contiguous spread {r['contiguous']['spread']:.4f}", file=sys.stderr)
        for it, k in r["kmeans"].items():
            e = k.get("error")
            es = f" err {e['no_residual']:.4f}/{e['residual']:.4f}" if e else ""
            print(f"#   k-means {it:3d} iters: {k['ms']:.2f} ms spread {k['spread']:.4f}{es}",
                  file=sys.stderr)
        if r["kmeans_ms_per_iter"] is not None:
            print(f"#   k-means per iteration: {r['kmeans_ms_per_iter']:.3f} ms", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    print(json.dumps({"grouping_compare": rows}))


if __name__ == "__main__":
    main()
