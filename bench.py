#!/usr/bin/env python3
"""Benchmark of the MC-Sparse attention hot path on one MI355X.

One step = one pass of the whole hot path over one synthetic layer: the anchor
step (mcs_group -> mcs_anchor_select -> mcs_residual) followed by the layer's
reuse steps (mcs_sparse_attn on drifted Q/K/V, cached metadata).  Default
workload: the HunyuanVideo-13B-shaped 720p layer (B1 H24 N118800 -> 118912,
d128, C128, 25% density, k = 29700, 1 anchor + 8 reuse steps); the same layer
at 15% density (k = 17820: a second selection on the same inputs and groups)
is measured beside it.  To keep the CPU-side input generation short, the reuse
steps cycle over `--reuse-inputs` distinct drifted inputs (default 2) instead
of drawing one per step; the kernels' work does not depend on the values.

Headline metric: effective TFLOP/s of the reuse-step sparse attention
(4*B*H*N_pad*k*d executed flops / kernel time, HIP events on the launch
stream), and the achieved fraction of the ideal 1/s speed-up over the library's
own dense kernel (mcs_dense_attn) at the same shape: (k/N) * t_dense / t_sparse.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config hunyuan720p_25]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="hunyuan720p_25")
    ap.add_argument("--also-density", type=int, default=None,
                    help="second density (percent) measured on the same inputs "
                         "(default: 15 for the 25%% Hunyuan layer, none otherwise; 0 = none)")
    ap.add_argument("--reuse-inputs", type=int, default=2,
                    help="distinct drifted reuse-step inputs the reuse steps cycle over")
    ap.add_argument("--ratio-reps", type=int, default=10, help="reps of the dense-vs-sparse timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="time budget of the CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--reuse", type=int, default=None,
                    help="reuse steps per bench step (default: the layer config's own count)")
    ap.add_argument("--only", choices=["sparse", "dense", "anchor", "group", "copy"], default=None,
                    help="profile helper: run only this call in a loop (no JSON line)")
    return ap.parse_args()


def source_hash(*names):
    """Hash of the kernel sources' code: // comments and blank lines are
    dropped and whitespace collapsed, so that a comment edit does not
    invalidate a measurement taken on the same code."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_attention_diffusion_attn_amd", "csrc", n)) as f:
            for line in f:
                code = " ".join(line.split("//", 1)[0].split())
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic(config, kernel_src_hash):
    """HBM traffic per launch measured with rocprofv3 --pmc (FETCH_SIZE and
    WRITE_SIZE) on this config's sparse launch, stored with the hash of the
    kernel source it was taken on."""
    path = os.path.join(ROOT, "profiles", f"sparse_attn_{config}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_hash") != kernel_src_hash:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(cfg, q, k, v, perm, kv, budget_s):
    """The fp64 oracle's sparse attention on the first query groups of the
    layer (as many as fit in `budget_s`), one thread; returns its effective
    TFLOP/s in the metric's unit."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import mcs_oracle as orc

    flops_per_group = 4.0 * cfg.group_size * cfg.topk * cfg.head_dim
    perm_h, kv_h = perm.cpu().numpy(), kv.cpu().numpy()
    done, heads, t0 = 0, 0, time.perf_counter()
    with threadpool_limits(limits=1):
        for h in range(cfg.heads):
            qh = q[0, h].float().numpy().astype(np.float64)
            kh = k[0, h].float().numpy().astype(np.float64)
            vh = v[0, h].float().numpy().astype(np.float64)
            heads += 1
            for g in range(cfg.groups):
                orc.sparse_attention(qh, kh, vh, perm_h[0, h], kv_h[0, h][[g]], cfg.n_valid,
                                     cfg.group_size, cfg.scale, groups=[g])
                done += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": flops_per_group * done / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"fp64 oracle sparse attention of {done} query groups (C={cfg.group_size}, "
                      f"k={cfg.topk}, d={cfg.head_dim}) from the first {heads} head(s) of the same layer "
                      f"(reuse step 1, the GPU's metadata), one thread, "
                      f"{dt:.1f} s; host {model}, {os.cpu_count()} logical CPUs, {usable} usable"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "heads would shard across GPUs with no exchange, which is not implemented.", file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import torch
    import sparse_attention_diffusion_attn_amd as mcs
    import synthdata as sd

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mcs.lib()
    dev = torch.device("cuda:0")
    cfg = sd.CONFIGS[args.config]
    if args.reuse is not None:
        cfg = dataclasses.replace(cfg, n_reuse=args.reuse)
    also = args.also_density
    if also is None and args.config == "hunyuan720p_25":
        also = 15
    B, H, nv, n_pad, d, C, k = cfg.batch, cfg.heads, cfg.n_valid, cfg.n_pad, cfg.head_dim, cfg.group_size, cfg.topk
    sc = cfg.scale
    n_inputs = max(1, min(args.reuse_inputs, cfg.n_reuse))
    t_gen = time.perf_counter()
    steps_cpu = sd.generate(cfg, steps=1 + n_inputs)
    print(f"# generated the anchor and {n_inputs} reuse-step inputs of {cfg.name} in "
          f"{time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    steps = [tuple(t.to(dev) for t in s) for s in steps_cpu]
    q0, k0, v0 = steps[0]
    reuse_in = [steps[1 + i % n_inputs] for i in range(cfg.n_reuse)]
    dims = mcs.make_dims(B, H, nv, n_pad, d, C)
    G = cfg.groups
    perm = torch.empty((B, H, n_pad), dtype=torch.int32, device=dev)
    o_full = torch.empty_like(q0)
    lse = torch.empty((B, H, n_pad), dtype=torch.float32, device=dev)
    kv = torch.empty((B, H, G, k), dtype=torch.int32, device=dev)
    r = torch.empty_like(q0)
    outs = [torch.empty_like(q0) for _ in range(n_inputs)]
    ws_g = torch.empty(mcs.group_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(mcs.anchor_select_workspace_bytes(dims, k), dtype=torch.uint8, device=dev)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    stage_names = ["group", "anchor_select", "residual", "sparse_attn"]

    def one_step(record):
        marks = []
        e = ev(); e.record(); marks.append(e)
        mcs.group(q0, nv, C, cfg.power_iters, perm=perm, workspace=ws_g)
        e = ev(); e.record(); marks.append(e)
        mcs.anchor_select(q0, k0, v0, perm, nv, C, k, sc, o_full=o_full, lse=lse, kv_idx=kv, workspace=ws_a)
        e = ev(); e.record(); marks.append(e)
        mcs.residual(q0, k0, v0, perm, kv, o_full, nv, C, sc, r=r)
        e = ev(); e.record(); marks.append(e)
        for i, (qt, kt, vt) in enumerate(reuse_in):
            mcs.sparse_attn(qt, kt, vt, perm, kv, r, nv, C, sc, o=outs[i % n_inputs])
            e = ev(); e.record(); marks.append(e)
        record.append(marks)

    if args.only == "copy":
        # profiling helper: a plain 1 GiB device copy, to calibrate the HBM
        # byte counters against a kernel of known traffic
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# ran {args.steps} x 1 GiB copy", file=sys.stderr)
        return
    if args.only:
        # profiling helper: warm up the metadata, then loop one call
        one_step([])
        torch.cuda.synchronize()
        for _ in range(args.steps):
            if args.only == "sparse":
                mcs.sparse_attn(*steps[1], perm, kv, r, nv, C, sc, o=outs[0])
            elif args.only == "group":
                mcs.group(q0, nv, C, cfg.power_iters, perm=perm, workspace=ws_g)
            elif args.only == "dense":
                mcs.dense_attn(q0, k0, v0, nv, C, sc, o=o_full, lse=lse)
            else:
                mcs.anchor_select(q0, k0, v0, perm, nv, C, k, sc, o_full=o_full, lse=lse, kv_idx=kv, workspace=ws_a)
        torch.cuda.synchronize()
        print(f"# ran {args.steps} x {args.only}", file=sys.stderr)
        return

    for _ in range(args.warmup):
        one_step([])
    torch.cuda.synchronize()
    print(f"# warm-up done ({args.warmup} steps)", file=sys.stderr, flush=True)
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    stage_ms = {n: [] for n in stage_names}
    for marks in recs:
        stage_ms["group"].append(marks[0].elapsed_time(marks[1]))
        stage_ms["anchor_select"].append(marks[1].elapsed_time(marks[2]))
        stage_ms["residual"].append(marks[2].elapsed_time(marks[3]))
        for i in range(3, len(marks) - 1):
            stage_ms["sparse_attn"].append(marks[i].elapsed_time(marks[i + 1]))
    t_sparse_ms = statistics.mean(stage_ms["sparse_attn"])
    sparse_flops = 4.0 * B * H * n_pad * k * d
    eff_tflops = sparse_flops / (t_sparse_ms * 1e-3) / 1e12
    print(f"# step {ms_per_step:.2f} ms; stages (ms): " +
          ", ".join(f"{n} {statistics.mean(v):.3f}" for n, v in stage_ms.items()), file=sys.stderr, flush=True)

    # sanity: the reuse outputs are finite and padded rows are zero
    for o in outs:
        assert torch.isfinite(o.float()).all().item()
        assert (o[:, :, nv:] == 0).all().item()

    # dense vs sparse at the same shape.  Every timed call is preceded by a
    # read of a 512 MiB buffer that evicts L2 / MALL (a read, so no dirty
    # lines are written back during the timed kernel).  Headline protocol:
    # each kernel in its own steady state, i.e. a stream of back-to-back calls
    # of about the same length for both (n_d dense calls, n_d*N/k sparse
    # calls), in the order dense, sparse, sparse, dense; per-call medians.
    # Secondary protocol (reported beside it): single calls alternating
    # dense / sparse, where every sparse call starts right after a dense call
    # several times longer and inherits its lowered clock.
    flush = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
    q1, k1, v1 = steps[1]
    o_d = torch.empty_like(q0)

    def ratio(kv_sel, r_sel, topk):
        def call(which):
            if which == "dense":
                mcs.dense_attn(q1, k1, v1, nv, C, sc, o=o_d, want_lse=False)
            else:
                mcs.sparse_attn(q1, k1, v1, perm, kv_sel, r_sel, nv, C, sc, o=outs[0])

        def stream(which, n):
            marks = []
            for _ in range(n):
                flush.sum()
                a, b = ev(), ev()
                a.record()
                call(which)
                b.record()
                marks.append((a, b))
            torch.cuda.synchronize()
            return [a.elapsed_time(b) for a, b in marks]

        density = topk / nv
        n_d = max(2, args.ratio_reps // 2)
        n_s = max(2, round(n_d / density))
        t_d, t_s = [], []
        for which in ("dense", "sparse", "sparse", "dense"):
            (t_d if which == "dense" else t_s).extend(stream(which, n_d if which == "dense" else n_s))
        td, ts = statistics.median(t_d), statistics.median(t_s)
        a_d, a_s = [], []
        for _ in range(args.ratio_reps):
            a_d.extend(stream("dense", 1))
            a_s.extend(stream("sparse", 1))
        return {"density": density, "td": td, "ts": ts, "frac": density * td / ts,
                "frac_alt": density * statistics.median(a_d) / statistics.median(a_s),
                "td_min": min(t_d), "ts_min": min(t_s), "n_d": n_d, "n_s": n_s}

    rt = ratio(kv, r, k)
    td, ts = rt["td"], rt["ts"]
    dense_flops = 4.0 * B * H * n_pad * nv * d
    dense_tflops = dense_flops / (td * 1e-3) / 1e12
    print(f"# ratio protocol at {cfg.density_pct}%: dense {td:.3f} ms, sparse {ts:.3f} ms, "
          f"ideal-1/s fraction {rt['frac']:.4f}", file=sys.stderr, flush=True)

    # the same layer at a second density: a second selection on the same
    # inputs and groups, its residual, its reuse-step sparse attention
    second = None
    if also:
        k2 = (nv * also + 99) // 100
        kv2 = torch.empty((B, H, G, k2), dtype=torch.int32, device=dev)
        r2 = torch.empty_like(q0)
        t_sel, t_res, t_sp = [], [], []
        for rep in range(1 + args.steps):
            m = [ev() for _ in range(4)]
            m[0].record()
            mcs.anchor_select(q0, k0, v0, perm, nv, C, k2, sc, o_full=o_full, lse=lse, kv_idx=kv2, workspace=ws_a)
            m[1].record()
            mcs.residual(q0, k0, v0, perm, kv2, o_full, nv, C, sc, r=r2)
            m[2].record()
            mcs.sparse_attn(*steps[1], perm, kv2, r2, nv, C, sc, o=outs[0])
            m[3].record()
            torch.cuda.synchronize()
            if rep:
                t_sel.append(m[0].elapsed_time(m[1]))
                t_res.append(m[1].elapsed_time(m[2]))
                t_sp.append(m[2].elapsed_time(m[3]))
        rt2 = ratio(kv2, r2, k2)
        t2 = statistics.mean(t_sp)
        fl2 = 4.0 * B * H * n_pad * k2 * d
        second = {"density_pct": also, "topk": k2,
                  "sparse_ms_in_step": round(t2, 4),
                  "effective_tflops": round(fl2 / (t2 * 1e-3) / 1e12, 2),
                  "mfma_frac": round(fl2 / (t2 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "ideal_1_over_s_frac": round(rt2["frac"], 4),
                  "ideal_1_over_s_frac_alternating": round(rt2["frac_alt"], 4),
                  "dense_ms": round(rt2["td"], 4), "sparse_ms": round(rt2["ts"], 4),
                  "stage_ms": {"anchor_select": round(statistics.mean(t_sel), 4),
                               "residual": round(statistics.mean(t_res), 4)}}
        print(f"# second density {also}%: sparse {t2:.3f} ms in step, ideal-1/s fraction {rt2['frac']:.4f}",
              file=sys.stderr, flush=True)

    # torch's own fused attention at the same shape (valid tokens only), as a
    # sanity reference for the dense kernel; not a target
    sdpa_ms = None
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        qs, ks_, vs = q1[:, :, :nv], k1[:, :, :nv], v1[:, :, :nv]
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            torch.nn.functional.scaled_dot_product_attention(qs, ks_, vs, scale=sc)
            t_sd = []
            for _ in range(3):
                flush.sum()
                a, b = ev(), ev()
                a.record()
                torch.nn.functional.scaled_dot_product_attention(qs, ks_, vs, scale=sc)
                b.record()
                torch.cuda.synchronize()
                t_sd.append(a.elapsed_time(b))
        sdpa_ms = statistics.median(t_sd)
    except (RuntimeError, ImportError) as e:  # no fused backend for this shape / build
        print(f"# torch SDPA reference skipped: {e}", file=sys.stderr)

    kernel_hash = source_hash("attn.hip", "mcs_common.h")
    traffic = load_traffic(args.config, kernel_hash)
    kname = f"attn_kernel<{d},{C},1> (mcs_sparse_attn)"
    roofline = {"bound": "mfma", "achieved": round(eff_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(eff_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": kname,
                "flops_per_launch": sparse_flops, "avg_launch_ms": round(t_sparse_ms, 4),
                "kernel_src_hash": kernel_hash}
    # the HBM side of the same launch: L2-fill bytes per launch (the traffic
    # counters) over its time, against the 8 TB/s peak; and the rate at which
    # the kernel consumes gathered K/V rows (4 * k * (d + 1) bytes per group,
    # K and V rows plus the index), mostly served by L2 / MALL
    gathered = 4.0 * B * H * (n_pad // C) * k * (d + 1)
    hbm = {"gathered_bytes_per_launch": gathered,
           "gathered_GBps": round(gathered / (t_sparse_ms * 1e-3) / 1e9, 1)}
    if traffic is not None:
        gbps = traffic / (t_sparse_ms * 1e-3) / 1e9
        hbm.update({"traffic_GBps": round(gbps, 1), "hbm_peak_GBps": PEAK_HBM_GBS,
                    "hbm_frac": round(gbps / PEAK_HBM_GBS, 4)})

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, steps_cpu[1][0], steps_cpu[1][1], steps_cpu[1][2], perm, kv, args.cpu_seconds)

    anchor_ms = (statistics.mean(stage_ms["group"]) + statistics.mean(stage_ms["anchor_select"]) +
                 statistics.mean(stage_ms["residual"]))
    line = {
        "metric": "sparse-attn effective TFLOP/s + % of ideal 1/s speedup vs dense, at 15/25% density",
        "value": round(eff_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded clustered Q/K, Gaussian V; no model weights)",
        "config": {
            "workload": f"{cfg.name} video-DiT attention layer: B{B} H{H} N{nv}->{n_pad} d{d} C{C} "
                        f"density {cfg.density_pct}% (k={k}), 1 anchor + {cfg.n_reuse} reuse steps per step "
                        f"(reuse inputs cycle over {n_inputs} drifted draws)",
            "batch": B, "heads": H, "n_valid": nv, "n_pad": n_pad, "head_dim": d, "group_size": C,
            "topk": k, "density_pct": cfg.density_pct, "reuse_steps": cfg.n_reuse,
            "reuse_inputs": n_inputs, "power_iters": cfg.power_iters, "parallelism": "single GPU"},
        "ideal_1_over_s_frac": round(rt["frac"], 4),
        "ratio_protocol": f"steady-state streams ({2 * rt['n_d']} dense, {2 * rt['n_s']} sparse calls), "
                          "512 MiB cache-evicting read before each call, per-call medians",
        "dense_ms": round(td, 4),
        "sparse_ms": round(ts, 4),
        "ideal_1_over_s_frac_alternating": round(rt["frac_alt"], 4),
        "dense_ms_min": round(rt["td_min"], 4),
        "sparse_ms_min": round(rt["ts_min"], 4),
        "dense_tflops": round(dense_tflops, 2),
        "torch_sdpa_ms": None if sdpa_ms is None else round(sdpa_ms, 4),
        "dense_speedup_vs_torch_sdpa": None if sdpa_ms is None else round(sdpa_ms / td, 3),
        "dense_mfma_frac": round(dense_tflops / PEAK_BF16_TFLOPS, 4),
        "stage_ms": {n: round(statistics.mean(v), 4) for n, v in stage_ms.items()},
        # extra anchor work over a dense step, spread over the anchor's steps,
        # in units of the dense step (density-equivalent overhead)
        "anchor_overhead_ds": round((anchor_ms - td) / (cfg.n_reuse + 1) / td, 4),
        "second_density": second,
        "roofline": roofline,
        "sparse_hbm": hbm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
