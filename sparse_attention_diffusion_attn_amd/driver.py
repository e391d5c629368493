"""Multi-step, multi-layer driver: anchor refresh schedule, per-layer metadata
cache, and offload of inactive layers' metadata to pinned host memory with a
prefetch one layer ahead.

The onedev.kr summary ("what is different", "how it is used") alternates
anchor and reuse steps: an anchor is the last step of a dense warm-up or of a
refresh interval; every layer caches its query groups, KV indices and residual
at the anchor and reuses them until the next one.  When GPU memory is short,
inactive cache entries are offloaded to the CPU and prefetched one layer ahead
to hide the transfer ("how it is used", last paragraph; "assumptions and
limits").

Readings:
  R35  Schedule over n_steps: steps before the first anchor are dense; the
       first anchor is step `warmup` - 1 (the last warm-up step; step 0 when
       warmup = 0); after it an anchor recurs every `refresh` steps (never if
       refresh = 0); all other steps reuse the last anchor's metadata.
  R36  Offload keeps every layer's (perm, kv_idx, R) in pinned host memory and
       two device slots; layer l uses slot l % 2.  While layer l runs its
       sparse attention on the compute stream, layer l+1's entry (layer 0 of
       the next step after the last layer) is copied into the other slot on a
       copy stream; a slot is overwritten only after the layer that last used
       it has finished.  At an anchor the freshly written metadata goes back
       to the host on the copy stream.

All attention work runs in the library (mcs_group, mcs_anchor_select,
mcs_residual, mcs_sparse_attn, mcs_dense_attn); this module only orders calls,
copies and events.  Both streams have the default priority.

Usage: python -m sparse_attention_diffusion_attn_amd.driver [--config 480p]
       [--layers 8] [--steps 6]                      offload vs resident
       python -m sparse_attention_diffusion_attn_amd.driver --schedule
       [--config 480p] [--n-steps 50] [--warmup 10] [--refresh 0,20,10]
                                                     a whole denoising run
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time
from typing import List, Optional

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import sparse_attention_diffusion_attn_amd as mcs  # noqa: E402


class Schedule:
    """Kind of every denoising step (R35): 'dense', 'anchor' or 'reuse'."""

    def __init__(self, n_steps: int, warmup: int, refresh: int):
        if n_steps < 1 or warmup < 0 or refresh < 0:
            raise ValueError("n_steps >= 1, warmup >= 0, refresh >= 0")
        self.n_steps, self.warmup, self.refresh = n_steps, warmup, refresh
        self.first_anchor = max(warmup - 1, 0)

    def kind(self, step: int) -> str:
        if step < self.first_anchor:
            return "dense"
        off = step - self.first_anchor
        if off == 0 or (self.refresh > 0 and off % self.refresh == 0):
            return "anchor"
        return "reuse"

    def kinds(self) -> List[str]:
        return [self.kind(s) for s in range(self.n_steps)]


@dataclasses.dataclass
class LayerShape:
    batch: int
    heads: int
    n_valid: int
    n_pad: int
    head_dim: int
    group_size: int
    topk: int

    @property
    def groups(self) -> int:
        return self.n_pad // self.group_size

    def entry_bytes(self) -> int:
        b, h = self.batch, self.heads
        return b * h * (self.n_pad * 4 + self.groups * self.topk * 4 + self.n_pad * self.head_dim * 2)


class MetadataStore:
    """Per-layer (perm, kv_idx, R), resident on the device or offloaded (R36).

    Offloaded, every device slot carries two events: `copied`, recorded on the
    copy stream after the last copy that read or wrote the slot, and `used`,
    recorded on the compute stream after the last kernel that read or wrote
    it.  Compute waits for `copied` before touching a slot; the copy stream
    waits for `used` before writing a slot and for the anchor's kernels before
    reading one back."""

    def __init__(self, n_layers: int, shape: LayerShape, offload: bool, device="cuda:0"):
        self.n, self.s, self.offload, self.dev = n_layers, shape, offload, torch.device(device)
        b, h, n_pad, d, G, k = shape.batch, shape.heads, shape.n_pad, shape.head_dim, shape.groups, shape.topk

        def alloc(where, pin=False):
            kw = dict(device=where, pin_memory=pin) if where == "cpu" else dict(device=where)
            return (torch.empty((b, h, n_pad), dtype=torch.int32, **kw),
                    torch.empty((b, h, G, k), dtype=torch.int32, **kw),
                    torch.empty((b, h, n_pad, d), dtype=torch.bfloat16, **kw))

        if offload:
            self.host = [alloc("cpu", pin=True) for _ in range(n_layers)]
            self.slots = [alloc(self.dev) for _ in range(2)]
            self.copy_stream = torch.cuda.Stream(device=self.dev)
            self.loaded = [None, None]     # layer whose entry each slot holds
            self.copied = [None, None]
            self.used = [None, None]
        else:
            self.resident = [alloc(self.dev) for _ in range(n_layers)]

    def _event(self, stream):
        ev = torch.cuda.Event()
        ev.record(stream)
        return ev

    def for_write(self, layer: int):
        """Device tensors the anchor of `layer` writes (its slot once every
        earlier copy of that slot is done)."""
        if not self.offload:
            return self.resident[layer]
        slot = layer % 2
        if self.copied[slot] is not None:
            torch.cuda.current_stream(self.dev).wait_event(self.copied[slot])
        self.loaded[slot] = layer
        return self.slots[slot]

    def after_anchor(self, layer: int) -> None:
        """The anchor wrote `layer`'s entry: copy it back to the host."""
        if not self.offload:
            return
        slot = layer % 2
        self.used[slot] = self._event(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(self.copy_stream):
            self.copy_stream.wait_event(self.used[slot])
            for src, dst in zip(self.slots[slot], self.host[layer]):
                dst.copy_(src, non_blocking=True)
            self.copied[slot] = self._event(self.copy_stream)

    def prefetch(self, layer: int) -> None:
        """Start copying `layer`'s entry into its slot (no-op if it is there)."""
        if not self.offload:
            return
        slot = layer % 2
        if self.loaded[slot] == layer:
            return
        with torch.cuda.stream(self.copy_stream):
            if self.used[slot] is not None:
                self.copy_stream.wait_event(self.used[slot])
            for src, dst in zip(self.host[layer], self.slots[slot]):
                dst.copy_(src, non_blocking=True)
            self.copied[slot] = self._event(self.copy_stream)
        self.loaded[slot] = layer

    def acquire(self, layer: int):
        """Device tensors of `layer`, the compute stream ordered after their
        transfer."""
        if not self.offload:
            return self.resident[layer]
        self.prefetch(layer)
        slot = layer % 2
        torch.cuda.current_stream(self.dev).wait_event(self.copied[slot])
        return self.slots[slot]

    def release(self, layer: int) -> None:
        """The compute stream is done with `layer`'s slot once it gets here."""
        if self.offload:
            self.used[layer % 2] = self._event(torch.cuda.current_stream(self.dev))


class Stack:
    """A stack of attention layers of one shape driven over a schedule.  Each
    layer has its own inputs per step from `inputs(layer, step)`."""

    def __init__(self, n_layers: int, shape: LayerShape, inputs, offload: bool, scale: float,
                 power_iters: int = 20, device="cuda:0"):
        self.n, self.s, self.inputs, self.scale = n_layers, shape, inputs, scale
        self.power_iters = power_iters
        self.store = MetadataStore(n_layers, shape, offload, device)
        s = shape
        dims = mcs.make_dims(s.batch, s.heads, s.n_valid, s.n_pad, s.head_dim, s.group_size)
        self.ws_g = torch.empty(mcs.group_workspace_bytes(dims), dtype=torch.uint8, device=device)
        self.ws_a = torch.empty(mcs.anchor_select_workspace_bytes(dims, s.topk), dtype=torch.uint8,
                                device=device)
        self.o_full = torch.empty((s.batch, s.heads, s.n_pad, s.head_dim), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((s.batch, s.heads, s.n_pad), dtype=torch.float32, device=device)

    def step(self, step: int, kind: str, outs: Optional[list] = None) -> None:
        s, st = self.s, self.store
        for layer in range(self.n):
            q, k, v = self.inputs(layer, step)
            o = outs[layer] if outs is not None else None
            if kind == "dense":
                mcs.dense_attn(q, k, v, s.n_valid, s.group_size, self.scale, o=o, want_lse=False)
            elif kind == "anchor":
                perm, kv, r = st.for_write(layer)
                mcs.group(q, s.n_valid, s.group_size, self.power_iters, perm=perm, workspace=self.ws_g)
                mcs.anchor_select(q, k, v, perm, s.n_valid, s.group_size, s.topk, self.scale,
                                  o_full=self.o_full, lse=self.lse, kv_idx=kv, workspace=self.ws_a)
                mcs.residual(q, k, v, perm, kv, self.o_full, s.n_valid, s.group_size, self.scale, r=r)
                if o is not None:
                    o.copy_(self.o_full)
                st.after_anchor(layer)
            else:
                perm, kv, r = st.acquire(layer)
                mcs.sparse_attn(q, k, v, perm, kv, r, s.n_valid, s.group_size, self.scale, o=o)
                st.release(layer)
                # prefetch the next layer of this step, or layer 0 of the next
                st.prefetch((layer + 1) % self.n)

    def run(self, schedule: Schedule, outs_per_step: Optional[list] = None) -> None:
        for step, kind in enumerate(schedule.kinds()):
            self.step(step, kind, None if outs_per_step is None else outs_per_step[step])


def schedule_run(cfg, n_steps: int, warmup: int, refreshes, dev="cuda:0"):
    """One layer over whole denoising schedules: per-kind step times, the
    effective density (attention time / that of all-dense steps) and the
    anchor overhead spread over the run (R23 over a schedule)."""
    import synthdata as sd
    shape = LayerShape(cfg.batch, cfg.heads, cfg.n_valid, cfg.n_pad, cfg.head_dim, cfg.group_size, cfg.topk)
    (q0, k0, v0), (q1, k1, v1) = [tuple(t.to(dev) for t in s) for s in sd.generate(cfg, steps=2)]
    inputs = lambda layer, step: (q0, k0, v0) if step % 2 == 0 else (q1, k1, v1)  # noqa: E731
    stack = Stack(1, shape, inputs, False, cfg.scale, cfg.power_iters, dev)
    o = [torch.empty_like(q0)]
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(kind, reps):
        ts = []
        for r in range(reps + 1):
            a, b = ev(), ev()
            a.record()
            stack.step(r, kind, o)
            b.record()
            torch.cuda.synchronize()
            if r:
                ts.append(a.elapsed_time(b))
        return sum(ts) / len(ts)

    t = {"dense": timed("dense", 3), "anchor": timed("anchor", 2), "reuse": timed("reuse", 5)}
    rows = []
    for r in refreshes:
        kinds = Schedule(n_steps, warmup, r).kinds()
        total = sum(t[k] for k in kinds)
        n_anchor = kinds.count("anchor")
        rows.append({
            "n_steps": n_steps, "warmup": warmup, "refresh": r, "anchors": n_anchor,
            "dense_steps": kinds.count("dense"), "reuse_steps": kinds.count("reuse"),
            "ms_total": round(total, 2), "ms_all_dense": round(n_steps * t["dense"], 2),
            "speedup_vs_dense": round(n_steps * t["dense"] / total, 3),
            # anchors beyond the dense step they replace, in dense-step units per step
            "delta_s": round(n_anchor * (t["anchor"] - t["dense"]) / t["dense"] / n_steps, 4),
        })
    return {k: round(v, 3) for k, v in t.items()}, rows


def main():
    import synthdata as sd
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="480p")
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--steps", type=int, default=6, help="reuse steps timed after one anchor")
    ap.add_argument("--schedule", action="store_true", help="time whole denoising schedules")
    ap.add_argument("--n-steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--refresh", default="0,20,10")
    args = ap.parse_args()
    assert torch.cuda.is_available(), "the driver runs on the GPU"
    mcs.lib()
    cfg = sd.CONFIGS[args.config]
    if args.schedule:
        t, rows = schedule_run(cfg, args.n_steps, args.warmup, [int(x) for x in args.refresh.split(",")])
        print(json.dumps({"workload": f"{args.config} attention layer, whole schedules",
                          "density_pct": cfg.density_pct, "ms_per_step": t, "schedules": rows}))
        return
    dev = "cuda:0"
    shape = LayerShape(cfg.batch, cfg.heads, cfg.n_valid, cfg.n_pad, cfg.head_dim, cfg.group_size, cfg.topk)
    (q0, k0, v0), (q1, k1, v1) = [tuple(t.to(dev) for t in s) for s in sd.generate(cfg, steps=2)]
    inputs = lambda layer, step: (q0, k0, v0) if step == 0 else (q1, k1, v1)  # noqa: E731
    sched = Schedule(1 + args.steps, warmup=1, refresh=0)
    o = torch.empty_like(q0)
    res = {}
    for offload in (False, True):
        stack = Stack(args.layers, shape, inputs, offload, cfg.scale, cfg.power_iters, dev)
        stack.step(0, "anchor")                    # metadata of every layer
        stack.step(1, "reuse", [o] * args.layers)  # warm the prefetch path
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for st in range(args.steps):
            stack.step(1 + st, "reuse", [o] * args.layers)
        torch.cuda.synchronize()
        res["offload" if offload else "resident"] = (time.perf_counter() - t0) * 1e3 / (args.steps * args.layers)
        del stack
        torch.cuda.empty_cache()
    # one layer's entry host -> device alone
    ent = MetadataStore(1, shape, True, dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(3):
        for src, dst in zip(ent.host[0], ent.slots[0]):
            dst.copy_(src, non_blocking=True)
    ev1.record()
    torch.cuda.synchronize()
    t_copy = ev0.elapsed_time(ev1) / 3
    line = {
        "workload": f"{args.config} attention layer stack: {args.layers} layers, "
                    f"{args.steps} reuse steps after one anchor",
        "entry_bytes_per_layer": shape.entry_bytes(),
        "ms_per_layer_resident": round(res["resident"], 3),
        "ms_per_layer_offload_prefetch": round(res["offload"], 3),
        "ms_h2d_per_layer_alone": round(t_copy, 3),
        "h2d_GBps": round(shape.entry_bytes() / t_copy / 1e6, 1),
        "transfer_hidden_frac": round(max(0.0, min(1.0, 1.0 - (res["offload"] - res["resident"]) / t_copy)), 3),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
