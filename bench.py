"""Benchmark: column-wise-mask (FlashMask) attention forward + backward on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
fm_tile_bounds -> fm_bwd_plan -> fm_fwd -> fm_bwd_ds (the backward that forms dQ from stored dS tiles; the
workspace for them is sized once from the plan before timing). With --bwd recompute the step is
fm_tile_bounds -> fm_fwd -> fm_bwd instead; with --schedule, fm_tile_schedule runs after the bounds and
the kernels launch in its order. The metric counts only unmasked FLOPs:
    FLOP per step = 14 * d * U   (forward 4 d U: Q K^T and P V; backward 10 d U: the S recompute,
                                  dP, dV, dK and dQ products), U = unmasked (query, key) pairs.
The default workload is the long-context configuration with a causal document mask (B=1, H=8,
N=131072, d=128, bf16; document lengths log-uniform in [1K, 32K]), the largest head-dim-128 workload.

Prints one JSON line. Options: --gpus (must be 1), --steps, --warmup, --workload, --no-cpu-baseline,
--schedule, --bwd {stored, recompute},
--sweep (also time every (config, mask) workload a few steps each with both backward forms, the
context-parallel rank shares, key compaction and the hash workloads, reported under "sweep"; with
--records FILE one JSON line per (config, mask) workload is written there, and --parity FILE merges the
whole-tensor parity errors and oracle timings that the full-size GPU tests write),
--copy-calibration (after timing, one 1 GiB device-to-device copy, the reference kernel for scaling
hardware byte counters in profiling runs).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "FlashMask fwd+bwd TFLOP/s (unmasked FLOPs) bf16 hd128; % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)

WORKLOADS = {
    "sft_packing_causal_document": (2, "causal_document"),
    "sft_packing_causal_window_1024": (2, "causal_window_1024"),
    "dpo_rm_share_question": (3, "share_question"),
    "dpo_rm_prefix_lm": (3, "prefix_lm"),
    "dpo_rm_causal_key_drop": (3, "causal_key_drop"),
    "long_context_causal_document": (4, "causal_document"),
    "long_context_causal_document_window_4096": (4, "causal_document_window_4096"),
    "long_context_causal_document_block_sparse": (4, "causal_document_block_sparse"),
    "bert_base_full": (1, "full"),
    "bert_base_causal": (1, "causal"),
}
DEFAULT_WORKLOAD = "long_context_causal_document"
ROOFLINE_KERNEL = "fm_bwd"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fm_bwd_ds_long_context_causal_document_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "mask_aware_exact_amd", "csrc", f)
                  for f in ("fm_common.h", "fm_launch.h", "fm_bwd.hip", "fm_dstore.hip")]


def kernel_source_digest() -> str:
    """Digest of the measured kernels' code: the sources with comments and whitespace removed, so that a
    comment edit keeps the recorded counters valid while any code change invalidates them."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, call: str = "fm_bwd_ds"):
    """HBM bytes per backward call from the committed counter summary, or None when that summary is
    missing, covers another workload or call, or was taken from other kernel sources."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and line.startswith("- "):
                    k, v = line[2:].split(":", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get("workload") != workload or fields.get("kernel_source_digest") != kernel_source_digest():
            return None
        if fields.get("call", "fm_bwd") != call:
            return None
        return int(float(fields["hbm_bytes_per_call"]))
    except (OSError, KeyError, ValueError):
        return None


def unmasked_pairs(spec: W.MaskSpec, H: int, rows=None) -> int:
    """U by per-column interval union (inclusion-exclusion over at most three intervals), over all query
    rows or over the row block rows = (a, b)."""
    N = spec.N
    ra, rb = (0, N) if rows is None else rows
    j = np.arange(N, dtype=np.int64)
    zero = np.zeros(N, dtype=np.int64)
    total = 0
    for b in range(spec.B):
        for hm in range(spec.Hm):
            ivs = [(zero, j) if spec.causal else (zero, zero)]
            for s, e in ((spec.lts, spec.lte), (spec.uts, spec.ute)):
                if s is None:
                    ivs.append((zero, zero))
                else:
                    s_ = np.clip(s[b, hm].astype(np.int64), 0, N)
                    e_ = np.maximum(np.clip(e[b, hm].astype(np.int64), 0, N), s_)
                    ivs.append((s_, e_))

            def ln(a):
                return np.maximum(a[1] - a[0], 0)

            def meet(a, c):
                return np.maximum(a[0], c[0]), np.minimum(a[1], c[1])

            blk = (np.full(N, ra, np.int64), np.full(N, rb, np.int64))
            A, Bv, Cv = (meet(x, blk) for x in ivs)
            union = ln(A) + ln(Bv) + ln(Cv) - ln(meet(A, Bv)) - ln(meet(A, Cv)) - ln(meet(Bv, Cv)) \
                + ln(meet(meet(A, Bv), Cv))
            total += ((rb - ra) * N - int(union.sum())) * (H if spec.Hm == 1 else 1)
    return total


class Workload:
    def __init__(self, name: str, device, cfg_mask=None):
        import torch
        cfg_idx, mask = WORKLOADS[name] if cfg_mask is None else cfg_mask
        cfg = W.CONFIGS[cfg_idx]
        self.name, self.cfg, self.mask = name, cfg, mask
        self.B, self.H, self.N, self.d = cfg.B, cfg.H, cfg.N, cfg.d
        mi = cfg.masks.index(mask) if mask in cfg.masks else 0
        self.spec = W.make_mask(cfg.index, mask, cfg.B, cfg.H, cfg.N, mi)
        self.mask_index = mi
        q, k, v, do = W.make_tensors(cfg.index, mi, cfg.B, cfg.H, cfg.N, cfg.d)
        self.host = (q, k, v, do)
        to = lambda x: torch.from_numpy(x).to(device=device).to(torch.bfloat16)  # noqa: E731
        self.q, self.k, self.v, self.do = (to(x) for x in (q, k, v, do))
        self.vecs = [None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device)
                     for x in self.spec.vectors()]
        self.has_vecs = any(x is not None for x in self.vecs)
        self.scale = 1.0 / math.sqrt(self.d)
        self.U = unmasked_pairs(self.spec, self.H)
        self.flop_fwd = 4.0 * self.d * self.U
        self.flop_bwd = 10.0 * self.d * self.U
        self.flop = self.flop_fwd + self.flop_bwd


def unmasked_per_row(spec: W.MaskSpec, H: int) -> np.ndarray:
    """int64 [N]: unmasked (row, key) pairs of each query row, summed over the H heads. Per column the
    masked rows are the union of up to three intervals (causal [0, j), LT, UT); inclusion-exclusion over
    them, accumulated as +-1 steps in a difference array over the rows, gives every row's masked count."""
    N = spec.N
    j = np.arange(N, dtype=np.int64)
    zero = np.zeros(N, dtype=np.int64)
    total = np.zeros(N, dtype=np.int64)
    for b in range(spec.B):
        for hm in range(spec.Hm):
            ivs = [(zero, j if spec.causal else zero)]
            for s_, e_ in ((spec.lts, spec.lte), (spec.uts, spec.ute)):
                if s_ is None:
                    ivs.append((zero, zero))
                else:
                    lo = np.clip(s_[b, hm].astype(np.int64), 0, N)
                    ivs.append((lo, np.maximum(np.clip(e_[b, hm].astype(np.int64), 0, N), lo)))

            def meet(x, y):
                return np.maximum(x[0], y[0]), np.minimum(x[1], y[1])

            A, Bv, Cv = ivs
            diff = np.zeros(N + 1, dtype=np.int64)
            for (lo, hi), w in ((A, 1), (Bv, 1), (Cv, 1), (meet(A, Bv), -1), (meet(A, Cv), -1), (meet(Bv, Cv), -1),
                                (meet(meet(A, Bv), Cv), 1)):
                ok = hi > lo
                np.add.at(diff, lo[ok], w)
                np.add.at(diff, hi[ok], -w)
            masked = np.cumsum(diff[:N])
            total += (N - masked) * (H if spec.Hm == 1 else 1)
    return total


def balanced_row_blocks(spec: W.MaskSpec, H: int, ranks: int, align: int = 128):
    """Row-block boundaries that give each rank about the same number of unmasked pairs (the load-balancing
    goal of the FlashMask-3 summary's balancer, on one GPU's row blocks), rounded to `align` rows."""
    cum = np.cumsum(unmasked_per_row(spec, H))
    cuts = [0]
    for r in range(1, ranks):
        c = int(np.searchsorted(cum, cum[-1] * r / ranks))
        c = int(round(c / align)) * align
        cuts.append(min(max(c, cuts[-1]), spec.N))
    cuts.append(spec.N)
    return cuts


def stored_default(d: int) -> bool:
    """The backward the bench times: stored dS tiles (fm_bwd_ds) at head dim 128, the recomputing fm_bwd at
    head dim 64, where the dS bytes (2 per pair at any d) cost more than the halved recompute they save
    (measured on MI355X: 8-10% slower on the BERT-like workloads)."""
    return d >= 128


def time_workload(fm, wl: Workload, steps: int, warmup: int, use_sched: bool = False, stored: bool = True):
    """One step = fm_tile_bounds (when the mask has vectors), fm_tile_schedule (longest-first dispatch
    order, only with use_sched), then with `stored` fm_bwd_plan, fm_fwd and fm_bwd_ds (dQ from stored dS
    tiles, workspace sized once from the plan before timing), else fm_fwd and fm_bwd (dQ recomputed); all
    of it timed. Returns the wall time of the timed steps, the mean per-part milliseconds (bounds,
    schedule, plan, fwd, bwd) and a finiteness flag."""
    import torch
    dev = wl.q.device
    stream = torch.cuda.current_stream(dev)
    B, H, Hm, N, d = wl.B, wl.H, wl.spec.Hm, wl.N, wl.d
    bounds = torch.empty(fm.fm_bounds_elems(B, Hm, N) or 8, dtype=torch.int32, device=dev)
    sched_buf = torch.empty(fm.fm_schedule_elems(B, Hm, N, N), dtype=torch.int32, device=dev)
    out = torch.empty_like(wl.q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(wl.q), torch.empty_like(wl.k), torch.empty_like(wl.v)
    plan = None
    if stored:
        b0 = fm.fm_tile_bounds(*wl.vecs, B, Hm, N, bounds=bounds) if wl.has_vecs else None
        plan = fm.fm_bwd_plan(b0, B, H, Hm, N, wl.spec.causal, device=dev)
        ws_bytes = fm.fm_bwd_ds_workspace_bytes(torch.bfloat16, B, H, N, d, fm.plan_tiles(plan))
    else:
        ws_bytes = fm.fm_bwd_workspace_bytes(torch.bfloat16, B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        b = None
        if wl.has_vecs:
            b = fm.fm_tile_bounds(*wl.vecs, B, Hm, N, bounds=bounds)
        if evs is not None:
            evs[1].record(stream)
        sc = None
        if use_sched:
            sc = fm.fm_tile_schedule(b, B, Hm, N, N, wl.spec.causal, sched=sched_buf)
        if evs is not None:
            evs[2].record(stream)
        if stored:
            fm.fm_bwd_plan(b, B, H, Hm, N, wl.spec.causal, plan=plan)
        if evs is not None:
            evs[3].record(stream)
        fm.fm_fwd(wl.q, wl.k, wl.v, *wl.vecs, bounds=b, sched=sc, causal=wl.spec.causal, scale=wl.scale, out=out,
                  lse=lse)
        if evs is not None:
            evs[4].record(stream)
        if stored:
            fm.fm_bwd_ds(wl.q, wl.k, wl.v, out, wl.do, lse, plan, *wl.vecs, bounds=b, sched=sc,
                         causal=wl.spec.causal, scale=wl.scale, dq=dq, dk=dk, dv=dv, workspace=ws)
        else:
            fm.fm_bwd(wl.q, wl.k, wl.v, out, wl.do, lse, *wl.vecs, bounds=b, sched=sc, causal=wl.spec.causal,
                      scale=wl.scale, dq=dq, dk=dk, dv=dv, workspace=ws)
        if evs is not None:
            evs[5].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    parts = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(5)] for e in events])  # ms
    ok = bool(torch.isfinite(out.float()).all() and torch.isfinite(dq.float()).all()
              and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all())
    del ws
    return wall, parts.mean(axis=0), ok


def bounds_bytes(B: int, Hm: int, N: int, nvec: int) -> int:
    """Algorithmic HBM bytes of one fm_tile_bounds call: every vector element read once, 32 bytes of
    bounds written per 64-column key tile."""
    return 4 * nvec * B * Hm * N + 32 * B * Hm * ((N + 63) // 64)


def time_bounds(fm, B: int, Hm: int, N: int, dev, reps: int = 20):
    """Mean fm_tile_bounds time (ms, HIP events on the launch stream) on four seeded vectors of
    [B, Hm, N] with values in [0, N]."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    vecs = [torch.randint(0, N + 1, (B, Hm, N), dtype=torch.int32, device=dev, generator=g) for _ in range(4)]
    out = torch.empty(fm.fm_bounds_elems(B, Hm, N), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(3):
        fm.fm_tile_bounds(*vecs, B, Hm, N, bounds=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fm.fm_tile_bounds(*vecs, B, Hm, N, bounds=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del vecs, out
    return ms


def time_workload_compacted(fm, wl: Workload, steps: int, warmup: int):
    """The same step through key compaction: fm_compact_keys, fm_gather_rows (K, V), fm_tile_bounds,
    fm_fwd and fm_bwd without the causal flag, fm_gather_rows (dK, dV back). All of it is timed."""
    import torch
    dev = wl.q.device
    Hm = wl.spec.Hm
    dk, dv = torch.empty_like(wl.k), torch.empty_like(wl.v)
    ws = torch.empty(fm.fm_bwd_workspace_bytes(torch.bfloat16, wl.B, wl.H, wl.N, wl.d), dtype=torch.uint8,
                     device=dev)
    bounds = torch.empty(fm.fm_bounds_elems(wl.B, Hm, wl.N), dtype=torch.int32, device=dev)
    k2, v2 = torch.empty_like(wl.k), torch.empty_like(wl.v)
    out = torch.empty_like(wl.q)
    lse = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device=dev)
    dq, dk2, dv2 = torch.empty_like(wl.q), torch.empty_like(wl.k), torch.empty_like(wl.v)

    def step():
        kidx, kpos, counts, vecs2 = fm.fm_compact_keys(*wl.vecs, wl.B, Hm, wl.N, wl.spec.causal)
        fm.fm_gather_rows(wl.k, kidx, y=k2)
        fm.fm_gather_rows(wl.v, kidx, y=v2)
        b = fm.fm_tile_bounds(*vecs2, wl.B, Hm, wl.N, bounds=bounds)
        fm.fm_fwd(wl.q, k2, v2, *vecs2, bounds=b, causal=False, scale=wl.scale, out=out, lse=lse)
        fm.fm_bwd(wl.q, k2, v2, out, wl.do, lse, *vecs2, bounds=b, causal=False, scale=wl.scale, dq=dq, dk=dk2,
                  dv=dv2, workspace=ws)
        fm.fm_gather_rows(dk2, kpos, y=dk)
        fm.fm_gather_rows(dv2, kpos, y=dv)
        return counts

    for _ in range(warmup):
        counts = step()
    torch.cuda.synchronize()
    ok = int(counts.min()) >= 0
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, ok


def time_rows(fm, wl: Workload, a: int, b: int, steps: int, warmup: int):
    """fm_fwd_rows + fm_bwd_rows of the query rows [a, b) against all keys: one rank's share under
    context parallelism, at its real shape."""
    import torch
    q = wl.q[:, :, a:b].contiguous()
    do = wl.do[:, :, a:b].contiguous()
    bounds = fm.fm_tile_bounds(*wl.vecs, wl.B, wl.spec.Hm, wl.N) if wl.has_vecs else None
    out = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, b - a), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(wl.k), torch.empty_like(wl.v)
    ws = torch.empty(fm.fm_bwd_workspace_bytes(torch.bfloat16, wl.B, wl.H, b - a, wl.d), dtype=torch.uint8,
                     device=q.device)

    def step():
        fm.fm_fwd_rows(q, wl.k, wl.v, a, *wl.vecs, bounds=bounds, causal=wl.spec.causal, scale=wl.scale, out=out,
                       lse=lse)
        fm.fm_bwd_rows(q, wl.k, wl.v, out, do, lse, a, *wl.vecs, bounds=bounds, causal=wl.spec.causal,
                       scale=wl.scale, dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


class HashWorkload:
    """Hash-bucket attention at a configuration's shape: seeded Q, K, V, dO and one random rotation per
    head; the buckets come from the library's own hash inside the timed step."""

    def __init__(self, name: str, device):
        import torch
        cfg_idx, nb = W.HASH_WORKLOADS[name]
        cfg = W.CONFIGS[cfg_idx]
        self.name, self.cfg, self.nb = name, cfg, nb
        self.B, self.H, self.N, self.d = cfg.B, cfg.H, cfg.N, cfg.d
        host = W.make_tensors(cfg_idx, W.HASH_MASK_INDEX, cfg.B, cfg.H, cfg.N, cfg.d)
        to = lambda x: torch.from_numpy(x).to(device=device).to(torch.bfloat16)  # noqa: E731
        self.q, self.k, self.v, self.do = (to(x) for x in host)
        del host
        self.rot = torch.from_numpy(W.make_rotation(cfg_idx, W.HASH_MASK_INDEX, cfg.H, cfg.d, nb)).to(device)
        self.scale = 1.0 / math.sqrt(self.d)


def time_hash_workload(fm, wl: HashWorkload, steps: int, warmup: int, graph: bool = False):
    """One step: fm_lsh_buckets of Q and K, fm_bucket_sort, fm_gather_rows of Q, K, V, dO into bucket
    order, fm_tile_bounds, then fm_fwd_mapped and fm_bwd_mapped (no causal flag), which store out, dq, dk
    and dv straight into the original token order. All of it is timed. U is counted afterwards from the
    reordered problem's vectors. With `graph` the 12 launches of a step are captured once in a HIP graph
    and the timed steps are graph replays (the library allocates nothing and issues no memset, so the
    step replays as captured); the eager step is the workload's rate and the replay time is reported
    beside it."""
    import torch
    B, H, N = wl.B, wl.H, wl.N
    qs, ks, vs, dos = (torch.empty_like(x) for x in (wl.q, wl.k, wl.v, wl.do))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=wl.q.device)
    out, dq, dk, dv = (torch.empty_like(x) for x in (wl.q, wl.q, wl.k, wl.v))
    ws = torch.empty(fm.fm_bwd_workspace_bytes(torch.bfloat16, B, H, N, wl.d), dtype=torch.uint8,
                     device=wl.q.device)
    bounds = torch.empty(fm.fm_bounds_elems(B, H, N), dtype=torch.int32, device=wl.q.device)
    qb = torch.empty((B, H, N), dtype=torch.int32, device=wl.q.device)
    kb = torch.empty_like(qb)

    def step():
        fm.fm_lsh_buckets(wl.q, wl.rot, wl.nb, out=qb)
        fm.fm_lsh_buckets(wl.k, wl.rot, wl.nb, out=kb)
        qidx, qpos, kidx, kpos, vecs = fm.fm_bucket_sort(qb, kb, wl.nb)
        fm.fm_gather_rows(wl.q, qidx, y=qs)
        fm.fm_gather_rows(wl.do, qidx, y=dos)
        fm.fm_gather_rows(wl.k, kidx, y=ks)
        fm.fm_gather_rows(wl.v, kidx, y=vs)
        b = fm.fm_tile_bounds(*vecs, B, H, N, bounds=bounds)
        fm.fm_fwd_mapped(qs, ks, vs, qidx, *vecs, bounds=b, causal=False, scale=wl.scale, out=out, lse=lse)
        fm.fm_bwd_mapped(qs, ks, vs, out, dos, lse, qidx, kidx, *vecs, bounds=b, causal=False, scale=wl.scale,
                         dq=dq, dk=dk, dv=dv, workspace=ws)
        return vecs

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        ref = out.clone()  # the eager step's result, which every replay must reproduce
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise RuntimeError("graph replay of the hash step differs from the eager step")
        run = g.replay
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    ok = bool(torch.isfinite(out.float()).all() and torch.isfinite(dk.float()).all())
    # U from the reordered problem's vectors (untimed; the same buckets as every timed step)
    fm.fm_lsh_buckets(wl.q, wl.rot, wl.nb, out=qb)
    fm.fm_lsh_buckets(wl.k, wl.rot, wl.nb, out=kb)
    lts, _, _, ute = fm.fm_bucket_sort(qb, kb, wl.nb)[4]
    U = int(torch.clamp(lts.long() - ute.long(), min=0).sum())
    return dt, U, ok


def cpu_baseline(wl: Workload, budget_heads: int, max_tokens: int):
    """The oracle, as it stands, timed on a bounded sample of the same workload: the first heads and
    the first `max_tokens` tokens (for a causal mask the leading tokens form a closed sub-problem)."""
    import torch
    from oracle import attention as OA
    q, k, v, do = wl.host
    nh = min(wl.H, budget_heads)
    n = min(wl.N, max_tokens)
    r = lambda x: torch.from_numpy(np.ascontiguousarray(x[:1, :nh, :n])).to(torch.bfloat16).to(  # noqa: E731
        torch.float64).numpy()
    qs, ks, vs, dos = (r(x) for x in (q, k, v, do))
    hm = 1 if wl.spec.Hm == 1 else nh
    sub = W.MaskSpec(n, 1, hm, wl.spec.causal,
                     *[None if x is None else np.ascontiguousarray(x[:1, :hm, :n]) for x in wl.spec.vectors()])
    workers = min(nh, 16, os.cpu_count() or 1)
    t0 = time.perf_counter()
    _, _, _, _, _, used = OA.fwd_bwd(qs, ks, vs, dos, sub.vectors(), sub.causal, wl.scale, sub.Hm, workers=workers)
    dt = time.perf_counter() - t0
    U = unmasked_pairs(sub, nh)
    flop = 14.0 * wl.d * U
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "sample": f"heads 0..{nh - 1} of {wl.H}, tokens 0..{n - 1} of {wl.N} of {wl.name} "
                      f"(fp64 NumPy fwd+bwd, U={U}), {dt:.1f} s",
            "seconds": round(dt, 2), "cpu": platform.processor() or platform.machine()}


def prepass_record(fm, wl: Workload, bounds_ms: float, dev):
    """Achieved HBM rate of fm_tile_bounds (HBM-bound): on the workload's own vectors, where a ~1 MiB
    read leaves it launch-latency bound, and at B*Hm*N = 2^26 (1 GiB of four vectors) to show the
    bandwidth regime."""
    nvec = sum(v is not None for v in wl.vecs)
    rec = {"unit": "GB/s", "peak": PEAK_HBM_GBS}
    if nvec:
        b = bounds_bytes(wl.B, wl.spec.Hm, wl.N, nvec)
        rec["workload"] = {"vectors": nvec, "bytes": b, "ms": round(bounds_ms, 4),
                           "achieved": round(b / (bounds_ms * 1e-3) / 1e9, 1)}
    B, Hm, N = 1, 512, 131072  # 2^26 columns
    ms = time_bounds(fm, B, Hm, N, dev)
    b = bounds_bytes(B, Hm, N, 4)
    ach = b / (ms * 1e-3) / 1e9
    rec["2^26 columns (B=1, Hm=512, N=131072, four vectors)"] = {
        "bytes": b, "ms": round(ms, 4), "achieved": round(ach, 1), "frac": round(ach / PEAK_HBM_GBS, 4)}
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS) + sorted(W.HASH_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8)
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--schedule", action="store_true",
                    help="compute the longest-first dispatch schedule each step and launch in its order")
    ap.add_argument("--bwd", choices=("stored", "recompute"), default="stored",
                    help="backward: fm_bwd_ds (dQ from stored dS tiles, the default) or fm_bwd (dQ recomputed)")
    ap.add_argument("--records", default=None,
                    help="with --sweep: write one JSON line per (config, mask) workload to this file")
    ap.add_argument("--parity", default=None,
                    help="with --records: merge the whole-tensor parity results (JSON by workload) into the records")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mask_aware_exact_amd as fm
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fm.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.workload in W.HASH_WORKLOADS:
        hw = HashWorkload(args.workload, dev)
        t, U, okh = time_hash_workload(fm, hw, args.steps, args.warmup)
        te, _, _ = time_hash_workload(fm, hw, args.steps, args.warmup, graph=True)
        tfl = 14.0 * hw.d * U / t / 1e12
        print(json.dumps({
            "metric": METRIC, "value": round(tfl, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(t * 1e3, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": hw.name, "B": hw.B, "H": hw.H, "N": hw.N, "d": hw.d, "buckets": hw.nb,
                       "unmasked_pairs": U, "flop_formula": "14*d*U"},
            "pct_of_peak": round(100.0 * tfl / PEAK_BF16_TFLOPS, 2), "finite_outputs": okh,
            "launch": "eager", "ms_per_step_graph_replay": round(te * 1e3, 4)}),
            flush=True)
        return

    wl = Workload(args.workload, dev)
    use_sched = args.schedule
    stored = args.bwd == "stored" and stored_default(wl.d)
    wall, parts_ms, ok = time_workload(fm, wl, args.steps, args.warmup, use_sched, stored)
    ms_per_step = wall * 1e3 / args.steps
    tflops = wl.flop / (ms_per_step * 1e-3) / 1e12
    bwd_ms = float(parts_ms[4])
    bwd_tflops = wl.flop_bwd / (bwd_ms * 1e-3) / 1e12
    bwd_name = "fm_bwd_ds" if stored else "fm_bwd"
    bwd_kernels = ("fm_bwd_ds (bwd_dq_kernel forming D only, bwd_dkdv_pair_kernel storing dS, dq_stream_kernel)"
                   if stored else "fm_bwd (bwd_dq_kernel then bwd_dkdv_pair_kernel)")
    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d, "mask": wl.mask,
                   "causal": bool(wl.spec.causal), "unmasked_pairs": int(wl.U),
                   "flop_per_step": wl.flop, "flop_formula": "14*d*U"},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "peak_tflops_used": PEAK_BF16_TFLOPS,
        "schedule": "longest-first" if use_sched else "default order",
        "backward": "stored dS (fm_bwd_plan + fm_bwd_ds)" if stored else "recomputed dQ (fm_bwd)",
        "parts_ms": {"fm_tile_bounds": round(float(parts_ms[0]), 4),
                     "fm_tile_schedule": round(float(parts_ms[1]), 4) if use_sched else None,
                     "fm_bwd_plan": round(float(parts_ms[2]), 4) if stored else None,
                     "fm_fwd": round(float(parts_ms[3]), 4),
                     bwd_name: round(bwd_ms, 4)},
        "parts_tflops": {"fm_fwd": round(wl.flop_fwd / (parts_ms[3] * 1e-3) / 1e12, 2),
                         bwd_name: round(bwd_tflops, 2)},
        "finite_outputs": ok,
        "prepass": prepass_record(fm, wl, float(parts_ms[0]), dev),
        "roofline": {"bound": "mfma", "kernel": bwd_kernels,
                     "achieved": round(bwd_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(wl.name, bwd_name),
                     "flop_per_call": wl.flop_bwd, "flop_formula": "10*d*U"},
    }
    if args.copy_calibration:
        n = 1 << 28  # 1 GiB of float32
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_heads, args.cpu_tokens)
    if args.sweep:
        sweep = {}
        parity = {}
        if args.parity:
            with open(args.parity) as f:
                parity = json.load(f)
        records = []
        for name in WORKLOADS:
            print(f"sweep: {name}", file=sys.stderr, flush=True)
            if name != wl.name:
                del wl
                torch.cuda.empty_cache()
                wl = Workload(name, dev)
            # enough steps for about 0.15 s of timed work (short steps need many), after 3 warmup steps
            wq, _, _ = time_workload(fm, wl, 2, 1, use_sched, stored_default(wl.d))
            n = int(min(200, max(5, math.ceil(0.15 / max(wq / 2, 1e-5)))))
            w2, p2, ok2 = time_workload(fm, wl, n, 3, use_sched, stored_default(wl.d))
            w0, p0, _ = time_workload(fm, wl, n, 3, use_sched, not stored_default(wl.d))
            ms = w2 * 1e3 / n
            nvec = sum(v is not None for v in wl.vecs)
            bb = bounds_bytes(wl.B, wl.spec.Hm, wl.N, nvec) if nvec else 0
            r = {"workload": name, "config_index": wl.cfg.index, "mask": wl.mask, "B": wl.B, "H": wl.H,
                 "N": wl.N, "d": wl.d, "dtype": "bf16", "U": int(wl.U), "flop_per_step": wl.flop,
                 "t_bounds_us": round(float(p2[0]) * 1e3, 2), "t_plan_us": round(float(p2[2]) * 1e3, 2),
                 "t_fwd_ms": round(float(p2[3]), 4), "t_bwd_ms": round(float(p2[4]), 4),
                 "ms_per_step": round(ms, 4), "TFLOP/s": round(wl.flop / (ms * 1e-3) / 1e12, 2),
                 "pct_of_peak": round(100.0 * wl.flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                 "fwd_TFLOP/s": round(wl.flop_fwd / (float(p2[3]) * 1e-3) / 1e12, 2),
                 "bwd_TFLOP/s": round(wl.flop_bwd / (float(p2[4]) * 1e-3) / 1e12, 2),
                 "prepass_GB/s": round(bb / (float(p2[0]) * 1e-3) / 1e9, 1) if nvec else None,
                 "backward": "fm_bwd_ds (stored dS)" if stored_default(wl.d) else "fm_bwd (dQ recomputed)",
                 "t_bwd_other_form_ms": round(float(p0[4]), 4),
                 "ms_per_step_other_form": round(w0 * 1e3 / n, 4),
                 "finite": ok2, "schedule": "longest-first" if use_sched else "default order",
                 "steps": n}
            r.update(parity.get(name, {}))
            records.append(r)
            sweep[name] = {k: r[k] for k in ("TFLOP/s", "pct_of_peak", "ms_per_step", "t_fwd_ms", "t_bwd_ms",
                                              "backward", "t_bwd_other_form_ms")}
        if args.records:
            with open(args.records, "w") as f:
                for r in records:
                    f.write(json.dumps(r) + "\n")
        # one context-parallel rank's share at its real shape: the long-context workload over 8 ranks,
        # each rank's contiguous 16384 query rows against all keys
        del wl
        torch.cuda.empty_cache()
        print("sweep: context-parallel rank shares", file=sys.stderr, flush=True)
        wl = Workload("long_context_causal_document", dev)
        ranks = 8
        per = wl.N // ranks
        cp = []
        for r in range(ranks):
            a, b = r * per, (r + 1) * per
            t = time_rows(fm, wl, a, b, max(2, args.steps // 8), 1)
            u = unmasked_pairs(wl.spec, wl.H, rows=(a, b))
            cp.append({"rank": r, "rows": [a, b], "ms": round(t * 1e3, 3), "U": int(u),
                       "TFLOP/s": round(14.0 * wl.d * u / t / 1e12, 2)})
        ms = [c["ms"] for c in cp]
        sweep["long_context_causal_document, context-parallel rank shares (8 ranks)"] = {
            "ranks": cp, "max_ms": max(ms), "mean_ms": round(sum(ms) / len(ms), 3),
            "imbalance_max_over_mean": round(max(ms) / (sum(ms) / len(ms)), 3)}
        # the same 8 shares with boundaries that balance the unmasked pairs per rank
        cuts = balanced_row_blocks(wl.spec, wl.H, ranks)
        cpb = []
        for r in range(ranks):
            a, b = cuts[r], cuts[r + 1]
            t = time_rows(fm, wl, a, b, max(2, args.steps // 8), 1)
            u = unmasked_pairs(wl.spec, wl.H, rows=(a, b))
            cpb.append({"rank": r, "rows": [a, b], "ms": round(t * 1e3, 3), "U": int(u),
                        "TFLOP/s": round(14.0 * wl.d * u / t / 1e12, 2)})
        ms = [c["ms"] for c in cpb]
        sweep["long_context_causal_document, context-parallel rank shares (8 ranks, balanced by unmasked pairs)"] = {
            "ranks": cpb, "max_ms": max(ms), "mean_ms": round(sum(ms) / len(ms), 3),
            "imbalance_max_over_mean": round(max(ms) / (sum(ms) / len(ms)), 3)}
        del wl
        torch.cuda.empty_cache()
        print("sweep: key compaction", file=sys.stderr, flush=True)
        wl = Workload("dpo_rm_causal_key_drop", dev)
        n = max(3, args.steps // 4)
        w3, ok3 = time_workload_compacted(fm, wl, n, 1)
        sweep["dpo_rm_causal_key_drop (key compaction)"] = {
            "TFLOP/s": round(wl.flop / (w3 * 1e3 / n * 1e-3) / 1e12, 2), "ms_per_step": round(w3 * 1e3 / n, 3),
            "U": int(wl.U), "compactable": ok3}
        # hash-bucket attention, against plain causal attention at the same shape
        for name in W.HASH_WORKLOADS:
            print(f"sweep: {name}", file=sys.stderr, flush=True)
            del wl
            torch.cuda.empty_cache()
            hw = HashWorkload(name, dev)
            n = max(3, args.steps // 4)
            t, U, okh = time_hash_workload(fm, hw, n, 1)
            te, _, _ = time_hash_workload(fm, hw, n, 1, graph=True)
            cfg_i, hd = W.HASH_WORKLOADS[name][0], hw.d
            del hw
            torch.cuda.empty_cache()
            wl = Workload(name + " (plain causal)", dev, cfg_mask=(cfg_i, "causal"))
            wc, _, _ = time_workload(fm, wl, n, 1)
            causal_ms = wc * 1e3 / n
            sweep[name] = {"TFLOP/s": round(14.0 * hd * U / t / 1e12, 2), "ms_per_step": round(t * 1e3, 3),
                           "ms_per_step_graph_replay": round(te * 1e3, 3),
                           "U": U, "buckets": W.HASH_WORKLOADS[name][1], "finite": okh,
                           "plain_causal_ms_per_step": round(causal_ms, 3),
                           "speedup_vs_plain_causal": round(causal_ms / (t * 1e3), 2)}
        rec["sweep"] = sweep
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
