"""Benchmark one paged GQA decode step on one MI355X.

Default workload: the single long context (B=1, Hq=32, Hkv=8, d=128,
32768 tokens, bf16, 4096-page shuffled pool, S=32 split). Prints ONE JSON
line. The step time is the GPU time of K back-to-back steps on one stream
(one HIP event pair around all of them) divided by K; ``value`` is the
step's algorithmic bytes (K/V of the exact tokens + q + out + used
block-table entries + seq_lens) divided by that time.

Inputs are made once and stay in HBM. To keep the 256 MB Infinity Cache from
serving repeated steps, the timed loop rotates over several identical copies
of the pools (so each copy is evicted by the others before it is read again).
Before the timed steps the step runs for --ramp-ms of wall time, so the GPU
is at its steady clocks whatever --warmup is.

The default line also carries: the same K/V bytes read by a plain streaming
kernel (``stream_ceiling``: the one-pass read ceiling in this run), the
same tiles read through the block table with the decode's own work split
and load path but no arithmetic, state or merge (``paged_read``: what the
paged gather alone costs in this run; per config ``paged_read_us``), the
mixed batch of 8 and the batch-4 regime (``configs``: mixed8 in the policy's
mode; b4 unsplit, split, work queue and the policy's pick), and the CPU
oracle on the host (``cpu_baseline``, with the 64-sequence step
extrapolated from a sample of its rows).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--ramp-ms 100]
                       [--config long] [--mode split] [--splits 32] [--chunk 0]
                       [--no-cpu] [--no-configs] [--no-stream]
                       [--merge fused|kernel] [--seed N] [--identity-table]
       python bench.py --config mixed8 --sweep | --ablation   (one line per candidate)
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged GQA decode µs/step + effective HBM GB/s (% of MI355X peak)"
PEAK_HBM_GBPS = 8000.0
MALL_BYTES = 256 * 2 ** 20


# ---------------------------------------------------------------- HIP events

class HipEvents:
    """Raw hipEvent_t handles via libamdhip64 (timing only)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def ms(self, a, b):
        self.lib.hipEventSynchronize(b)
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def record(self, e, stream):
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        if self.lib.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


# ---------------------------------------------------------------- workload

def make_inputs(name, seed, device):
    import workloads as W
    spec = W.CONFIGS[name]
    if name == "b64":
        dev = W.make_device_case(name, seed, device=device)
        return spec, dev, None
    case = W.make_case(name, seed, poison=False)
    dev = W.case_to_device(case, device=device)
    dev.update(seq_lens_host=case.seq_lens, block_table_host=case.block_table,
               num_pages=case.num_pages, sm_scale=case.sm_scale, spec=spec)
    return spec, dev, case


def to_identity_table(dev):
    """Same cache, pages rewritten so that each sequence's pages are
    consecutive in the pool in logical order (block table = running index):
    the paging diagnostic (what the indirection costs against a dense
    layout). Outputs are unchanged bit for bit."""
    import torch
    lens = np.asarray(dev["seq_lens_host"])
    bt = np.asarray(dev["block_table_host"])
    pages = (lens + 15) // 16
    order = np.concatenate([bt[b, :pages[b]] for b in range(len(lens))]).astype(np.int64)
    idx = torch.from_numpy(order).to(dev["k_pool"].device)
    new_bt = np.zeros_like(bt)
    off = 0
    for b in range(len(lens)):
        new_bt[b, :pages[b]] = np.arange(off, off + pages[b], dtype=np.int32)
        off += pages[b]
    dev = dict(dev)
    dev["k_pool"] = dev["k_pool"].index_select(0, idx).contiguous()
    dev["v_pool"] = dev["v_pool"].index_select(0, idx).contiguous()
    dev["block_table"] = torch.from_numpy(new_bt).to(idx.device)
    dev["block_table_host"] = new_bt
    dev["num_pages"] = int(len(order))
    return dev


def partial_kernel_bytes(stats, spec, batch):
    """Algorithmic bytes the partial kernel moves per launch: K/V of the exact
    tokens, q, used block-table entries, seq_lens, plus out when that launch
    writes it (unsplit, or the merge fused into its tail: one launch)."""
    d, Hq = spec.head_dim, spec.num_q_heads
    out_bytes = batch * Hq * d * 2
    b = stats["algorithmic_bytes"] - out_bytes
    return b + (out_bytes if stats["launches"] == 1 else 0)


def kernel_sources() -> bytes:
    """The partial kernel's source and the headers it includes, in a fixed
    order: what a committed counter summary was taken on."""
    paths = [("paged_kv_gqa_04_amd", "csrc", "decode.hip"),
             ("paged_kv_gqa_04_amd", "csrc", "pkv_internal.h"), ("include", "pkv.h")]
    return b"".join(open(os.path.join(ROOT, *p), "rb").read() for p in paths)


# Committed rocprofv3 FETCH_SIZE / WRITE_SIZE summaries, by the launch they
# were taken on: (workload, mode, splits, merge) -> file.
TRAFFIC_PROFILES = {
    ("long", "split", 32, "fused"): "partial_kernel_long_split32_traffic.md",
    ("mixed8", "workqueue", 14, "fused"): "partial_kernel_mixed8_workqueue_traffic.md",
    ("b4", "workqueue", 13, "fused"): "partial_kernel_b4_workqueue_traffic.md",
    ("b64", "workqueue", 16, "fused"): "partial_kernel_b64_workqueue_traffic.md",
}


def measured_traffic(workload, mode, splits, merge):
    """HBM bytes per partial-kernel launch from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, scaled by the plain-copy factors it
    records; None when no summary covers this launch or the kernel source
    has changed since the counters were taken."""
    import hashlib
    name = TRAFFIC_PROFILES.get((workload, mode, splits, merge))
    if name is None:
        return None
    try:
        text = open(os.path.join(ROOT, "profiles", name)).read()
        src = kernel_sources()
    except OSError:
        return None
    fields = dict(l.split(": ", 1) for l in text.splitlines()
                  if l.startswith(("traffic_bytes_per_launch:", "kernel_source_sha256:")))
    if fields.get("kernel_source_sha256", "").strip() != hashlib.sha256(src).hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def ramp(launch, min_ms):
    """Run ``launch(i)`` in batches, synchronising between them, until
    ``min_ms`` of wall time has passed: the GPU reaches its steady clocks
    under this load (a fixed step count would not: a step can be 0.03 µs or
    1 ms long). Returns (steps, ms)."""
    import torch
    if min_ms <= 0:
        return 0, 0.0
    t0, n = time.perf_counter(), 0
    while True:
        for _ in range(32):
            launch(n)
            n += 1
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) * 1e3
        if el >= min_ms:
            return n, el


def time_mode(P, dev, spec, mode, splits, chunk, steps, warmup, replicas, ev, merge="fused",
              ramp_ms=0.0, light=False, paged_read=False):
    """Time `steps` back-to-back decode steps (one event pair around all of
    them: per-step markers would add their own overhead) after a clock ramp
    of `ramp_ms` and `warmup` more steps; with `paged_read`, then as many
    back-to-back paged reads with the same plan and pool copies (the gather
    alone: `paged_read_us`); unless `light`, then the same number of steps
    with markers around the partial kernel alone, and the synchronized wall
    time with host planning."""
    import torch
    B = len(dev["seq_lens_host"])
    shape = P.make_shape(B, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                         dev["block_table_host"].shape[1], dev["num_pages"], spec.dtype,
                         dev["sm_scale"])
    plan = P.Plan(shape, dev["seq_lens_host"], P.make_opts(mode, splits, chunk, merge=merge))
    plan.upload()
    stats = plan.stats()
    out = torch.empty_like(dev["q"])
    pools = dev["replicas"][:replicas]
    stream = torch.cuda.current_stream().cuda_stream
    args = lambda r: (dev["q"], pools[r][0], pools[r][1], dev["block_table"], dev["seq_lens"], out)
    ramp_steps, ramp_done = ramp(
        lambda i: P.pkv_decode(plan.handle, *args(i % len(pools)), stream), ramp_ms)
    for i in range(warmup):
        P.pkv_decode(plan.handle, *args(i % len(pools)), stream)
    torch.cuda.synchronize()
    # 1) back-to-back steps
    e_all = ev.create(2)
    t0 = time.perf_counter()
    P.pkv_decode_marked(plan.handle, *args(0), stream, e_all[0], None, None)
    for i in range(1, steps):
        P.pkv_decode(plan.handle, *args(i % len(pools)), stream)
    ev.record(e_all[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = ev.ms(e_all[0], e_all[1]) / steps
    ev.destroy(e_all)
    extra = {}
    if paged_read and stats["mode_name"] != "bucketed":
        extra["paged_read_us"] = time_paged_read(P, plan, dev, pools, steps, ev)
    if light:
        plan.close()
        return {"stats": stats, "step_us": step_ms * 1e3, "wall_us_per_step": wall / steps * 1e6,
                "ramp_steps": ramp_steps, "ramp_ms": ramp_done, **extra}
    # 2) per-step markers around the partial kernel (includes marker cost)
    evs = ev.create(2 * steps)
    for i in range(steps):
        P.pkv_decode_marked(plan.handle, *args(i % len(pools)), stream, evs[2 * i],
                            evs[2 * i + 1], None)
    torch.cuda.synchronize()
    part = [ev.ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps)]
    ev.destroy(evs)
    # synchronized wall time of a step including host planning + upload: as
    # the library runs it (the re-planned image is unchanged, so nothing is
    # copied), and with the copy forced
    def sync_wall(force):
        sync = []
        for i in range(min(100, steps)):
            torch.cuda.synchronize()
            t = time.perf_counter()
            plan.update(dev["seq_lens_host"])
            plan.upload(force=force)
            P.pkv_decode(plan.handle, *args(i % len(pools)), stream)
            torch.cuda.synchronize()
            sync.append(time.perf_counter() - t)
        return sync
    sync = sync_wall(False)
    sync_copy = sync_wall(True)
    plan.close()
    return {
        "stats": stats,
        "step_us": step_ms * 1e3,
        "partial_marked_us": float(np.mean(part)) * 1e3,
        "partial_marked_us_p10_p90": [float(np.percentile(part, 10)) * 1e3,
                                      float(np.percentile(part, 90)) * 1e3],
        "wall_us_per_step": wall / steps * 1e6,
        "sync_wall_us_with_plan": float(np.median(sync)) * 1e6,
        "sync_wall_us_with_plan_copy": float(np.median(sync_copy)) * 1e6,
        "ramp_steps": ramp_steps,
        "ramp_ms": ramp_done,
        **extra,
    }


def time_paged_read(P, plan, dev, pools, steps, ev):
    """µs per paged read (pkv_paged_read: every K/V tile the decode with
    `plan` reads, with its work split and load path, nothing else), timed
    back to back over the same pool copies right after the decode's steps."""
    import torch
    sink = torch.zeros(1, dtype=torch.int32, device=dev["q"].device)
    stream = torch.cuda.current_stream().cuda_stream
    read = lambda i: P.pkv_paged_read(plan.handle, pools[i % len(pools)][0],
                                      pools[i % len(pools)][1], dev["block_table"],
                                      dev["seq_lens"], sink, stream)
    for i in range(min(steps, 50)):
        read(i)
    e = ev.create(2)
    ev.record(e[0], stream)
    for i in range(steps):
        read(i)
    ev.record(e[1], stream)
    torch.cuda.synchronize()
    us = ev.ms(e[0], e[1]) / steps * 1e3
    ev.destroy(e)
    return us


def time_graph(P, dev, spec, mode, splits, chunk, steps, warmup, replicas, ev, merge="fused"):
    """The same steps launched from a HIP graph: one graph holds one decode
    per pool copy (so the copies still rotate) and is replayed back to back;
    returns µs per step."""
    import torch
    B = len(dev["seq_lens_host"])
    shape = P.make_shape(B, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                         dev["block_table_host"].shape[1], dev["num_pages"], spec.dtype,
                         dev["sm_scale"])
    plan = P.Plan(shape, dev["seq_lens_host"], P.make_opts(mode, splits, chunk, merge=merge))
    plan.upload()
    out = torch.empty_like(dev["q"])
    pools = dev["replicas"][:replicas]

    def one(r):
        plan.decode(dev["q"], pools[r][0], pools[r][1], dev["block_table"], dev["seq_lens"], out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for r in range(len(pools)):
            one(r)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(len(pools)):
            one(r)
    reps = max(1, steps // len(pools))
    for _ in range(max(1, warmup // len(pools))):
        graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e = ev.create(2)
    ev.record(e[0], stream)
    for _ in range(reps):
        graph.replay()
    ev.record(e[1], stream)
    torch.cuda.synchronize()
    us = ev.ms(e[0], e[1]) / (reps * len(pools)) * 1e3
    ev.destroy(e)
    del graph
    plan.close()
    return us


def sweep(P, dev, spec, replicas, ev, a, seed):
    """Policy calibration: time unsplit, split over a range of S and the work
    queue over a range of chunk sizes, plus the policy's own choice."""
    lens = np.asarray(dev["seq_lens_host"])
    max_pages = int((lens.max() + 15) // 16)
    cands = [("auto", 0, 0), ("unsplit", 0, 0)]
    for S in (2, 4, 8, 16, 24, 32, 48, 64, 96, 128, 192, 256):
        if S <= max_pages:
            cands.append(("split", S, 0))
    for c in (4, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512, 1024, 2048):
        if c <= max_pages:
            cands.append(("workqueue", 0, c))
    for mode, S, c in cands:
        r = time_mode(P, dev, spec, mode, S, c, a.steps, a.warmup, replicas, ev, a.merge)
        st = r["stats"]
        print(json.dumps({
            "workload": spec.name, "seed": seed, "mode": mode,
            "resolved": st["mode_name"], "num_splits": st["num_splits"],
            "chunk_pages": st["chunk_pages"], "grid": st["grid"],
            "us_per_step": round(r["step_us"], 2),
            "gbps": round(st["algorithmic_bytes"] / (r["step_us"] * 1e-6) / 1e9, 1),
        }), flush=True)


def ablation(P, dev, spec, replicas, ev, a, seed):
    """The scheduling comparators of the PersistentKV explainer (Results,
    scheduling overhead) on one workload: the policy's choice, the unsplit
    path, the rectangular split grid, the compact work queue and
    exact-length bucketing (the last two also with the pages' separate merge
    launch). One JSON line each, with the scheduler counters."""
    cands = [("auto", "fused"), ("unsplit", "fused"), ("split", "fused"), ("split", "kernel"),
             ("workqueue", "fused"), ("workqueue", "kernel"), ("bucketed", "fused"),
             ("bucketed", "kernel")]
    for mode, merge in cands:
        r = time_mode(P, dev, spec, mode, 0, 0, a.steps, a.warmup, replicas, ev, merge)
        st = r["stats"]
        print(json.dumps({
            "workload": spec.name, "seed": seed, "mode": mode, "merge": merge,
            "resolved": st["mode_name"], "num_splits": st["num_splits"],
            "chunk_pages": st["chunk_pages"], "grid": st["grid"],
            "launches": st["launches"], "bucket_launches": st["bucket_launches"],
            "num_slots": st["num_slots"], "partial_bytes": st["partial_bytes"],
            "us_per_step": round(r["step_us"], 2),
            "gbps": round(st["algorithmic_bytes"] / (r["step_us"] * 1e-6) / 1e9, 1),
            "sync_wall_us_with_plan": round(r["sync_wall_us_with_plan"], 2),
            "sync_wall_us_with_plan_copy": round(r["sync_wall_us_with_plan_copy"], 2),
        }), flush=True)


def time_append(P, dev, spec, steps, warmup, ev):
    """Time the append step (the new token's K/V of every row written through
    the block table) as `steps` back-to-back launches. Each row rewrites its
    last token (position N_b - 1, a page the table already holds), so every
    launch does the full work without growing the cache."""
    import torch
    lens = np.asarray(dev["seq_lens_host"])
    B, Hkv, d = len(lens), spec.num_kv_heads, spec.head_dim
    td = dev["k_pool"].dtype
    g = torch.Generator(device=dev["k_pool"].device).manual_seed(1)
    k_new = torch.randn((B, Hkv, d), generator=g, device=dev["k_pool"].device).to(td)
    v_new = torch.randn((B, Hkv, d), generator=g, device=dev["k_pool"].device).to(td)
    pos = torch.from_numpy(np.maximum(lens - 1, 0).astype(np.int32)).to(k_new.device)
    shape = P.make_shape(B, spec.num_q_heads, Hkv, d, dev["block_table_host"].shape[1],
                         dev["num_pages"], spec.dtype)
    stream = torch.cuda.current_stream().cuda_stream
    args = (k_new, v_new, dev["k_pool"], dev["v_pool"], dev["block_table"], pos)
    for _ in range(warmup):
        P.pkv_append(shape, *args, None, stream)
    torch.cuda.synchronize()
    e = ev.create(2)
    ev.record(e[0], stream)
    for _ in range(steps):
        P.pkv_append(shape, *args, None, stream)
    ev.record(e[1], stream)
    torch.cuda.synchronize()
    us = ev.ms(e[0], e[1]) / steps * 1e3
    ev.destroy(e)
    # new K/V read + written, plus one table entry and one length per row
    nbytes = 2 * 2 * B * Hkv * d * 2 + 8 * B
    return {"us_per_launch": round(us, 3), "bytes_per_launch": int(nbytes),
            "gbps": round(nbytes / (us * 1e-6) / 1e9, 1), "rows": int(B)}


def time_step_with_append(P, dev, spec, mode, splits, chunk, steps, warmup, replicas, ev):
    """A decode step that also appends each row's new token, timed two ways
    over `steps` back-to-back steps: pkv_append then pkv_decode (two
    launches), and pkv_decode_append (one launch). As in time_append, each
    row rewrites its last token (position N_b - 1), so the plan for the
    lengths N_b serves every step."""
    import torch
    lens = np.asarray(dev["seq_lens_host"])
    B, Hkv, d = len(lens), spec.num_kv_heads, spec.head_dim
    shape = P.make_shape(B, spec.num_q_heads, Hkv, d, dev["block_table_host"].shape[1],
                         dev["num_pages"], spec.dtype, dev["sm_scale"])
    plan = P.Plan(shape, lens, P.make_opts(mode, splits, chunk))
    plan.upload()
    td = dev["k_pool"].dtype
    g = torch.Generator(device=dev["k_pool"].device).manual_seed(2)
    k_new = torch.randn((B, Hkv, d), generator=g, device=dev["k_pool"].device).to(td)
    v_new = torch.randn((B, Hkv, d), generator=g, device=dev["k_pool"].device).to(td)
    pos = torch.from_numpy(np.maximum(lens - 1, 0).astype(np.int32)).to(k_new.device)
    new_lens = torch.empty_like(pos)
    out = torch.empty_like(dev["q"])
    pools = dev["replicas"][:replicas]
    stream = torch.cuda.current_stream().cuda_stream

    def two(i):
        kp, vp = pools[i % len(pools)]
        P.pkv_append(shape, k_new, v_new, kp, vp, dev["block_table"], pos, new_lens, stream)
        P.pkv_decode(plan.handle, dev["q"], kp, vp, dev["block_table"], new_lens, out, stream)

    def one(i):
        kp, vp = pools[i % len(pools)]
        P.pkv_decode_append(plan.handle, dev["q"], k_new, v_new, kp, vp, dev["block_table"],
                            pos, out, new_lens, stream)

    res = {}
    for name, fn in (("append_then_decode_us", two), ("decode_append_us", one)):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e = ev.create(2)
        ev.record(e[0], stream)
        for i in range(steps):
            fn(i)
        ev.record(e[1], stream)
        torch.cuda.synchronize()
        res[name] = round(ev.ms(e[0], e[1]) / steps * 1e3, 2)
        ev.destroy(e)
    plan.close()
    return res


def serve_loop(P, name, seed, mode, steps, warmup):
    """A decode loop as a server runs it, every step on the host clock: the
    page pool gives a page to each row whose new token opens one (the table
    goes to the device when it changed), the plan is re-made for the new
    lengths and its queue copied only when it changed, and one launch
    appends every row's new token and decodes (pkv_decode_append), then the
    host waits for it. The ai-trend study note ("How it works", steps two
    and four) describes this loop; the PersistentKV explainer (Evaluation
    protocol) reports synchronized wall time including planning. One pool
    copy only (the appends write into it), so the cache may be served from
    the Infinity Cache: these are per-step latencies, not bandwidth."""
    import torch
    import workloads as W
    spec = W.CONFIGS[name]
    total = steps + warmup
    grow = total // W.PAGE_TOKENS + 2  # pages each row may take
    case = W.make_case(name, seed, poison=False)
    B = case.batch
    # the pool's spare pages, plus room for the growth in a wider table
    extra = B * grow
    fill = np.arange(extra) % case.num_pages  # contents of the added pages: any data
    k = np.concatenate([case.k_pool, case.k_pool[fill]])
    v = np.concatenate([case.v_pool, case.v_pool[fill]])
    num_pages = case.num_pages + extra
    assert k.shape[0] == num_pages and v.shape[0] == num_pages
    stride0 = case.block_table.shape[1]
    bt = np.full((B, stride0 + grow), -1, np.int32)
    bt[:, :stride0] = case.block_table
    lens = case.seq_lens.astype(np.int32).copy()
    pool = P.Pool(num_pages)
    pool.alloc(num_pages)
    used = set()
    for b in range(B):
        used.update(int(x) for x in bt[b, :W.pages_for(int(lens[b]))])
    pool.free(np.array(sorted(set(range(num_pages)) - used), np.int32))
    td = W.torch_dtype(case.dtype)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kp, vp = dev(k.view(np.int16)).view(td), dev(v.view(np.int16)).view(td)
    bt_d, lens_d = dev(bt), dev(lens)
    new_d = torch.empty_like(lens_d)
    g = torch.Generator(device="cuda").manual_seed(3)
    q = torch.randn((B, spec.num_q_heads, spec.head_dim), generator=g, device="cuda").to(td)
    kn = torch.randn((B, spec.num_kv_heads, spec.head_dim), generator=g, device="cuda").to(td)
    vn = torch.randn((B, spec.num_kv_heads, spec.head_dim), generator=g, device="cuda").to(td)
    out = torch.empty_like(q)
    shape = P.make_shape(B, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, bt.shape[1],
                         num_pages, case.dtype, case.sm_scale)
    plan = P.Plan(shape, lens + 1, P.make_opts(mode, 0, 0))
    plan.upload()
    times, copies, table_updates = [], 0, 0
    for step in range(total):
        torch.cuda.synchronize()
        t = time.perf_counter()
        if pool.prepare(lens, bt):
            bt_d.copy_(torch.from_numpy(bt))
            table_updates += step >= warmup
        plan.update(lens + 1)
        if P.pkv_plan_upload_needed(plan.handle):
            copies += step >= warmup
        plan.upload()
        plan.decode_append(q, kn, vn, kp, vp, bt_d, lens_d, out, new_d)
        torch.cuda.synchronize()
        if step >= warmup:
            times.append(time.perf_counter() - t)
        lens += 1
        lens_d, new_d = new_d, lens_d
    st = plan.stats()
    plan.close()
    pool.close()
    assert np.array_equal(lens_d.cpu().numpy(), lens), "device lengths diverged"
    us = np.asarray(times) * 1e6
    return {"serve": name, "seed": seed, "mode": st["mode_name"], "steps": steps,
            "warmup": warmup, "rows": int(B), "final_kv_tokens": int(lens.sum()),
            "sync_wall_us_p50": round(float(np.median(us)), 2),
            "sync_wall_us_p90": round(float(np.percentile(us, 90)), 2),
            "steps_with_queue_copy": int(copies), "steps_with_table_copy": int(table_updates)}


def stream_ceiling(P, dev, kv_bytes, steps, ramp_ms, ev, grids=(256, 512, 768, 1024, 2048)):
    """The same number of K/V bytes as one step, read once by a plain
    streaming kernel (half from each pool, rotating over the same pool
    copies as the decode): the HBM ceiling a one-pass read of these bytes
    reaches in this run. Returns µs per read for each grid and the best."""
    import torch
    each = kv_bytes // 2 // 16 * 16
    pools = dev["replicas"]
    if any(t.numel() * t.element_size() < each for kv in pools for t in kv):
        return None
    sink = torch.zeros(1, dtype=torch.int32, device=pools[0][0].device)
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for grid in grids:
        launch = lambda i: P.pkv_stream_read(pools[i % len(pools)][0], pools[i % len(pools)][1],
                                             each, grid, sink, stream)
        ramp(launch, ramp_ms)
        e = ev.create(2)
        ev.record(e[0], stream)
        for i in range(steps):
            launch(i)
        ev.record(e[1], stream)
        torch.cuda.synchronize()
        res[grid] = ev.ms(e[0], e[1]) / steps * 1e3
        ev.destroy(e)
    best = min(res, key=res.get)
    return {"bytes": int(2 * each), "us_by_grid": {str(g): round(u, 2) for g, u in res.items()},
            "us": round(res[best], 2), "grid": best,
            "gbps": round(2 * each / (res[best] * 1e-6) / 1e9, 1)}


def replicate(dev, name_touched_bytes, replicas=0):
    """Enough identical pool copies that each is evicted from the 256 MB
    Infinity Cache before it is read again."""
    touched = name_touched_bytes
    n = replicas or (1 if touched > 4 * MALL_BYTES else
                     min(8, math.ceil(2 * MALL_BYTES / max(1, touched)) + 1))
    reps = [(dev["k_pool"], dev["v_pool"])]
    for _ in range(n - 1):
        reps.append((dev["k_pool"].clone(), dev["v_pool"].clone()))
    dev["replicas"] = reps
    return n


def config_line(P, name, seed, steps, warmup, ramp_ms, ev, modes, stream=True):
    """Time one workload in each of `modes` (lighter than the headline: no
    per-step markers); returns a dict per mode with the policy's choice and,
    with `stream`, the plain streaming read of the same K/V bytes timed in
    the same run (each mode's time over it in `over_stream`)."""
    import torch
    spec, dev, _ = make_inputs(name, seed, "cuda")
    touched = int(np.sum(dev["seq_lens_host"])) * spec.num_kv_heads * spec.head_dim * 4
    nrep = replicate(dev, touched)
    B = len(dev["seq_lens_host"])
    out = {"description": spec.description, "pool_replicas": nrep}
    for mode in modes:
        r = time_mode(P, dev, spec, mode, 0, 0, steps, warmup, nrep, ev, ramp_ms=ramp_ms,
                      light=True, paged_read=True)
        st = r["stats"]
        alg = st["algorithmic_bytes"]
        gbps = alg / (r["step_us"] * 1e-6) / 1e9
        part = partial_kernel_bytes(st, spec, B)
        entry = {
            "resolved": st["mode_name"], "num_splits": st["num_splits"],
            "chunk_pages": st["chunk_pages"], "grid": st["grid"], "launches": st["launches"],
            "us_per_step": round(r["step_us"], 2), "gbps": round(gbps, 1),
            "pct_of_peak_hbm": round(100 * gbps / PEAK_HBM_GBPS, 1),
            "algorithmic_bytes_per_step": int(alg),
            "ramp_ms": round(r["ramp_ms"], 1), "ramp_steps": r["ramp_steps"],
        }
        if st["launches"] == 1:  # the launch is the whole step
            entry["partial_kernel_frac"] = round(part / (r["step_us"] * 1e-6) / 1e9 /
                                                 PEAK_HBM_GBPS, 4)
        if "paged_read_us" in r:
            entry["paged_read_us"] = round(r["paged_read_us"], 2)
            entry["over_paged_read"] = round(r["step_us"] / r["paged_read_us"], 3)
        out[mode] = entry
    if stream:
        kv = int(st["kv_tokens"]) * spec.num_kv_heads * spec.head_dim * 4
        sc = stream_ceiling(P, dev, kv, steps, ramp_ms, ev)
        if sc is not None:
            out["stream_ceiling"] = sc
            for mode in modes:
                out[mode]["over_stream"] = round(out[mode]["us_per_step"] / sc["us"], 3)
    del dev
    torch.cuda.empty_cache()
    return out


def host_info():
    """Host CPU facts for the CPU baseline."""
    info = {"host_cpus": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    import subprocess
    try:  # lscpu's view of the same CPU: model, family and topology
        text = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        keys = {"Model name": "model_name", "CPU family": "cpu_family", "Model": "model",
                "Socket(s)": "sockets", "Core(s) per socket": "cores_per_socket",
                "Thread(s) per core": "threads_per_core", "CPU(s)": "cpus"}
        lscpu = {}
        for line in text.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in keys:
                lscpu[keys[k.strip()]] = v.strip()
        if lscpu:
            info["lscpu"] = lscpu
    except (OSError, subprocess.SubprocessError):  # pragma: no cover
        pass
    return info


def cpu_b64_extrapolated(seed, rows=4):
    """The oracle on a seeded sample of the 64-sequence workload's rows (their
    pages copied from the device case), scaled up by the token fraction:
    an extrapolated CPU time for the whole step."""
    import torch
    import workloads as W
    from oracle import paged_gqa as O
    dev = W.make_device_case("b64", seed, device="cuda")
    lens = np.asarray(dev["seq_lens_host"])
    pick = np.sort(np.random.default_rng(seed).choice(len(lens), size=rows, replace=False))
    sub = W.host_subcase_from_device(dev, pick)
    del dev
    torch.cuda.empty_cache()
    t = time.perf_counter()
    O.decode_case(sub)
    sec = time.perf_counter() - t
    frac = float(lens[pick].sum()) / float(lens.sum())
    return {"us_per_step": round(sec / frac * 1e6, 1), "kind": "oracle, extrapolated",
            "sample": f"rows {pick.tolist()} of 64 ({100 * frac:.1f}% of the step's tokens), "
                      f"one run, scaled by the token fraction",
            "sample_seconds": round(sec, 2)}


def cpu_baseline(case, target_s=10.0, cap_s=30.0, single_thread=False):
    """Time the CPU oracle on the bench workload until ~target_s of work
    (with the BLAS pool limited to one thread when `single_thread`)."""
    from oracle import paged_gqa as O
    if single_thread:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            return cpu_baseline(case, target_s, cap_s)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    times = []
    t_start = time.perf_counter()
    while True:
        t = time.perf_counter()
        O.decode_case(case)
        times.append(time.perf_counter() - t)
        el = time.perf_counter() - t_start
        if el >= target_s or el + times[-1] > cap_s:
            break
    return float(np.median(times)), len(times), threads


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # Untimed steps after the clock ramp (the ramp, not this count, brings the
    # GPU to its steady clocks).
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--ramp-ms", type=float, default=100.0,
                    help="before timing, run the step for at least this many ms of wall "
                         "time (clock ramp; independent of --warmup)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the mixed-batch and batch-4 sub-results of the default line")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the plain streaming-read ceiling")
    ap.add_argument("--config", default="long")
    ap.add_argument("--mode", default=None)
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--merge", default="fused", choices=["fused", "kernel"])
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-auto", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes 5 times "
                         "(reference kernel for scaling rocprof byte counters)")
    ap.add_argument("--identity-table", action="store_true",
                    help="paging diagnostic: the same cache with each sequence's pages "
                         "consecutive in the pool (identity block table)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a HIP graph")
    ap.add_argument("--append", action="store_true",
                    help="also time the append step (new-token K/V written through "
                         "the block table) on the workload")
    ap.add_argument("--ablation", action="store_true",
                    help="time the scheduling comparators (unsplit, rectangular split, "
                         "work queue, exact-length bucketing), one JSON line each")
    ap.add_argument("--serve", action="store_true",
                    help="time a serving loop (page allocation, re-planning, queue copy "
                         "when changed, append folded into the decode, synchronisation) "
                         "on the host clock, per step")
    ap.add_argument("--sweep", action="store_true",
                    help="time a grid of (mode, splits / chunk) candidates for the "
                         "workload, one JSON line each (policy calibration)")
    a = ap.parse_args()

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        sys.stderr.write("bench.py measures one GPU only: this library has no "
                         "multi-GPU path (run with --gpus 1)\n")
        sys.exit(2)

    import torch

    if a.copy_bytes:
        src = torch.ones(a.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.copy_bytes, "calls": 5}))
        return

    import paged_kv_gqa_04_amd as P
    import workloads as W

    seed = W.SEED_HOLDOUT if a.seed is None else a.seed
    torch.cuda.set_device(0)
    if a.serve:
        if a.config == "b64":
            sys.exit("--serve builds its inputs on the host: not for b64")
        print(json.dumps(serve_loop(P, a.config, seed, a.mode or "auto", a.steps, a.warmup)),
              flush=True)
        return
    spec, dev, case = make_inputs(a.config, seed, "cuda")
    if a.identity_table:
        dev = to_identity_table(dev)
    mode = a.mode or spec.mode
    splits = a.splits if a.splits is not None else (spec.num_splits or 0)
    if mode != "split":
        splits = a.splits or 0

    touched = int(np.sum(dev["seq_lens_host"])) * spec.num_kv_heads * spec.head_dim * 4
    replicas = replicate(dev, touched, a.replicas)
    ev = HipEvents()

    if a.sweep:
        sweep(P, dev, spec, replicas, ev, a, seed)
        return
    if a.ablation:
        ablation(P, dev, spec, replicas, ev, a, seed)
        return
    r = time_mode(P, dev, spec, mode, splits, a.chunk, a.steps, a.warmup, replicas, ev, a.merge,
                  ramp_ms=a.ramp_ms, paged_read=not a.no_stream)
    st = r["stats"]
    B = len(dev["seq_lens_host"])
    alg = st["algorithmic_bytes"]
    gbps = alg / (r["step_us"] * 1e-6) / 1e9
    part_bytes = partial_kernel_bytes(st, spec, B)
    # The partial kernel's duration: with the merge fused it is the whole
    # step (back-to-back, launch gaps included: conservative); with a
    # separate merge kernel, the marked partial-kernel time.
    kern_us = r["step_us"] if st["launches"] == 1 else r["partial_marked_us"]
    part_gbps = part_bytes / (kern_us * 1e-6) / 1e9

    line = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ramp_ms": round(r["ramp_ms"], 1),
        "ramp_steps": r["ramp_steps"],
        "ms_per_step": round(r["step_us"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {
            "workload": spec.name, "description": spec.description, "batch": B,
            "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
            "head_dim": spec.head_dim, "page_size": 16,
            "kv_tokens": int(st["kv_tokens"]), "pool_pages": int(dev["num_pages"]),
            "mode": st["mode_name"], "num_splits": st["num_splits"],
            "chunk_pages": st["chunk_pages"], "merge": a.merge, "seed": seed,
            "pool_replicas": replicas,
            "block_table": "identity" if a.identity_table else "shuffled",
        },
        "us_per_step": round(r["step_us"], 2),
        "pct_of_peak_hbm": round(100 * gbps / PEAK_HBM_GBPS, 1),
        "algorithmic_bytes_per_step": int(alg),
        "wall_us_per_step": round(r["wall_us_per_step"], 2),
        "sync_wall_us_with_plan": round(r["sync_wall_us_with_plan"], 2),
        "sync_wall_us_with_plan_copy": round(r["sync_wall_us_with_plan_copy"], 2),
        "partial_kernel_marked_us": round(r["partial_marked_us"], 2),
        "partial_kernel_marked_p10_p90_us": [round(x, 2) for x in r["partial_marked_us_p10_p90"]],
        "roofline": {
            "kernel": "partial_kernel",
            "bound": "hbm",
            "achieved": round(part_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(part_gbps / PEAK_HBM_GBPS, 4),
            "traffic": measured_traffic(spec.name, st["mode_name"], st["num_splits"], a.merge),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-scaled)",
            "bytes_per_launch": int(part_bytes),
            "avg_launch_us": round(kern_us, 2),
        },
        "scheduler": {k: st[k] for k in ("grid", "num_items", "empty_items", "num_slots",
                                         "launches", "bucket_launches", "partial_bytes",
                                         "upload_bytes")},
    }
    if not a.no_stream:
        sc = stream_ceiling(P, dev, int(st["kv_tokens"]) * spec.num_kv_heads * spec.head_dim * 4,
                            a.steps, a.ramp_ms, ev)
        if sc is not None:
            sc["decode_over_stream"] = round(r["step_us"] / sc["us"], 3)
            line["stream_ceiling"] = sc
    if "paged_read_us" in r:
        line["paged_read"] = {"us": round(r["paged_read_us"], 2),
                              "gbps": round(alg / (r["paged_read_us"] * 1e-6) / 1e9, 1),
                              "decode_over_paged_read": round(r["step_us"] / r["paged_read_us"], 3)}
    if not a.no_auto and mode != "auto":
        ra = time_mode(P, dev, spec, "auto", 0, 0, a.steps, a.warmup, replicas, ev,
                       ramp_ms=a.ramp_ms, light=True)
        sa = ra["stats"]
        line["auto"] = {
            "mode": sa["mode_name"], "num_splits": sa["num_splits"],
            "chunk_pages": sa["chunk_pages"], "grid": sa["grid"],
            "us_per_step": round(ra["step_us"], 2),
            "gbps": round(sa["algorithmic_bytes"] / (ra["step_us"] * 1e-6) / 1e9, 1),
        }
    if a.graph:
        gus = time_graph(P, dev, spec, mode, splits, a.chunk, a.steps, a.warmup, replicas, ev,
                         a.merge)
        line["graph"] = {"us_per_step": round(gus, 2),
                         "gbps": round(alg / (gus * 1e-6) / 1e9, 1)}
    if a.append:
        line["append"] = time_append(P, dev, spec, a.steps, a.warmup, ev)
        line["append"]["step"] = time_step_with_append(P, dev, spec, mode, splits, a.chunk,
                                                       a.steps, a.warmup, replicas, ev)
    if not a.no_configs and spec.name == "long" and not a.identity_table:
        # The other configurations the 70% goal names (mixed batch) and the
        # batch-4 regime question (unsplit vs split vs work queue, and the
        # policy's pick), measured in the same run.
        cfgs = {"mixed8": config_line(P, "mixed8", seed, a.steps, a.warmup, a.ramp_ms, ev,
                                      ["auto"], stream=not a.no_stream),
                "b4": config_line(P, "b4", seed, a.steps, a.warmup, a.ramp_ms, ev,
                                  ["unsplit", "split", "workqueue", "auto"],
                                  stream=not a.no_stream)}
        b4 = cfgs["b4"]
        timed = {m: b4[m]["us_per_step"] for m in ("unsplit", "split", "workqueue")}
        b4["auto_pick"] = b4["auto"]["resolved"]
        b4["fastest"] = min(timed, key=timed.get)
        line["configs"] = cfgs
    if not a.no_cpu and case is not None:
        sec, reps_done, threads = cpu_baseline(case)
        line["cpu_baseline"] = {
            "value": round(alg / sec / 1e9, 3),
            "unit": "GB/s",
            "us_per_step": round(sec * 1e6, 1),
            "cores": int(threads),
            **host_info(),
            "kind": "oracle",
            "sample": f"whole {spec.name} step (all {B} sequence(s) x {spec.num_kv_heads} "
                      f"KV heads), float64 numpy oracle, median of {reps_done} runs",
        }
        sec1, reps1, _ = cpu_baseline(case, target_s=5.0, cap_s=15.0, single_thread=True)
        line["cpu_baseline"]["single_thread"] = {
            "value": round(alg / sec1 / 1e9, 3), "us_per_step": round(sec1 * 1e6, 1),
            "cores": 1, "sample": f"the same step, BLAS limited to 1 thread, median of {reps1} runs"}
        if spec.name == "long":
            line["cpu_baseline"]["b64"] = cpu_b64_extrapolated(seed)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
