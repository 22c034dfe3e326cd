#!/usr/bin/env python3
"""Benchmark of one denoising step's partitioned attention with selective state reuse.

Workload: the 29-frame 720p-shaped video (B=1, 24 heads, head_dim 64, 8 latent frames x
45x80 patches = 28800 tokens, 32 context partitions of 900 tokens, 10 denoising steps:
an anchor step, then 9 steps with a 40 % fresh budget; bf16 Q/K/V, bf16 O + f32 lse cache,
f32 output).  Inputs come from the seeded generator and are staged in HBM before timing.

One bench step = one denoising step's attention: the host block policy, the fresh blocks,
their cache writeback, the reuse fold and the log-sum-exp merge (dita_set_block_policy +
dita_attn_step).  Steps walk the 10-step schedule cyclically; each cycle starts with a cache
reset and the anchor step.  With the default step counts (multiples of 10) the timed region
is whole denoising runs.

Prints one JSON line: dense-equivalent attention TFLOP/s (4 B H N^2 D per step, the cost of
full attention), ms per step, the dominant kernel's MFMA roofline fraction (fresh-block
FLOPs / its measured duration), the combined MFMA+HBM roofline of the step, and the fp64
oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from workloads import CONFIGS  # noqa: E402
from workloads.gen import head_steps_packed, head_steps  # noqa: E402

METRIC = "dense-equiv attention TFLOP/s + ms/step, % of MFMA+HBM roofline, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)
def kernel_label(head_dim, planner, fp8, fixed=True):
    """Name of the step kernel instantiation a run's steady steps launch: <padded head dim,
    planner measurement compiled in, fp8 cache, fixed reference>.  Steps after the anchor run
    the fixed-reference pass (followed by the running-maximum kernel as a conditional second
    pass, which exits at once unless a reference was rejected); anchor steps run the
    running-maximum kernel."""
    dp = 64 if head_dim <= 64 else (96 if head_dim <= 96 else 128)
    t = lambda b: "true" if b else "false"
    return f"step_bf16<{dp}, {t(planner)}, {t(fp8)}, {t(fixed)}>"


def _gen_job(args):
    cfg, b, h, steps = args
    return b, h, head_steps_packed(cfg, b, h, steps)


def _oracle_job(args):
    """fp64 oracle on one head for `steps` steps; returns (b, h, steps, wall time) with one
    BLAS thread (inputs drawn before the clock starts)."""
    cfg, b, h, steps = args
    from threadpoolctl import threadpool_limits
    import oracle
    inputs = head_steps(cfg, b, h, steps)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.run_head(cfg, b, h, steps=steps, inputs=inputs)
        return b, h, steps, time.perf_counter() - t0


def cpu_share():
    """Host CPUs this process may run on (its affinity set), else os.cpu_count()."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def cpu_baseline(pool, procs, cfg, anchor_steps, steady_steps):
    """The fp64 oracle as it stands, timed on the host: one process per core, one BLAS thread
    each.  procs / 2 heads each run twice at once, as step 1 alone (the anchor) and as steps
    1-2 (anchor + one steady step; every steady step of the schedule has the same blocks), so
    a head's steady step is the difference of its two runs.  The per-step time of the whole
    workload on `procs` cores weights anchor and steady steps as the GPU run did and spreads
    the B*H heads over the cores (heads are independent)."""
    nh = max(1, procs // 2)
    heads = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)][:nh]
    jobs = [(cfg, b, h, n) for (b, h) in heads for n in (1, 2)]
    t1 = time.perf_counter()
    res = pool.map(_oracle_job, jobs, chunksize=1)
    wall = time.perf_counter() - t1
    one = {(b, h): t for b, h, n, t in res if n == 1}
    two = {(b, h): t for b, h, n, t in res if n == 2}
    t_anchor = float(np.median(list(one.values())))
    t_steady = float(np.median([two[k] - one[k] for k in heads]))
    per_head = (anchor_steps * t_anchor + steady_steps * t_steady) / (anchor_steps + steady_steps)
    ms_step = per_head * cfg.batch * cfg.heads / procs * 1e3
    dense = 4.0 * cfg.batch * cfg.heads * cfg.tokens ** 2 * cfg.head_dim
    return {
        "value": round(dense / (ms_step * 1e-3) / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": procs,
        "ms_per_step": round(ms_step, 1),
        "anchor_step_s_per_head": round(t_anchor, 3),
        "steady_step_s_per_head": round(t_steady, 3),
        "host_logical_cpus": os.cpu_count(),
        "cpu_share": cpu_share(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle (one process per core, 1 BLAS thread, {len(jobs)} "
                  f"processes): heads {heads[0]}..{heads[-1]} of {cfg.batch}x{cfg.heads}, each "
                  f"as step 1 alone and as steps 1-2; per-head step time weighted "
                  f"{anchor_steps} anchor : {steady_steps} steady as in the timed GPU steps, "
                  f"times {cfg.batch * cfg.heads} heads / {procs} cores (sample wall "
                  f"{wall:.1f} s)"}


def mask_work(M, reuse_ptr, n, bh, D, cache_elem=2):
    """(fresh FLOPs, cache read bytes, cache write bytes) of one step's plan (mask: 1 = fresh,
    2 = reuse; reuse_ptr: states read per row, a merged group counting once): 4 n_i n_j D
    per fresh block, n_i (D s_c + 4) bytes per state read or written, times B*H."""
    F = M == 1
    flops = float(4.0 * D * (n[:, None] * n[None, :])[F].sum()) * bh
    per_row = n * (D * cache_elem + 4)
    rd = float((np.diff(reuse_ptr) * per_row).sum()) * bh
    wr = float((F * per_row[:, None]).sum()) * bh
    return flops, rd, wr


def kernel_source_digest():
    """Digest of the kernel sources' code: comments and whitespace are left out, so that a
    comment edit keeps the stored counter figures valid."""
    h = hashlib.sha256()
    for f in ("dita_kernels.hip", "dita_internal.h"):
        with open(os.path.join(ROOT, "partial_state_reuse_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(digest, kernel, workload):
    """HBM bytes per launch of the dominant kernel (the fixed-reference pass of a steady step)
    from committed rocprofv3 FETCH_SIZE and WRITE_SIZE runs, each scaled by what the counter
    reads for a plain device copy of known size; only if they were taken on the current kernel
    source, the same kernel instantiation and the same workload (else None)."""
    path = os.path.join(ROOT, "profiles", "step_bf16_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_digest") != digest or t.get("kernel") != kernel or \
            not str(t.get("workload", "")).startswith(workload):
        return None
    return (t["fetch_size_kib_fixed_pass_mean"] * 1024 * t["fetch_scale"]
            + t["write_size_kib_fixed_pass_mean"] * 1024 * t["write_scale"])


def hbm_roofline(traffic, cache_bytes, kernel_ms):
    """The dominant kernel's HBM rate against the 8 TB/s peak: its counted traffic per launch
    (rocprofv3 FETCH_SIZE + WRITE_SIZE) when the stored counters match this kernel and
    workload, else its algorithmic cache bytes (reused states read + fresh states written
    back), each over its measured duration."""
    sec = kernel_ms * 1e-3
    cache_gbs = cache_bytes / sec / 1e9
    counted = traffic / sec / 1e9 if traffic else None
    achieved = counted if counted is not None else cache_gbs
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
            "basis": "rocprofv3 FETCH_SIZE + WRITE_SIZE" if counted is not None
            else "algorithmic cache bytes",
            "cache_algorithmic_gb_s": round(cache_gbs, 1)}


def time_offload(dita, cache, stream):
    """One offload of the cache's state to pinned host memory and its restore into a new
    device buffer, each timed with HIP events on the stream (host buffers allocated first)."""
    import ctypes
    import torch
    n = cache.offload_bytes()
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    new_buf = torch.empty(cache.required_bytes, dtype=torch.uint8, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    sh = ctypes.c_void_p(stream.cuda_stream)
    torch.cuda.synchronize()
    ev[0].record(stream)
    rc = dita._lib.dita_cache_offload(cache._h, ctypes.c_void_p(host.data_ptr()), n, sh)
    ev[1].record(stream)
    if rc:
        raise dita.DitaError(rc, dita._lib.dita_last_error().decode())
    ev[2].record(stream)
    rc = dita._lib.dita_cache_restore(cache._h, ctypes.c_void_p(new_buf.data_ptr()),
                                      cache.required_bytes, ctypes.c_void_p(host.data_ptr()),
                                      n, sh)
    ev[3].record(stream)
    if rc:
        raise dita.DitaError(rc, dita._lib.dita_last_error().decode())
    torch.cuda.synchronize()
    cache.buffer = new_buf
    d2h, h2d = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    return {"bytes": n, "d2h_ms": round(d2h, 3), "h2d_ms": round(h2d, 3),
            "d2h_gb_s": round(n / d2h / 1e6, 2), "h2d_gb_s": round(n / h2d / 1e6, 2),
            "note": "host link, pinned memory; outside the timed steps"}


def cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, then family / model / stepping
    (which identify the generation where the name is generic), or None."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break                          # the first processor's block only
                k, _, v = line.partition(":")
                fields[k.strip()] = v.strip()
    except OSError:
        return None
    name = fields.get("model name")
    if name is None:
        return None
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return name + (f" ({', '.join(ids)})" if ids else "")


def describe_policy(pol, P):
    """One-line description of a fixed block policy (for the bench line's config)."""
    from workloads import configs as wc
    if pol.anchor:
        d = "anchor (every active block fresh)"
    elif pol.kind == wc.FRAME_THRESHOLD:
        d = f"fresh iff frame distance <= {pol.max_fresh_frame_dist}, else reused"
    elif pol.kind == wc.CENTROID_THRESHOLD:
        d = f"fresh iff doubled centroid distance <= {pol.max_fresh_centroid2}, else reused"
    elif pol.kind == wc.FRESH_BUDGET:
        r = min((pol.reuse_percent * P + 50) // 100, P - 1)
        d = f"fresh budget {P - r}/{P} per row ({pol.reuse_percent} % reused)"
    else:
        d = f"policy kind {pol.kind}"
    return d + ("; tile-sparse 3D frame mask" if pol.tile_sparse else "")


def describe_schedule(cfg):
    """The workload's fixed schedule as runs of steps with one policy each."""
    parts, start = [], 1
    for s in range(1, cfg.steps + 1):
        if s == cfg.steps or cfg.policy(s + 1) != cfg.policy(s):
            rng = f"step {start}" if start == s else f"steps {start}-{s}"
            parts.append(f"{rng}: {describe_policy(cfg.policy(s), cfg.num_partitions)}")
            start = s + 1
    return "; ".join(parts)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3,
                    help="workload number (the bench line is workload 3; others for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--policy", choices=["schedule", "planner"], default="schedule",
                    help="schedule: the workload's fixed block schedule (the bench line); "
                         "planner: the selection planner at the same reuse budget")
    ap.add_argument("--cache", choices=["bf16", "fp8"], default="bf16",
                    help="cached O precision: bf16 (the bench line) or fp8 e4m3 (compressed)")
    ap.add_argument("--merge", type=str, default="",
                    help="comma-separated group sizes (e.g. 2,4): after each run's anchor step, "
                         "merge the cached states of every aligned key group that the schedule "
                         "reuses on all later steps, in that order (group composition)")
    ap.add_argument("--layout", choices=["bhnd", "bnhd"], default="bhnd",
                    help="layout of Q, K, V and out: [B, H, N, D] or [B, N, H, D] (the inputs "
                         "are staged in that layout before the timed region)")
    ap.add_argument("--out", choices=["f32", "bf16"], default="f32",
                    help="output element type: f32 (the bench line) or bf16 (rounded from the "
                         "f32 result in the epilogue)")
    ap.add_argument("--static-scratch", action="store_true",
                    help="run the steps through dita_attn_step_static (the variant that "
                         "allocates nothing; its scratch is a static device array)")
    ap.add_argument("--compact", action="store_true",
                    help="with --merge: after each run's merges, compact the cache onto one "
                         "slot per stored state (and expand it back before the next anchor)")
    ap.add_argument("--offload", action="store_true",
                    help="after the timed steps, time one offload of the cache's state to "
                         "pinned host memory and its restore into a new device buffer "
                         "(reported as `offload`, outside the timed region)")
    ap.add_argument("--planner-group", type=int, default=1)
    ap.add_argument("--planner-anchor-period", type=int, default=0)
    ap.add_argument("--workers", type=int, default=min(16, cpu_share()),
                    help="host processes for the input generator and the CPU baseline (one "
                         "per core; at most 16, the host share of one GPU)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (outside the timed "
                         "region) as the reference for hardware traffic counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU path only (the step runs every partition on "
              "one GPU; there is no multi-GPU mode): use --gpus 1", file=sys.stderr)
        sys.exit(2)

    cfg = CONFIGS[args.workload]
    if args.cache == "fp8":
        import dataclasses
        cfg = dataclasses.replace(cfg, cache_dtype="fp8")
    S = cfg.steps
    B, H, N, D = cfg.batch, cfg.heads, cfg.tokens, cfg.head_dim
    # the worker pool is forked before this process touches the GPU
    pool = mp.get_context("fork").Pool(args.workers)
    t_gen = time.perf_counter()

    import torch
    import partial_state_reuse_amd as dita

    bf = cfg.qkv_dtype == "bf16"
    dt = torch.bfloat16 if bf else torch.float32
    dev = [[torch.empty((B, H, N, D), dtype=dt, device="cuda") for _ in range(3)]
           for _ in range(S)]
    jobs = [(cfg, b, h, S) for b in range(B) for h in range(H)]
    for b, h, st in pool.imap_unordered(_gen_job, jobs):
        for s in range(S):
            for t in range(3):
                src = torch.from_numpy(st[s][t])
                dev[s][t][b, h].copy_(src.view(torch.bfloat16) if bf else src)
    if args.layout == "bnhd":
        dev = [[t.transpose(1, 2).contiguous() for t in step] for step in dev]
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] inputs staged in HBM: {S} steps x 3 x {B}x{H}x{N}x{D} {cfg.qkv_dtype} "
          f"({t_gen:.1f} s)", file=sys.stderr, flush=True)

    geom = dita.geometry_from(cfg, out_dtype=args.out)
    geom.layout = dita.LAYOUT_BNHD if args.layout == "bnhd" else dita.LAYOUT_BHND
    # blocks that can ever be non-skip: the anchor step's active set
    act = (dita.dita_policy_mask(geom, dita.policy_from(cfg.policy(1).as_anchor())) != 0)
    cache = dita.Cache(geom, active_mask=act.astype(np.uint8))
    out = torch.empty((B, N, H, D) if args.layout == "bnhd" else (B, H, N, D),
                      dtype=torch.bfloat16 if args.out == "bf16" else torch.float32,
                      device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    if args.policy == "planner":
        from workloads import Policy, PLANNER
        pct = cfg.policy(2).reuse_percent
        pl = Policy(kind=PLANNER, reuse_percent=pct, group_size=args.planner_group,
                    anchor_period=args.planner_anchor_period,
                    tile_sparse=cfg.policy(1).tile_sparse)
        policies = [dita.policy_from(pl)] * S
        schedule_desc = (f"selection planner: step 1 anchor, then {pct} % reuse chosen by "
                         f"predicted error (importance x growth), group size "
                         f"{args.planner_group}, anchor period {args.planner_anchor_period}")
    else:
        policies = [dita.policy_from(cfg.policy(s)) for s in range(1, S + 1)]
        schedule_desc = describe_schedule(cfg)
    n_part = np.diff(dita.dita_partition_offsets(geom).astype(np.int64)).astype(np.float64)
    merge_sizes = [int(x) for x in args.merge.split(",") if x]
    merge_sel = []
    if merge_sizes:
        if args.policy != "schedule":
            sys.exit("--merge applies to the fixed schedule")
        P = cfg.num_partitions
        later = [dita.dita_policy_mask(geom, policies[s], np.ones((P, P), np.uint8))
                 for s in range(1, S)]
        for g in merge_sizes:
            NG = (P + g - 1) // g
            sel = np.zeros((P, NG), np.uint8)
            for i in range(P):
                for J in range(NG):
                    sel[i, J] = all(M[i, j] == dita.REUSE for M in later
                                    for j in range(J * g, min(P, J * g + g)))
            merge_sel.append((g, sel))
        schedule_desc += "; after the anchor, cached states merged in groups of " + \
            " then ".join(str(g) for g in merge_sizes)
    dense_flops = 4.0 * B * H * N * N * D
    stream = torch.cuda.current_stream()
    step_masks = []

    compact_bytes = []
    if args.compact:
        if not merge_sizes:
            sys.exit("--compact applies with --merge")
        spare = [torch.empty(cache.required_bytes, dtype=torch.uint8, device="cuda")]

    def run_step(k):
        s = k % S
        if s == 0:
            if args.compact and cache.buffer.numel() < cache.required_bytes:
                # back to the full slot table (into the spare buffer) before the anchor
                old = cache.buffer
                cache.expand(buffer=spare[0], stream=stream)
                spare[0] = old
            cache.reset()
        cache.set_policy(policies[s])
        q, kk, v = dev[s]
        cache.step(q, kk, v, out=out, lse=lse, stream=stream,
                   static_scratch=args.static_scratch)
        # host copy of the step's plan (no device wait), taken after the launch so that it
        # adds nothing between a planner step's decision and its kernels
        pl = cache.plan()
        step_masks.append((pl["mask"], pl["reuse_ptr"]))
        if s == 0:
            for g, sel in merge_sel:
                cache.merge_groups(g, select=sel, stream=stream)
            if args.compact:
                # onto one slot per stored state, in a buffer held aside for it
                need = cache.compact_bytes()
                if spare[0].numel() < need or not compact_bytes:
                    spare[0] = torch.empty(need, dtype=torch.uint8, device="cuda")
                old = cache.buffer
                cache.compact(buffer=spare[0][:need] if spare[0].numel() > need else spare[0],
                              stream=stream)
                spare[0] = old
                compact_bytes.append(need)

    for k in range(args.warmup):
        run_step(k)
    torch.cuda.synchronize()
    if args.copy_mib:
        n = args.copy_mib << 20
        src_c = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst_c = torch.empty_like(src_c)
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c

    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    cache.set_profiling(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for k in range(args.warmup, args.warmup + K):
        run_step(k)
        ev[k - args.warmup + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = cache.stats()
    cache.set_profiling(False)

    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(K)]
    kinds = [(args.warmup + i) % S for i in range(K)]
    anchor_ms = [m for m, s in zip(step_ms, kinds) if s == 0]
    steady_ms = [m for m, s in zip(step_ms, kinds) if s != 0]
    ms_per_step = wall * 1e3 / K
    value = dense_flops * K / wall / 1e12

    cache_elem = {"bf16": 2, "fp8": 1}.get(cfg.cache_dtype, 4)
    work = [mask_work(m, rp, n_part, B * H, D, cache_elem) for m, rp in step_masks[-K:]]
    fresh_flops = sum(w[0] for w in work)
    cache_bytes = sum(w[1] + w[2] for w in work)
    kern_ms = st["step_kernel_ms"]
    prep_ms = st["prep_kernel_ms"]
    launches = st["profiled_steps"]
    avg_kernel_ms = kern_ms / max(launches, 1)
    # The dominant kernel: the fixed-reference pass, which every step after a reset's first
    # runs (each of its fresh blocks has a state from an earlier step), timed by the library's
    # HIP events around it on its launch stream (with the conditional second pass after it,
    # which exits at once unless a reference was rejected).  The first step after a reset
    # runs the running-maximum kernel alone; it is reported on its own.
    fixed_steps = st["fixed_ref_steps"]
    steady_work = [w for w, s in zip(work, kinds) if s != 0]
    anchor_work = [w for w, s in zip(work, kinds) if s == 0]
    bf16_path = cfg.qkv_dtype == "bf16"
    timing = "library HIP events around the step kernels"
    if args.static_scratch:
        # the allocation-free step records no events of its own: the steps' times between
        # this stream's events (transpose, both passes and the merges of each step)
        timing = "stream events between steps (the allocation-free step is not profiled)"
        launches = K
        kern_ms = float(sum(step_ms))
        fixed_steps = len(steady_ms)
        st = dict(st, fixed_ref_kernel_ms=float(sum(steady_ms)))
        avg_kernel_ms = kern_ms / K
    elif bf16_path and fixed_steps != len(steady_work):
        sys.exit(f"bench: {fixed_steps} steps ran the fixed-reference pass, expected "
                 f"{len(steady_work)} (the steps after each reset's first)")
    if bf16_path and fixed_steps:
        fixed_ms = st["fixed_ref_kernel_ms"] / fixed_steps
        steady_flops = sum(w[0] for w in steady_work) / len(steady_work)
        achieved = steady_flops / (fixed_ms * 1e-3) / 1e12
        dom_ms, dom_flops = fixed_ms, steady_flops
        dom_cache_bytes = sum(w[1] + w[2] for w in steady_work) / len(steady_work)
    else:
        achieved = fresh_flops / launches / (avg_kernel_ms * 1e-3) / 1e12
        dom_ms, dom_flops = avg_kernel_ms, fresh_flops / launches
        dom_cache_bytes = cache_bytes / K
    anchor_launches = launches - fixed_steps
    anchor_roof = None
    if bf16_path and anchor_launches and anchor_work:
        a_ms = (kern_ms - st["fixed_ref_kernel_ms"]) / anchor_launches
        a_flops = sum(w[0] for w in anchor_work) / len(anchor_work)
        a_ach = a_flops / (a_ms * 1e-3) / 1e12
        anchor_roof = {"kernel": kernel_label(D, args.policy == "planner",
                                              cfg.cache_dtype == "fp8", fixed=False),
                       "steps": anchor_launches, "kernel_ms": round(a_ms, 4),
                       "fresh_tflop": round(a_flops / 1e12, 4),
                       "achieved": round(a_ach, 2), "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(a_ach / PEAK_BF16_TFLOPS, 4)}
    digest = kernel_source_digest()
    label = kernel_label(D, args.policy == "planner", cfg.cache_dtype == "fp8")
    # the counter run covers the fixed schedule without merging, on [B, H, N, D] inputs
    traffic = measured_traffic(digest, label, cfg.name) \
        if args.policy == "schedule" and not merge_sizes and args.layout == "bhnd" else None
    t_roof_sum = sum(w[0] / (PEAK_BF16_TFLOPS * 1e12) + (w[1] + w[2]) / (PEAK_HBM_GBS * 1e9)
                     for w in work)
    t_roof_max = sum(max(w[0] / (PEAK_BF16_TFLOPS * 1e12), (w[1] + w[2]) / (PEAK_HBM_GBS * 1e9))
                     for w in work)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic (seeded generator; N(0,1) + 3D sinusoidal position term, "
                "0.05-sigma drift per step)",
        "config": {"workload": cfg.name, "batch": B, "heads": H, "tokens": N, "head_dim": D,
                   "partitions": cfg.num_partitions, "denoise_steps": S,
                   "schedule": schedule_desc,
                   "cache": f"{cfg.cache_dtype} O + f32 lse", "out": args.out,
                   "entry_point": "dita_attn_step_static" if args.static_scratch
                   else "dita_attn_step",
                   "layout": args.layout},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": label,
                     "launches": fixed_steps if bf16_path else launches,
                     "kernel_ms": round(dom_ms, 4),
                     "fresh_tflop_per_launch": round(dom_flops / 1e12, 4),
                     "timing": timing,
                     "kernel_source_digest": digest},
        "roofline_anchor": anchor_roof,
        "roofline_hbm": hbm_roofline(traffic, dom_cache_bytes, dom_ms),
        "roofline_combined": {
            "t_roof_ms_per_step": round(t_roof_sum * 1e3 / K, 4),
            "frac_sum_form": round(t_roof_sum / wall, 4),
            "frac_max_form": round(t_roof_max / wall, 4),
            "cache_gb_per_step": round(cache_bytes / K / 1e9, 4)},
        "breakdown": {
            "anchor_step_ms": round(float(np.median(anchor_ms)), 4) if anchor_ms else None,
            "steady_step_ms": round(float(np.median(steady_ms)), 4) if steady_ms else None,
            "step_kernels_ms_per_step": round(avg_kernel_ms, 4),
            "prep_kernel_ms_per_step": round(prep_ms / max(launches, 1), 4),
            "device_fresh_blocks": st["device_fresh_blocks"],
            "host_fresh_blocks": st["host_fresh_blocks"]},
    }

    if compact_bytes:
        result["compaction"] = {"full_buffer_bytes": cache.required_bytes,
                                "compacted_buffer_bytes": compact_bytes[-1],
                                "ratio": round(compact_bytes[-1] / cache.required_bytes, 4)}
    if args.offload:
        result["offload"] = time_offload(dita, cache, stream)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(pool, args.workers, cfg, len(anchor_ms),
                                              len(steady_ms))
    pool.close()
    pool.join()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
