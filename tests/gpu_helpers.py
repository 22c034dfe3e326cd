"""Shared pieces of the GPU parity tests: input upload, the HIP run, the oracle run on the
same inputs, and the comparison with the tolerances of the workloads."""
from __future__ import annotations

import multiprocessing as mp
import os
import sys
import time

import numpy as np

from workloads.gen import bits_to_f32, head_steps_packed

# bf16 inputs with fp32 accumulation vs the fp64 oracle (pure fp64 cache).  With a bf16 cache
# the bar leaves room for half a bf16 ulp of every cached state (<= 2^-6 while |O| < 8) plus
# the fresh arithmetic error.
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-5


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


_POOL = None


def start_pool(workers=None):
    """Fork the generator pool (call before the process initialises the GPU)."""
    global _POOL
    if _POOL is None:
        n = workers or min(16, os.cpu_count() or 1)
        _POOL = mp.get_context("fork").Pool(n)
    return _POOL


def stop_pool():
    global _POOL
    if _POOL is not None:
        _POOL.close()
        _POOL.join()
        _POOL = None


def _job(args):
    cfg, b, h, steps = args
    return b, h, head_steps_packed(cfg, b, h, steps)


def _iter_heads(cfg, steps, heads):
    jobs = [(cfg, b, h, steps) for b, h in heads]
    if _POOL is not None and len(jobs) > 1:
        return _POOL.imap_unordered(_job, jobs)
    return map(_job, jobs)


def _as_f32(cfg, x):
    return bits_to_f32(x) if cfg.qkv_dtype == "bf16" else x


def host_inputs(cfg, steps, heads=None):
    """{(b, h): [(Q, K, V) per step]} float32 from the seeded generator."""
    heads = heads or [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    out = {}
    for b, h, st in _iter_heads(cfg, steps, heads):
        out[(b, h)] = [tuple(_as_f32(cfg, x) for x in s) for s in st]
    return out


def device_inputs(cfg, steps, keep_heads=(), device="cuda"):
    """Per-step device tensors (q, k, v) [B,H,N,D] in the workload dtype, plus the float32
    host copies of the heads in `keep_heads`."""
    import torch
    B, H, N, D = cfg.batch, cfg.heads, cfg.tokens, cfg.head_dim
    bf = cfg.qkv_dtype == "bf16"
    dt = torch.bfloat16 if bf else torch.float32
    heads = [(b, h) for b in range(B) for h in range(H)]
    dev = [[torch.empty((B, H, N, D), dtype=dt, device=device) for _ in range(3)]
           for _ in range(steps)]
    kept = {}
    for b, h, st in _iter_heads(cfg, steps, heads):
        for s in range(steps):
            for t in range(3):
                src = torch.from_numpy(st[s][t])
                dev[s][t][b, h].copy_(src.view(torch.bfloat16) if bf else src)
        if (b, h) in keep_heads:
            kept[(b, h)] = [tuple(_as_f32(cfg, x) for x in s) for s in st]
    return dev, kept


def sample_rows(offs, per_part, rng):
    """First two, last two and `per_part` random rows of every partition."""
    rows = set()
    for p in range(len(offs) - 1):
        lo, hi = offs[p], offs[p + 1]
        for r in (lo, lo + 1, hi - 2, hi - 1):
            if lo <= r < hi:
                rows.add(r)
        n = hi - lo
        for r in rng.choice(n, size=min(per_part, n), replace=False):
            rows.add(lo + int(r))
    return np.array(sorted(rows), dtype=np.int64)


# Longest block, in keys, held to the fp32 bar as stated: the small fp32 workload's blocks.
F32_STATED_KEYS = 64


def f32_bar(n_keys, vmax):
    """Max-abs bar of the f32 path for blocks of up to n_keys keys and values up to vmax:
    exactly 1e-5 (the bar stated for the small fp32 workload) for blocks of up to its 64 keys;
    for longer blocks, four standard deviations of the random walk of sequential fp32
    accumulation, 4 sqrt(n) 2^-24 max|V|, if that is larger."""
    if n_keys <= F32_STATED_KEYS:
        return F32_MAX_ABS
    return max(F32_MAX_ABS, 4.0 * np.sqrt(float(n_keys)) * 2.0 ** -24 * float(vmax))


def compare(got, want, bf16, what, f32_max=F32_MAX_ABS):
    err = np.abs(np.asarray(got, np.float64) - want)
    mx, mean = float(err.max()), float(err.mean())
    if bf16:
        ok = mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS
    else:
        ok = mx <= f32_max
    log(f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e} {'ok' if ok else 'FAIL'}")
    return ok, mx, mean


def bf16_ulp(x):
    """Spacing of bfloat16 values (8 significant bits) at |x|."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def bf16_out_bars(want):
    """Bars of a bf16 output against the fp64 reference `want`.  The kernel rounds its f32
    result o to bf16 (nearest even), which moves it by at most half a bf16 ulp at |o|, so
    |rne(o) - want| <= |o - want| + ulp(|o|) / 2, with |o| <= |want| + 2e-2 by the f32
    output's own bar.  Elementwise: 2e-2 + ulp(|want| + 2e-2) / 2; mean: 2e-3 plus the mean of
    those half ulps."""
    half = bf16_ulp(np.abs(np.asarray(want, np.float64)) + BF16_MAX_ABS) / 2
    return BF16_MAX_ABS + half, BF16_MEAN_ABS + float(half.mean())


def compare_cached(got, want_rounded, want_exact, bf16, what, f32_max=F32_MAX_ABS):
    """Cached states are rounded on both sides: round(a) and round(b) can differ by the
    arithmetic error |a - b| plus one ulp at the value, so the elementwise bar is the output
    bar plus one bf16 ulp of the exact value; the mean bar is unchanged."""
    err = np.abs(np.asarray(got, np.float64) - want_rounded)
    if bf16:
        ok = bool(np.all(err <= BF16_MAX_ABS + bf16_ulp(want_exact))) and \
            float(err.mean()) <= BF16_MEAN_ABS
    else:
        ok = float(err.max()) <= f32_max
    log(f"{what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e} {'ok' if ok else 'FAIL'}")
    return ok
