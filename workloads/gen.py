"""Seeded synthetic Q/K/V generator shared by the oracle's tests, the GPU tests and the bench.

It holds no attention arithmetic: it only draws inputs.  The recipe:

  * token position (t, y, x), flattened frame-major then row-major;
  * a sinusoidal position term PE in R^D.  3D: channel blocks [t | y | x] of widths
    d_t = D - 2*d_y, d_y = d_x = 2*floor(D/6).  2D (one frame): [y | x] with d_y = d_x = D/2.
    Inside a block of width w, channel pair k holds (sin(a*p), cos(a*p)) with
    a = 10000^(-2k/w) and integer position p;
  * X_1 = N(0,1) + scale * PE for X in {Q, K, V}: the same PE for the three tensors, every
    head and the whole batch, with independent noise;
  * drift: X_s = X_{s-1} + drift * N(0,1), accumulated on an fp32 master; bf16 workloads
    round each step's master to bf16 (round-to-nearest-even);
  * CFG workload: Q and K are shared by the two batch entries; V[b] = V[0] + offset * eps
    for b >= 1, eps ~ N(0,1) drawn once and kept for all steps;
  * seeds: numpy.random.default_rng([workload, tensor, b, h, step]) (PCG64), tensor 0 = Q,
    1 = K, 2 = V, 3 = CFG offset; step 0 is the base draw, step s >= 2 the drift of step s.
"""
from __future__ import annotations

import numpy as np

from .configs import Config

Q, K, V, CFG_EPS = 0, 1, 2, 3


def _sincos_block(pos: np.ndarray, width: int) -> np.ndarray:
    out = np.zeros((pos.shape[0], width), dtype=np.float64)
    for k in range(width // 2):
        a = 10000.0 ** (-2.0 * k / width)
        out[:, 2 * k] = np.sin(a * pos)
        out[:, 2 * k + 1] = np.cos(a * pos)
    return out


def position_term(cfg: Config) -> np.ndarray:
    """PE [N, D] float64 for the workload's token grid."""
    D = cfg.head_dim
    t, y, x = np.meshgrid(np.arange(cfg.frames), np.arange(cfg.grid_h),
                          np.arange(cfg.grid_w), indexing="ij")
    t, y, x = (a.reshape(-1).astype(np.float64) for a in (t, y, x))
    if cfg.pe_mode == "3d":
        dy = 2 * (D // 6)
        dt = D - 2 * dy
        blocks = [_sincos_block(t, dt), _sincos_block(y, dy), _sincos_block(x, dy)]
    elif cfg.pe_mode == "2d":
        if cfg.frames != 1:
            raise ValueError("2d position term needs a single frame")
        blocks = [_sincos_block(y, D // 2), _sincos_block(x, D - D // 2)]
    else:
        raise ValueError(cfg.pe_mode)
    return np.concatenate(blocks, axis=1)


def _noise(cfg: Config, tensor: int, b: int, h: int, step: int) -> np.ndarray:
    rng = np.random.default_rng([cfg.idx, tensor, b, h, step])
    return rng.standard_normal((cfg.tokens, cfg.head_dim), dtype=np.float32)


def round_bf16_via_torch(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (RNE) -> fp32, done by torch's conversion (input recipe only)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()


class HeadStream:
    """Iterates the per-step inputs of one (b, h).

    `step_tensors(s)` returns (Q, K, V) as float32 arrays [N, D] holding the exact values
    the step uses (bf16-representable for bf16 workloads).  Steps must be requested in
    increasing order starting at 1 (the master is accumulated as it goes).
    """

    def __init__(self, cfg: Config, b: int, h: int, pe32: np.ndarray | None = None,
                 drift: float | None = None):
        self.cfg, self.b, self.h = cfg, b, h
        self.drift = cfg.drift if drift is None else drift
        if pe32 is None:
            pe32 = (cfg.pe_scale * position_term(cfg)).astype(np.float32)
        self._pe32 = pe32
        self._step = 0
        self._master = None
        self._eps = None

    def _src_b(self, tensor: int) -> int:
        # Q and K (and V's own noise) are shared across the batch in the CFG workload.
        return 0 if self.cfg.cfg_v_offset != 0.0 else self.b

    def step_tensors(self, s: int):
        cfg = self.cfg
        if s != self._step + 1:
            raise ValueError(f"steps must be consecutive: have {self._step}, asked {s}")
        if s == 1:
            self._master = [(_noise(cfg, t, self._src_b(t), self.h, 0) + self._pe32)
                            .astype(np.float32) for t in (Q, K, V)]
        else:
            if self.drift != 0.0:
                d = np.float32(self.drift)
                for t in (Q, K, V):
                    self._master[t] = (self._master[t]
                                       + d * _noise(cfg, t, self._src_b(t), self.h, s)
                                       ).astype(np.float32)
        self._step = s
        out = list(self._master)
        if cfg.cfg_v_offset != 0.0 and self.b >= 1:
            if self._eps is None:
                self._eps = _noise(cfg, CFG_EPS, 0, self.h, 0)
            out[V] = (out[V] + np.float32(cfg.cfg_v_offset) * self._eps).astype(np.float32)
        if cfg.qkv_dtype == "bf16":
            out = [round_bf16_via_torch(x) for x in out]
        return tuple(out)


def head_steps(cfg: Config, b: int, h: int, steps: int | None = None, drift=None):
    """List over steps 1..steps of (Q, K, V) float32 [N, D] for one (b, h)."""
    hs = HeadStream(cfg, b, h, drift=drift)
    n = cfg.steps if steps is None else steps
    return [hs.step_tensors(s) for s in range(1, n + 1)]


def _gen_head_job(args):
    cfg, b, h, steps, drift = args
    return (b, h, head_steps(cfg, b, h, steps, drift))


def all_steps(cfg: Config, steps: int | None = None, workers: int = 1, drift=None):
    """Full [steps][3] list of float32 arrays [B, H, N, D].

    `workers` > 1 draws heads in a process pool (each head's stream is independent)."""
    n = cfg.steps if steps is None else steps
    B, H, N, D = cfg.batch, cfg.heads, cfg.tokens, cfg.head_dim
    out = [[np.empty((B, H, N, D), np.float32) for _ in range(3)] for _ in range(n)]
    jobs = [(cfg, b, h, n, drift) for b in range(B) for h in range(H)]
    if workers > 1:
        import multiprocessing as mp
        ctx = mp.get_context("fork")
        with ctx.Pool(workers) as pool:
            results = pool.imap_unordered(_gen_head_job, jobs)
            for b, h, st in results:
                for s in range(n):
                    for t in range(3):
                        out[s][t][b, h] = st[s][t]
    else:
        for job in jobs:
            b, h, st = _gen_head_job(job)
            for s in range(n):
                for t in range(3):
                    out[s][t][b, h] = st[s][t]
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-representable")
    return (u >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def head_steps_packed(cfg: Config, b: int, h: int, steps: int | None = None):
    """Like head_steps, but bf16 workloads come back as uint16 bit patterns (half the
    bytes to move between processes); f32 workloads as float32."""
    st = head_steps(cfg, b, h, steps)
    if cfg.qkv_dtype == "bf16":
        return [tuple(bf16_bits(x) for x in s) for s in st]
    return st
