"""Oracle side of the attention arithmetic: block states, log-sum-exp merge, the step loop.

TEST INFRASTRUCTURE ONLY (see the package docstring).  float64 numpy throughout.

Definitions followed (DiTango, gist.science 2607.15650, "State-Centric Parallel Runtime /
Composizione dello Stato"; "Anchor-Guided Selection Planner"):

  state of block (i, j) for query row r of partition i over key partition j:
      z_c   = tau * q_r . k_c            for c in partition j
      lse   = log sum_c exp(z_c)
      O     = sum_c exp(z_c - lse) v_c   (normalised within the block)
  composition of the states of one row over its non-skipped blocks:
      L     = log sum_j exp(lse_j)
      out   = sum_j exp(lse_j - L) O_j
  a fresh block recomputes its state from this step's Q, K, V and writes it to its cache
  slot (rounded to the cache precision); a reused block reads the state its slot holds,
  i.e. the one from the step where the block was last fresh.  The step's own merge uses the
  unrounded fresh states.  tau = 1/sqrt(D) (the pages do not state the scale).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .policy import (FRESH, REUSE, SKIP, partition_offsets, policy_mask, work_lists)


def block_state(q: np.ndarray, k: np.ndarray, v: np.ndarray, tau: float):
    """(O [r, D], lse [r]) of query rows q [r, D] over keys k [n, D] / values v [n, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    z = tau * (q @ k.T)
    mu = z.max(axis=1)
    e = np.exp(z - mu[:, None])
    ell = e.sum(axis=1)
    lse = mu + np.log(ell)
    out = (e @ v) / ell[:, None]
    return out, lse


def merge_states(states):
    """Log-sum-exp composition of a list of (O [r, D], lse [r]) states of the same rows.
    An empty list, or rows whose every lse is -inf, give O = 0 and L = -inf."""
    if not states:
        raise ValueError("merge_states needs at least one state")
    lses = np.stack([s[1] for s in states], axis=0)           # [k, r]
    outs = np.stack([s[0] for s in states], axis=0)           # [k, r, D]
    top = lses.max(axis=0)
    finite = np.isfinite(top)
    safe_top = np.where(finite, top, 0.0)
    w = np.exp(lses - safe_top[None, :])                      # [k, r]
    tot = w.sum(axis=0)
    L = np.where(finite, safe_top + np.log(np.where(finite, tot, 1.0)), -np.inf)
    wn = np.where(finite[None, :], w / np.where(finite, tot, 1.0)[None, :], 0.0)
    out = np.einsum("kr,krd->rd", wn, outs)
    return out, L


def round_f32(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even to float32, widened back to float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even from float64 straight to bfloat16 (8 significant bits),
    widened back to float64.  Values must be finite and zero or of normal float32 size."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_bf16: non-finite input")
    ax = np.abs(x)
    if np.any((ax != 0) & (ax < 2.0 ** -126)):
        raise ValueError("round_bf16: value below the normal float32 range")
    bits = x.view(np.uint64)
    drop = np.uint64(45)                          # 52 - 7 stored mantissa bits
    lsb = (bits >> drop) & np.uint64(1)
    half_minus_one = np.uint64((1 << 44) - 1)     # half of the dropped unit, minus 1
    rounded = (bits + (half_minus_one + lsb)) & ~np.uint64((1 << 45) - 1)
    return rounded.view(np.float64)


@dataclass
class OracleStep:
    step: int
    mask: np.ndarray                  # uint8 [P, P]
    fresh_ptr: np.ndarray
    fresh_cols: np.ndarray
    reuse_ptr: np.ndarray
    reuse_cols: np.ndarray
    counts: np.ndarray                # [skip, fresh, reuse]
    rows: np.ndarray                  # global token indices of the evaluated rows
    out: np.ndarray                   # float64 [len(rows), D]
    lse: np.ndarray                   # float64 [len(rows)]
    block_lse: dict = field(default_factory=dict)   # (i, j) -> lse rows used this step


def run_head(cfg, b: int, h: int, steps: int | None = None, rows=None,
             cache_mode: str = "emulate", policies=None, inputs=None, offsets=None,
             drift=None, keep_block_lse: bool = False):
    """Run the denoising steps of one (b, h) and return a list of OracleStep.

    rows        None (all tokens) or a sorted array of global token indices to evaluate;
                rows are independent, so a subset gives exactly those rows' results.
    cache_mode  "emulate": cache O rounded to the workload's cache precision (bf16 / f32)
                and lse to float32; "fp64": no rounding.
    policies    optional list of per-step policies (default: the workload's schedule).
    inputs      optional list of per-step (Q, K, V) [N, D]; default: the seeded generator.
    """
    n_steps = cfg.steps if steps is None else steps
    N, D = cfg.tokens, cfg.head_dim
    offs = partition_offsets(N, cfg.num_partitions) if offsets is None else list(offsets)
    P = len(offs) - 1
    tau = 1.0 / np.sqrt(D)
    rows = np.arange(N) if rows is None else np.asarray(sorted(rows), dtype=np.int64)
    part_rows = [rows[(rows >= offs[i]) & (rows < offs[i + 1])] for i in range(P)]
    if cache_mode == "fp64":
        rho_o, rho_l = (lambda a: np.array(a, dtype=np.float64)), (lambda a: np.array(a))
    elif cache_mode == "emulate":
        rho_o = round_bf16 if cfg.cache_dtype == "bf16" else round_f32
        rho_l = round_f32
    else:
        raise ValueError(cache_mode)
    if inputs is None:
        from workloads.gen import HeadStream
        stream = HeadStream(cfg, b, h, drift=drift)
        get = stream.step_tensors
    else:
        get = lambda s: inputs[s - 1]

    cache = {}                                   # (i, j) -> (O, lse, step)
    results = []
    for s in range(1, n_steps + 1):
        Qs, Ks, Vs = (np.asarray(t, dtype=np.float64) for t in get(s))
        pol = cfg.policy(s) if policies is None else policies[s - 1]
        valid = np.zeros((P, P), dtype=bool)
        for (i, j) in cache:
            valid[i, j] = True
        M = policy_mask(offs, cfg.frame_tokens, pol, valid)
        fp, fc, rp, rc, counts = work_lists(M)
        out = np.zeros((len(rows), D))
        lse = np.full(len(rows), -np.inf)
        blk = {}
        pos = 0
        for i in range(P):
            r = part_rows[i]
            states = []
            for j in range(P):
                if M[i, j] == SKIP:
                    continue
                if M[i, j] == FRESH:
                    sl = slice(offs[j], offs[j + 1])
                    O_ij, l_ij = block_state(Qs[r], Ks[sl], Vs[sl], tau)
                    cache[(i, j)] = (rho_o(O_ij), rho_l(l_ij), s)
                else:
                    O_ij, l_ij, _ = cache[(i, j)]
                states.append((O_ij, l_ij))
                if keep_block_lse:
                    blk[(i, j)] = l_ij
            if len(r):
                o_i, L_i = merge_states(states)
                out[pos:pos + len(r)] = o_i
                lse[pos:pos + len(r)] = L_i
            pos += len(r)
        results.append(OracleStep(s, M, fp, fc, rp, rc, counts, rows, out, lse, blk))
    return results
