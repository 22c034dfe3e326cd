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


def round_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even to OCP fp8 e4m3fn, saturating at +-448, widened back to float64.

    e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; normal values
    (1 + m/8) 2^(e-7) for e = 1..15 (largest 448 = 1.75 * 2^8), subnormals m/8 * 2^-6 (spacing
    2^-9), no infinity.  In a binade [2^k, 2^(k+1)), k >= -6, the spacing is 2^(k-3); below
    2^-6 it is 2^-9.  Values are rounded to a multiple of the spacing with ties to even."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_fp8_e4m3: non-finite input")
    ax = np.abs(x)
    k = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    spacing = np.exp2(np.maximum(k, -6.0) - 3.0)
    r = np.round(ax / spacing) * spacing           # numpy rounds halves to even
    r = np.minimum(r, 448.0)
    return np.copysign(r, x)


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
    block_o: dict = field(default_factory=dict)     # (i, j) -> O rows used (keep_block_lse)


def merge_groups(cache, head, P, act, group, select, rho_o, rho_l, step):
    """Group composition (DiTango, "Composizione Dinamica dei Gruppi"): per query partition
    i and aligned key group J of `group` partitions, merge the cached states of the group
    into one, kept at its first active member; head[(i, j)] then names that member for every
    member.  Eligible: J does not hold i, every active member has a state, the group covers
    at least two states, and no state inside J also covers a block outside it.
    Returns the number of groups merged."""
    n = 0
    NG = (P + group - 1) // group
    for i in range(P):
        for J in range(NG):
            j0, j1 = J * group, min(P, J * group + group)
            if j0 <= i < j1 or (select is not None and not select[i][J]):
                continue
            members = [j for j in range(j0, j1) if act[i, j]]
            if not members or any((i, j) not in cache for j in members):
                continue
            hs = sorted({head.get((i, j), j) for j in members})
            if len(hs) < 2 or any(not (j0 <= x < j1) for x in hs):
                continue
            if any(head.get((i, j), j) in hs for j in range(P) if not (j0 <= j < j1)):
                continue
            O, L = merge_states([cache[(i, x)][:2] for x in hs])
            dst = members[0]
            cache[(i, dst)] = (rho_o(O), rho_l(L), step)
            for j in members:
                head[(i, j)] = dst
            n += 1
    return n


def run_head(cfg, b: int, h: int, steps: int | None = None, rows=None,
             cache_mode: str = "emulate", policies=None, inputs=None, offsets=None,
             drift=None, keep_block_lse: bool = False, merges=None, active=None):
    """Run the denoising steps of one (b, h) and return a list of OracleStep.

    rows        None (all tokens) or a sorted array of global token indices to evaluate;
                rows are independent, so a subset gives exactly those rows' results.
    cache_mode  "emulate": cache O rounded to the workload's cache precision (bf16 / f32)
                and lse to float32; "fp64": no rounding.
    policies    optional list of per-step policies (default: the workload's schedule).
    inputs      optional list of per-step (Q, K, V) [N, D]; default: the seeded generator.
    merges      optional {step: [(group, select or None), ...]}: group compositions applied
                after that step (see merge_groups).  A merged group is then reused as one
                state, and a step that makes any member fresh recomputes every member.
    active      boolean [P, P] of blocks owning a cache slot (default: all).
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
        rho_o = {"bf16": round_bf16, "fp8": round_fp8_e4m3}.get(cfg.cache_dtype, round_f32)
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
    head = {}                                    # (i, j) -> block holding its merged state
    act = np.ones((P, P), dtype=bool) if active is None else np.asarray(active, dtype=bool)
    results = []
    for s in range(1, n_steps + 1):
        Qs, Ks, Vs = (np.asarray(t, dtype=np.float64) for t in get(s))
        pol = cfg.policy(s) if policies is None else policies[s - 1]
        valid = np.zeros((P, P), dtype=bool)
        for (i, j) in cache:
            valid[i, j] = True
        M = policy_mask(offs, cfg.frame_tokens, pol, valid)
        # merged groups are reused or recomputed as a whole
        covered = {k for k, v in head.items() if v != k[1]}
        for (i, j) in covered:
            hb = (i, head[(i, j)])
            if M[i, j] == FRESH or M[hb] == FRESH:
                M[i, j] = FRESH
                M[hb] = FRESH
        for (i, j) in covered:
            hb = (i, head[(i, j)])
            if M[hb] == FRESH:
                M[i, j] = FRESH
            if M[i, j] != M[hb]:
                raise ValueError(f"merged block ({i},{j}) not decided with its group")
        fp, fc, rp, rc, counts = work_lists(M)
        if covered:
            rp, rc = [0], []
            for i in range(P):
                rc += [j for j in range(P) if M[i, j] == REUSE and (i, j) not in covered]
                rp.append(len(rc))
            rp, rc = np.array(rp, dtype=np.int32), np.array(rc, dtype=np.int32)
        out = np.zeros((len(rows), D))
        lse = np.full(len(rows), -np.inf)
        blk = {}
        blk_o = {}
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
                    head.pop((i, j), None)
                elif (i, j) in covered:
                    continue                     # its group's state is read once, at its head
                else:
                    O_ij, l_ij, _ = cache[(i, j)]
                states.append((O_ij, l_ij))
                if keep_block_lse:
                    blk[(i, j)] = l_ij
                    blk_o[(i, j)] = O_ij
            if len(r):
                o_i, L_i = merge_states(states)
                out[pos:pos + len(r)] = o_i
                lse[pos:pos + len(r)] = L_i
            pos += len(r)
        results.append(OracleStep(s, M, fp, fc, rp, rc, counts, rows, out, lse, blk, blk_o))
        for (g, sel) in (merges or {}).get(s, []):
            merge_groups(cache, head, P, act, g, sel, rho_o, rho_l, s)
    return results
