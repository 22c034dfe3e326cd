"""Oracle side of the selection planner: importance, growth, predicted error, group decision.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows DiTango (gist.science 2607.15650), "Metodologia > 1. Anchor-Guided Selection
Planner", which names the ingredients but gives no formulas; the readings below are the
plainest ones the rest of the pages support:

  * error model ("Modellazione dell'Errore"): the error of reusing a state from an earlier
    step is a function of the partition's importance w and the temporal growth delta.  Read
    as E_ij = w_ij * (drift of the state since block (i, j) was last fresh), the drift being
    the accumulated growth;
  * importance: the share of a query row's softmax mass that falls in key partition j,
    w_ij = mean over (b, h, r in partition i) of exp(lse_ij[r] - L_i[r]), measured on anchor
    steps, which refresh it ("Anchor Steps");
  * growth ("Predizione Online"): the local state (the diagonal block, always computed)
    stands in for the remote states; delta_i(t) is the root mean square change of the
    cached diagonal state O_ii from step t-1 to t, over (b, h, rows, dims).  The growth of
    the step being planned is predicted as the last measured one;
  * groups ("Strategia per Gruppi"): spatially adjacent partitions form groups of G, and a
    decision covers a whole block group (I, J): high-error groups are computed, the rest
    reused, within a per-row budget.

Decision arithmetic (predicted errors, group sums, ranking) is done in float64 in the same
order as the library's, so that the two take identical decisions from identical inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .attention import block_state, merge_states, round_bf16, round_f32, round_fp8_e4m3
from .policy import FRESH, REUSE, SKIP, active_mask, partition_offsets, PolicyError

PLANNER = 4


def importance(block_lse: dict, act: np.ndarray) -> np.ndarray:
    """w [P, P] from the lse of every active block of an anchor step.

    block_lse[(i, j)] is an array of lse values (natural log) of the rows of partition i,
    all (b, h) concatenated in the same order for every j."""
    P = act.shape[0]
    w = np.zeros((P, P))
    for i in range(P):
        cols = [j for j in range(P) if act[i, j]]
        lses = np.stack([np.asarray(block_lse[(i, j)], dtype=np.float64) for j in cols])
        top = lses.max(axis=0)
        L = top + np.log(np.exp(lses - top).sum(axis=0))     # row log-sum-exp over blocks
        for k, j in enumerate(cols):
            w[i, j] = np.mean(np.exp(lses[k] - L))
    return w


def growth(new_diag: dict, old_diag: dict, D: int) -> np.ndarray:
    """delta [P]: RMS over all (b, h), rows and the first D dims of new - old cached O_ii.

    new_diag[i] / old_diag[i] are arrays [..., rows, >= D] (all heads stacked)."""
    P = len(new_diag)
    out = np.zeros(P)
    for i in range(P):
        d = np.asarray(new_diag[i], dtype=np.float64)[..., :D] - \
            np.asarray(old_diag[i], dtype=np.float64)[..., :D]
        out[i] = np.sqrt(np.mean(d * d))
    return out


def predicted_errors(w, delta_hist, fresh_step, valid, s: int) -> np.ndarray:
    """E [P, P] (float64) for planning step s (1-based since the reset).

    w          [P, P] importance (float32 values, widened exactly)
    delta_hist [s-1, P] measured growth delta_i(t), row t-1 for step t (0: not measured)
    fresh_step [P, P] step at which each block was last fresh (0 = never)
    E_ij = w_ij * ((Cum_i(s-1) - Cum_i(f_ij)) + delta_i(s-1)), Cum summed in step order."""
    w = np.asarray(w, dtype=np.float32)
    delta_hist = np.asarray(delta_hist, dtype=np.float64)
    P = w.shape[0]
    E = np.zeros((P, P))
    for i in range(P):
        cum = [0.0]
        for t in range(1, s):
            cum.append(cum[-1] + float(delta_hist[t - 1, i]))
        last = float(delta_hist[s - 2, i])
        for j in range(P):
            f = int(fresh_step[i, j])
            if not valid[i, j] or f <= 0:
                continue
            drift = (cum[s - 1] - cum[f]) + last
            E[i, j] = float(w[i, j]) * drift
    return E


def planner_mask(offsets, frame_tokens: int, policy, E, valid, anchor: bool) -> np.ndarray:
    """uint8 [P, P] mask of a planner step: block groups (I, J) of G partitions decided as
    units.  FRESH: the diagonal group, groups with a member whose slot holds no state, groups
    with summed error above max_error (if > 0), then the largest-error groups (ties: smaller
    J) until A - R are fresh, R = min(floor((pct A + 50) / 100), A - 1)."""
    P = len(offsets) - 1
    act = active_mask(offsets, frame_tokens, policy.tile_sparse)
    valid = np.zeros((P, P), bool) if valid is None else np.asarray(valid, dtype=bool)
    pct = policy.reuse_percent
    if not 0 <= pct <= 100:
        raise PolicyError("reuse_percent outside 0..100")
    G = max(1, int(getattr(policy, "group_size", 1) or 1))
    max_error = float(getattr(policy, "max_error", 0.0) or 0.0)
    groups = [list(range(g0, min(P, g0 + G))) for g0 in range(0, P, G)]
    M = np.zeros((P, P), dtype=np.uint8)
    for I, gi in enumerate(groups):
        cand = []                                # (J, summed error, forced fresh)
        for J, gj in enumerate(groups):
            members = [(i, j) for i in gi for j in gj if act[i, j]]
            if not members:
                continue
            e = 0.0
            for (i, j) in members:               # i ascending, then j ascending
                if not anchor and i != j:
                    e += float(E[i, j])
            invalid = any(not valid[i, j] for (i, j) in members)
            forced = anchor or J == I or invalid or (max_error > 0.0 and e > max_error)
            cand.append((J, e, forced))
        A = len(cand)
        n_reuse = min((pct * A + 50) // 100, A - 1)
        fresh = {J for (J, e, forced) in cand if forced}
        for (J, e, forced) in sorted((c for c in cand if not c[2]), key=lambda c: (-c[1], c[0])):
            if len(fresh) < A - n_reuse:
                fresh.add(J)
        for (J, e, forced) in cand:
            for i in gi:
                for j in groups[J]:
                    if act[i, j]:
                        M[i, j] = FRESH if J in fresh else REUSE
    for i in range(P):
        if M[i, i] != FRESH:
            raise PolicyError(f"diagonal block ({i},{i}) is not fresh")
    return M


@dataclass
class PlannerStep:
    step: int
    anchor: bool
    mask: np.ndarray
    out: dict = field(default_factory=dict)        # (b, h) -> [N, D]
    lse: dict = field(default_factory=dict)        # (b, h) -> [N]
    w: np.ndarray | None = None                    # importance measured at this (anchor) step
    delta: np.ndarray | None = None                # growth measured at this step (s >= 2)


def run_planner(cfg, heads, policy, steps=None, cache_mode="emulate", masks=None, inputs=None,
                offsets=None):
    """Run the planner schedule over the listed (b, h) pairs (all of them: the decision is
    shared by every head, and its measurements average over them).

    masks   optional list of per-step masks to use instead of the planner's own decisions
            (for replaying a device run); the measurements are still taken.
    inputs  optional dict (b, h) -> list of per-step (Q, K, V)."""
    n_steps = cfg.steps if steps is None else steps
    N, D = cfg.tokens, cfg.head_dim
    offs = partition_offsets(N, cfg.num_partitions) if offsets is None else list(offsets)
    P = len(offs) - 1
    tau = 1.0 / np.sqrt(D)
    act = active_mask(offs, cfg.frame_tokens, policy.tile_sparse)
    if cache_mode == "fp64":
        rho_o, rho_l = (lambda a: np.array(a, dtype=np.float64)), (lambda a: np.array(a))
    else:
        rho_o = {"bf16": round_bf16, "fp8": round_fp8_e4m3}.get(cfg.cache_dtype, round_f32)
        rho_l = round_f32
    if inputs is None:
        from workloads.gen import HeadStream
        streams = {bh: HeadStream(cfg, bh[0], bh[1]) for bh in heads}
        get = lambda bh, s: streams[bh].step_tensors(s)
    else:
        get = lambda bh, s: inputs[bh][s - 1]

    cache = {bh: {} for bh in heads}               # (i, j) -> (O, lse)
    fresh_step = np.zeros((P, P), dtype=np.int64)
    w = np.zeros((P, P), dtype=np.float32)
    have_w = False
    delta_hist = []
    A = int(getattr(policy, "anchor_period", 0) or 0)
    results = []
    for s in range(1, n_steps + 1):
        valid = fresh_step > 0
        anchor = bool(policy.anchor) or s == 1 or not have_w or (A > 0 and (s - 1) % A == 0)
        if masks is not None:
            M = np.asarray(masks[s - 1], dtype=np.uint8)
        else:
            E = None if anchor else predicted_errors(w, np.array(delta_hist).reshape(-1, P),
                                                     fresh_step, valid, s)
            M = planner_mask(offs, cfg.frame_tokens, policy, E, valid, anchor)
        st = PlannerStep(s, anchor, M)
        block_lse = {}
        new_diag, old_diag = {i: [] for i in range(P)}, {i: [] for i in range(P)}
        for bh in heads:
            Qs, Ks, Vs = (np.asarray(t, dtype=np.float64) for t in get(bh, s))
            out = np.zeros((N, D))
            lse = np.zeros(N)
            for i in range(P):
                r = slice(offs[i], offs[i + 1])
                states = []
                for j in range(P):
                    if M[i, j] == SKIP:
                        continue
                    if M[i, j] == FRESH:
                        sl = slice(offs[j], offs[j + 1])
                        O_ij, l_ij = block_state(Qs[r], Ks[sl], Vs[sl], tau)
                        stored = (rho_o(O_ij), rho_l(l_ij))
                        if j == i and s >= 2:
                            old_diag[i].append(cache[bh][(i, i)][0])
                            new_diag[i].append(stored[0])
                        cache[bh][(i, j)] = stored
                        block_lse.setdefault((i, j), []).append(stored[1])
                    else:
                        O_ij, l_ij = cache[bh][(i, j)]
                    states.append((O_ij, l_ij))
                o_i, L_i = merge_states(states)
                out[r] = o_i
                lse[r] = L_i
            st.out[bh] = out
            st.lse[bh] = lse
        if s >= 2:
            st.delta = growth({i: np.stack(new_diag[i]) for i in range(P)},
                              {i: np.stack(old_diag[i]) for i in range(P)}, D)
            delta_hist.append(st.delta)
        else:
            delta_hist.append(np.zeros(P))
        if anchor:
            st.w = importance({k: np.concatenate(v) for k, v in block_lse.items()}, act)
            w = st.w.astype(np.float32)
            have_w = True
        for i in range(P):
            for j in range(P):
                if M[i, j] == FRESH:
                    fresh_step[i, j] = s
        results.append(st)
    return results
