"""Oracle side of the block policy: partition map, active set, fresh/reuse/skip mask, work lists.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Integer arithmetic throughout.

Definitions followed:
  * contiguous context partitions of the frame-major token sequence (DiTango, "Problematica":
    context parallelism splits the sequence; lay summary: the video sequence is cut into
    segments); ragged sizes follow the numpy array_split rule;
  * the frame of a partition is the frame holding its centre token, computed on doubled
    centroids C_p = o_p + o_{p+1} - 1 so everything stays integer: f_p = C_p // (2 F);
  * tile-sparse active set (Efficient-vDiT abstract): query frame f attends to frames f,
    0 and f +- 1 only;
  * anchor steps: every active block is fresh (DiTango, "Anchor steps");
  * the local (diagonal) block is always fresh (DiTango, "Predizione Online");
  * a reused block needs a state written at an earlier step.
"""
from __future__ import annotations

import numpy as np

SKIP, FRESH, REUSE = 0, 1, 2

# policy kinds
EXPLICIT, FRAME_THRESHOLD, FRESH_BUDGET, CENTROID_THRESHOLD = 0, 1, 2, 3


class PolicyError(ValueError):
    """The requested mask is not a valid step plan."""


def partition_offsets(tokens: int, parts: int) -> list[int]:
    """o_0 = 0 < ... < o_P = N; the first N mod P partitions hold one extra token."""
    if not (1 <= parts <= tokens):
        raise PolicyError("need 1 <= partitions <= tokens")
    sizes = [tokens // parts + (1 if p < tokens % parts else 0) for p in range(parts)]
    offs = [0]
    for s in sizes:
        offs.append(offs[-1] + s)
    return offs


def centroids2(offsets) -> list[int]:
    """Doubled centroid of each partition: first + last token index."""
    return [offsets[p] + offsets[p + 1] - 1 for p in range(len(offsets) - 1)]


def partition_frames(offsets, frame_tokens: int) -> list[int]:
    return [c // (2 * frame_tokens) for c in centroids2(offsets)]


def active_mask(offsets, frame_tokens: int, tile_sparse: bool) -> np.ndarray:
    """Boolean [P, P]: blocks that may be computed or reused (not skipped)."""
    P = len(offsets) - 1
    act = np.ones((P, P), dtype=bool)
    if tile_sparse:
        f = partition_frames(offsets, frame_tokens)
        for i in range(P):
            for j in range(P):
                act[i, j] = f[j] == f[i] or f[j] == 0 or abs(f[j] - f[i]) == 1
    return act


def policy_mask(offsets, frame_tokens: int, policy, valid=None) -> np.ndarray:
    """uint8 [P, P] mask in {SKIP, FRESH, REUSE} for one step.

    `policy` carries kind / thresholds / tile_sparse / anchor / explicit_mask (the fields of
    workloads.Policy).  `valid` is a boolean [P, P] of slots holding a state from an earlier
    step (None = nothing cached yet).  Raises PolicyError when the plan is invalid.
    """
    P = len(offsets) - 1
    C = centroids2(offsets)
    f = partition_frames(offsets, frame_tokens)
    act = active_mask(offsets, frame_tokens, policy.tile_sparse)
    M = np.zeros((P, P), dtype=np.uint8)
    if policy.kind == EXPLICIT:
        if policy.explicit_mask is None or len(policy.explicit_mask) != P * P:
            raise PolicyError("explicit mask must have P*P entries")
        M = np.array(policy.explicit_mask, dtype=np.int64).reshape(P, P)
        if M.min() < 0 or M.max() > 2:
            raise PolicyError("mask value outside {0,1,2}")
        M = M.astype(np.uint8)
        if np.any((M != SKIP) & ~act):
            raise PolicyError("non-skip block outside the active set")
        if policy.anchor:
            M = np.where(M != SKIP, FRESH, SKIP).astype(np.uint8)
    else:
        for i in range(P):
            cols = [j for j in range(P) if act[i, j]]
            if policy.anchor:
                fresh = set(cols)
            elif policy.kind == FRAME_THRESHOLD:
                fresh = {j for j in cols if abs(f[i] - f[j]) <= policy.max_fresh_frame_dist}
            elif policy.kind == CENTROID_THRESHOLD:
                fresh = {j for j in cols if abs(C[i] - C[j]) <= policy.max_fresh_centroid2}
            elif policy.kind == FRESH_BUDGET:
                A = len(cols)
                pct = policy.reuse_percent
                if not 0 <= pct <= 100:
                    raise PolicyError("reuse_percent outside 0..100")
                n_reuse = min((pct * A + 50) // 100, A - 1)
                ranked = sorted(cols, key=lambda j: (abs(f[i] - f[j]), abs(C[i] - C[j]), j))
                fresh = set(ranked[:A - n_reuse])
            else:
                raise PolicyError(f"unknown policy kind {policy.kind}")
            for j in cols:
                M[i, j] = FRESH if j in fresh else REUSE
            M[i, i] = FRESH  # the local partition is always computed
    # validation
    for i in range(P):
        if M[i, i] != FRESH:
            raise PolicyError(f"diagonal block ({i},{i}) is not fresh")
    if np.any(M == REUSE):
        if valid is None or np.any((M == REUSE) & ~np.asarray(valid, dtype=bool)):
            raise PolicyError("reuse of a block with no cached state")
    return M


def work_lists(M: np.ndarray):
    """Per-row CSR lists: fresh_ptr[P+1], fresh_cols, reuse_ptr[P+1], reuse_cols (ascending
    j within a row) and counts [skip, fresh, reuse]."""
    P = M.shape[0]
    fp, fc, rp, rc = [0], [], [0], []
    for i in range(P):
        for j in range(P):
            if M[i, j] == FRESH:
                fc.append(j)
            elif M[i, j] == REUSE:
                rc.append(j)
        fp.append(len(fc))
        rp.append(len(rc))
    counts = [int(np.sum(M == SKIP)), int(np.sum(M == FRESH)), int(np.sum(M == REUSE))]
    as32 = lambda a: np.array(a, dtype=np.int32)
    return as32(fp), as32(fc), as32(rp), as32(rc), as32(counts)
