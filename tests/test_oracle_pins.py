"""Pins of the fp64 oracle against facts fixed by the pages and by the mathematics.

Each test names the fact it pins.  Page facts (DiTango, gist.science 2607.15650):
  * attention states (output, log-sum-exp) compose associatively and commutatively
    ("State-Centric Parallel Runtime / Composizione dello Stato");
  * anchor steps recompute every partition; the local partition is always computed
    ("Anchor-Guided Selection Planner");
  * reuse takes a state from an earlier step (same section, error model);
Efficient-vDiT (chatpaper abstract): tile-style sparse 3D attention, linear in frames.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from oracle.policy import (EXPLICIT, FRAME_THRESHOLD, FRESH, REUSE, SKIP, PolicyError,
                           active_mask, partition_offsets, policy_mask, work_lists)
from workloads import CONFIGS, Policy, custom_config


def sdpa64(q, k, v, mask=None):
    """torch's scaled_dot_product_attention in float64 on the CPU (library routine)."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))[None, None]
    am = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=am)
    return o[0, 0].numpy()


def lse64(q, k, mask=None):
    z = torch.from_numpy(q @ k.T / math.sqrt(q.shape[1]))
    if mask is not None:
        z = z.masked_fill(~torch.from_numpy(mask), float("-inf"))
    return torch.logsumexp(z, dim=1).numpy()


def rand_inputs(rng, steps, N, D, drift=0.3):
    base = [rng.standard_normal((N, D)) for _ in range(3)]
    out = []
    for s in range(steps):
        if s:
            base = [x + drift * rng.standard_normal((N, D)) for x in base]
        out.append(tuple(x.copy() for x in base))
    return out


def explicit(M):
    return Policy(kind=EXPLICIT, explicit_mask=tuple(int(x) for x in np.asarray(M).ravel()))


# ----------------------------------------------------------------------------------------
# P1: all-fresh, no skip == dense softmax attention
# ----------------------------------------------------------------------------------------
@pytest.mark.parametrize("N,D,P", [(37, 8, 5), (64, 16, 4), (90, 12, 7)])
def test_p1_all_fresh_is_dense_attention(N, D, P):
    rng = np.random.default_rng(N * 100 + D)
    cfg = custom_config(head_dim=D, frames=1, grid_h=1, grid_w=N, num_partitions=P, steps=1)
    inputs = rand_inputs(rng, 1, N, D)
    res = oracle.run_head(cfg, 0, 0, cache_mode="fp64", inputs=inputs,
                          policies=[Policy(kind=FRAME_THRESHOLD, anchor=True)])
    q, k, v = inputs[0]
    assert np.max(np.abs(res[0].out - sdpa64(q, k, v))) < 1e-12
    assert np.max(np.abs(res[0].lse - lse64(q, k))) < 1e-12


def test_p1_tiny_workload_anchor_step_is_dense_attention():
    cfg = CONFIGS[1]
    res = oracle.run_head(cfg, 0, 1, steps=1, cache_mode="fp64")
    from workloads.gen import head_steps
    q, k, v = (np.asarray(a, np.float64) for a in head_steps(cfg, 0, 1, steps=1)[0])
    assert np.max(np.abs(res[0].out - sdpa64(q, k, v))) < 1e-12


# ----------------------------------------------------------------------------------------
# P2: merging the states of any split, in any order, gives the unsplit state
# ----------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(6))
def test_p2_split_and_merge_order_invariance(seed):
    rng = np.random.default_rng(seed)
    r, n, D = 7, 53, 6
    q, k, v = (rng.standard_normal((m, D)) * 2 for m in (r, n, n))
    tau = 1 / math.sqrt(D)
    whole = oatt.block_state(q, k, v, tau)
    # random (non-contiguous) key groups, including singletons
    perm = rng.permutation(n)
    cuts = np.sort(rng.choice(np.arange(1, n), size=rng.integers(1, 12), replace=False))
    groups = np.split(perm, cuts)
    states = [oatt.block_state(q, k[g], v[g], tau) for g in groups]
    order = rng.permutation(len(states))
    merged = oatt.merge_states([states[i] for i in order])
    assert np.max(np.abs(merged[0] - whole[0])) < 1e-12
    assert np.max(np.abs(merged[1] - whole[1])) < 1e-12
    # associativity: merge of merges
    half = len(order) // 2
    if half:
        m1 = oatt.merge_states([states[i] for i in order[:half]])
        m2 = oatt.merge_states([states[i] for i in order[half:]])
        mm = oatt.merge_states([m2, m1])
        assert np.max(np.abs(mm[0] - whole[0])) < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_p2_random_ragged_partitions_all_fresh(seed):
    rng = np.random.default_rng(50 + seed)
    N, D = 41, 8
    cuts = np.sort(rng.choice(np.arange(1, N), size=6, replace=False))
    offs = [0] + [int(c) for c in cuts] + [N]           # includes size-1 partitions maybe
    cfg = custom_config(head_dim=D, frames=1, grid_h=1, grid_w=N, num_partitions=7, steps=1)
    inputs = rand_inputs(rng, 1, N, D)
    res = oracle.run_head(cfg, 0, 0, cache_mode="fp64", inputs=inputs, offsets=offs,
                          policies=[Policy(kind=FRAME_THRESHOLD, anchor=True)])
    q, k, v = inputs[0]
    assert np.max(np.abs(res[0].out - sdpa64(q, k, v))) < 1e-12


# ----------------------------------------------------------------------------------------
# P3: brute force over the closed "mixed-time" form on tiny inputs
# ----------------------------------------------------------------------------------------
def brute_force(inputs, offs, masks, D):
    """Scalar loops, no blocking, no log-sum-exp helper.  Row r of partition i at step s
    attends over the union of key partitions j it does not skip; block (i, j) uses the
    query row, keys and values of the step t_ij at which the block was last fresh."""
    P = len(offs) - 1
    N = offs[-1]
    tau = 1.0 / math.sqrt(D)
    last = {}
    outs = []
    for s, M in enumerate(masks):
        for i in range(P):
            for j in range(P):
                if M[i][j] == 1:
                    last[(i, j)] = s
        out = [[0.0] * D for _ in range(N)]
        for i in range(P):
            for r in range(offs[i], offs[i + 1]):
                terms = []                       # (logit, value row)
                for j in range(P):
                    if M[i][j] == 0:
                        continue
                    t = last[(i, j)]
                    Q, K, V = inputs[t]
                    for c in range(offs[j], offs[j + 1]):
                        z = 0.0
                        for d in range(D):
                            z += Q[r][d] * K[c][d]
                        terms.append((tau * z, V[c]))
                denom = 0.0
                for z, _ in terms:
                    denom += math.exp(z)
                for z, vrow in terms:
                    w = math.exp(z) / denom
                    for d in range(D):
                        out[r][d] += w * vrow[d]
        outs.append(np.array(out))
    return outs


def random_masks(rng, P, steps, skip_p=0.25):
    masks = []
    valid = np.zeros((P, P), dtype=bool)
    for s in range(steps):
        M = np.zeros((P, P), dtype=np.uint8)
        for i in range(P):
            for j in range(P):
                if i == j:
                    M[i, j] = FRESH
                    continue
                u = rng.random()
                if u < skip_p:
                    M[i, j] = SKIP
                elif valid[i, j] and u < skip_p + (1 - skip_p) / 2:
                    M[i, j] = REUSE
                else:
                    M[i, j] = FRESH
        valid |= M == FRESH
        masks.append(M)
    return masks


def p3_error(seed):
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.integers(12, 49))
    D = int(rng.integers(2, 9))
    P = int(rng.integers(2, 6))
    S = 3
    cuts = np.sort(rng.choice(np.arange(1, N), size=P - 1, replace=False))
    offs = [0] + [int(c) for c in cuts] + [N]
    inputs = rand_inputs(rng, S, N, D, drift=0.5)
    masks = random_masks(rng, P, S)
    cfg = custom_config(head_dim=D, frames=1, grid_h=1, grid_w=N, num_partitions=P, steps=S)
    res = oracle.run_head(cfg, 0, 0, cache_mode="fp64", inputs=inputs, offsets=offs,
                          policies=[explicit(M) for M in masks])
    bf = brute_force(inputs, offs, masks, D)
    return max(np.max(np.abs(r.out - b)) for r, b in zip(res, bf))


@pytest.mark.parametrize("seed", range(8))
def test_p3_brute_force_mixed_time(seed):
    assert p3_error(seed) < 1e-12


# ----------------------------------------------------------------------------------------
# P4: reuse of an unchanged state is a no-op
# ----------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(3))
def test_p4_no_drift_reuse_is_noop(seed):
    rng = np.random.default_rng(200 + seed)
    N, D, P, S = 40, 8, 5, 4
    base = tuple(rng.standard_normal((N, D)) for _ in range(3))
    inputs = [base] * S
    masks = random_masks(rng, P, S, skip_p=0.0)
    cfg = custom_config(head_dim=D, frames=1, grid_h=1, grid_w=N, num_partitions=P, steps=S)
    res = oracle.run_head(cfg, 0, 0, cache_mode="fp64", inputs=inputs,
                          policies=[explicit(M) for M in masks])
    for r in res[1:]:
        assert np.array_equal(r.out, res[0].out)          # bit-identical in pure fp64
        assert np.array_equal(r.lse, res[0].lse)


def test_p4_no_drift_tiny_workload_with_cache_rounding():
    cfg = CONFIGS[1]
    res = oracle.run_head(cfg, 0, 0, drift=0.0)            # f32 cache rounding emulated
    assert np.max(np.abs(res[1].out - res[0].out)) < 1e-6
    cfg3 = custom_config(head_dim=16, frames=4, grid_h=3, grid_w=4, num_partitions=4,
                         steps=2, qkv_dtype="bf16", cache_dtype="bf16",
                         schedule=CONFIGS[1].schedule)
    res = oracle.run_head(cfg3, 0, 0, drift=0.0)
    # bf16 cache: reused states carry at most half an ulp of bf16 each
    assert np.max(np.abs(res[1].out - res[0].out)) < 2e-2
    assert 0 < np.max(np.abs(res[1].out - res[0].out))


# ----------------------------------------------------------------------------------------
# P5: tile mask with everything fresh == dense attention under the boolean frame mask
# ----------------------------------------------------------------------------------------
@pytest.mark.parametrize("T", [3, 5, 7])
def test_p5_tile_mask_is_masked_dense_attention(T):
    gh, gw, D = 2, 3, 8
    F = gh * gw
    N = T * F
    cfg = custom_config(head_dim=D, frames=T, grid_h=gh, grid_w=gw, num_partitions=T, steps=1)
    rng = np.random.default_rng(T)
    inputs = rand_inputs(rng, 1, N, D)
    res = oracle.run_head(cfg, 0, 0, cache_mode="fp64", inputs=inputs,
                          policies=[Policy(kind=FRAME_THRESHOLD, tile_sparse=True,
                                           anchor=True)])
    frame = np.arange(N) // F
    fq, fk = frame[:, None], frame[None, :]
    tok_mask = (fk == fq) | (fk == 0) | (np.abs(fk - fq) == 1)
    q, k, v = inputs[0]
    assert np.max(np.abs(res[0].out - sdpa64(q, k, v, tok_mask))) < 1e-12
    assert np.max(np.abs(res[0].lse - lse64(q, k, tok_mask))) < 1e-12


# ----------------------------------------------------------------------------------------
# P6: merge weights sum to one; outputs stay inside the range of the values used
# ----------------------------------------------------------------------------------------
def test_p6_weights_and_convex_hull():
    rng = np.random.default_rng(7)
    N, D, P, S = 36, 6, 4, 3
    inputs = rand_inputs(rng, S, N, D, drift=1.0)
    masks = random_masks(rng, P, S, skip_p=0.2)
    cfg = custom_config(head_dim=D, frames=1, grid_h=1, grid_w=N, num_partitions=P, steps=S)
    offs = partition_offsets(N, P)
    res = oracle.run_head(cfg, 0, 0, cache_mode="fp64", inputs=inputs,
                          policies=[explicit(M) for M in masks], keep_block_lse=True)
    last = {}
    for s, r in enumerate(res):
        M = masks[s]
        for i in range(P):
            for j in range(P):
                if M[i, j] == FRESH:
                    last[(i, j)] = s
        for i in range(P):
            rows = slice(offs[i], offs[i + 1])
            wsum = sum(np.exp(r.block_lse[(i, j)] - r.lse[rows])
                       for j in range(P) if M[i, j] != SKIP)
            assert np.max(np.abs(wsum - 1.0)) < 1e-12
            used = np.concatenate([inputs[last[(i, j)]][2][offs[j]:offs[j + 1]]
                                   for j in range(P) if M[i, j] != SKIP])
            lo, hi = used.min(axis=0), used.max(axis=0)
            assert np.all(r.out[rows] >= lo - 1e-12) and np.all(r.out[rows] <= hi + 1e-12)


# ----------------------------------------------------------------------------------------
# P9: heads are independent; the mask is shared by every (b, h)
# ----------------------------------------------------------------------------------------
def test_p9_head_permutation():
    cfg = CONFIGS[1]
    r0 = oracle.run_head(cfg, 0, 0)
    r1 = oracle.run_head(cfg, 0, 1)
    from workloads.gen import head_steps
    i0, i1 = head_steps(cfg, 0, 0), head_steps(cfg, 0, 1)
    s0 = oracle.run_head(cfg, 0, 0, inputs=i1)           # head 1's inputs in slot 0
    for a, b in zip(s0, r1):
        assert np.array_equal(a.out, b.out)
    for a, b in zip(r0, r1):
        assert np.array_equal(a.mask, b.mask)
    assert not np.allclose(r0[1].out, r1[1].out)


# ----------------------------------------------------------------------------------------
# P10: CFG constant shift: V1 = V0 + 0.1 with shared Q, K gives O1 - O0 = 0.1 exactly
# ----------------------------------------------------------------------------------------
def test_p10_cfg_constant_shift():
    rng = np.random.default_rng(11)
    N, D, P, S = 30, 5, 3, 3
    in0 = rand_inputs(rng, S, N, D)
    in1 = [(q, k, v + 0.1) for q, k, v in in0]
    masks = random_masks(rng, P, S, skip_p=0.2)
    cfg = custom_config(head_dim=D, frames=1, grid_h=1, grid_w=N, num_partitions=P, steps=S)
    pol = [explicit(M) for M in masks]
    r0 = oracle.run_head(cfg, 0, 0, cache_mode="fp64", inputs=in0, policies=pol)
    r1 = oracle.run_head(cfg, 1, 0, cache_mode="fp64", inputs=in1, policies=pol)
    for a, b in zip(r0, r1):
        assert np.max(np.abs(b.out - a.out - 0.1)) < 1e-12
        assert np.array_equal(a.lse, b.lse)


# ----------------------------------------------------------------------------------------
# Rounding helpers against torch's conversions (library routines)
# ----------------------------------------------------------------------------------------
def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * 10.0 ** rng.integers(-6, 6, 200000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oatt.round_bf16(x.astype(np.float64)), want)
    # exact ties round to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert oatt.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert oatt.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # just above the tie rounds up (a value float32 cannot hold: no double rounding)
    assert oatt.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1 + 2.0 ** -7


def test_round_f32_hand_worked_values():
    """Round-to-nearest-even to float32 (24 significant bits) on values worked out by hand,
    so that truncation, rounding half away from zero or half up, or a lost sign fail."""
    u = 2.0 ** -23                     # float32 spacing in [1, 2)
    cases = [
        (1 + u / 2, 1.0),              # tie between 1 and 1 + u: the even one, 1
        (1 + 3 * u / 2, 1 + 2 * u),    # tie between 1 + u and 1 + 2u: the even one, 1 + 2u
        (1 + u / 2 + 2.0 ** -40, 1 + u),   # just above a tie: up
        (1 + u / 2 - 2.0 ** -40, 1.0),     # just below a tie: down
        (-(1 + 3 * u / 2), -(1 + 2 * u)),  # the same tie, negative
        (2 - 2.0 ** -25, 2.0),         # above the midpoint 2 - 2^-24 of [2 - u, 2]: up to 2
        (2 - 3 * 2.0 ** -25, 2 - u),   # below that midpoint: down to 2 - u
        # 1/3 = 2^-25 * (2^25 / 3) and 2^25 / 3 = 11184810.67 has 24 significant bits
        (1.0 / 3.0, 11184811 * 2.0 ** -25),
        (1.5 * 2.0 ** -149, 2.0 ** -148),  # subnormal tie between 1 and 2 units: 2 (even)
        (2.0 ** -150, 0.0),            # subnormal tie between 0 and 1 unit: 0 (even)
        (1.0 + 2.0 ** -30, 1.0),
        (-7.25, -7.25),                # exact values stay
    ]
    x = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    got = oatt.round_f32(x)
    assert np.array_equal(got, want), list(zip(x, got, want))
    assert np.signbit(oatt.round_f32(np.array([-(2.0 ** -150)])))[0]   # rounds to -0


# ----------------------------------------------------------------------------------------
# Planted mistakes: each plausible slip in the oracle's arithmetic fails a pin above
# ----------------------------------------------------------------------------------------
def _mut_reversed_values(q, k, v, tau):
    return ORIG_BLOCK(q, k, v[::-1], tau)


def _mut_no_scale(q, k, v, tau):
    return ORIG_BLOCK(q, k, v, 1.0)


def _mut_lse_without_log(q, k, v, tau):
    o, lse = ORIG_BLOCK(q, k, v, tau)
    z = tau * (np.asarray(q) @ np.asarray(k).T)
    return o, z.max(axis=1)


def _mut_unnormalised(q, k, v, tau):
    o, lse = ORIG_BLOCK(q, k, v, tau)
    z = tau * (np.asarray(q) @ np.asarray(k).T)
    return o * np.exp(z - z.max(axis=1, keepdims=True)).sum(axis=1)[:, None], lse


def _mut_merge_sign(states):
    o, L = ORIG_MERGE(states)
    flipped = [(s[0], -s[1]) for s in states]
    return ORIG_MERGE(flipped)[0], L


ORIG_BLOCK = oatt.block_state
ORIG_MERGE = oatt.merge_states


@pytest.mark.parametrize("mutant", [_mut_reversed_values, _mut_no_scale,
                                    _mut_lse_without_log, _mut_unnormalised,
                                    _mut_merge_sign])
def test_planted_mistakes_fail_a_pin(monkeypatch, mutant):
    if mutant is _mut_merge_sign:
        monkeypatch.setattr(oatt, "merge_states", mutant)
    else:
        monkeypatch.setattr(oatt, "block_state", mutant)
    errs = [p3_error(seed) for seed in range(3)]
    assert max(errs) > 1e-6, "brute-force pin did not catch the planted mistake"
