"""Pins of the oracle's group composition (DiTango, "State-Centric Parallel Runtime /
Composizione Dinamica dei Gruppi": cached states merged recursively into coarser groups,
without recomputation), CPU only.

The composition is exact because states compose associatively: in float64 with no cache
rounding, reusing a merged group must give the same output as reusing its members one by
one, and merging in two levels (2, then 4) the same as merging groups of 4 at once."""
import numpy as np
import pytest

import oracle
from oracle.policy import FRESH, REUSE, active_mask, partition_offsets
from workloads import Policy, custom_config
import workloads.configs as wcfg


def _cfg():
    # 8 frames x 8 tokens, 8 partitions of one frame each; the frame-distance rule keeps
    # frames |f_i - f_j| <= 1 fresh and reuses the rest every step
    return custom_config(name="groups-tiny", idx=75, heads=1, head_dim=16, frames=8, grid_h=2,
                         grid_w=4, num_partitions=8, steps=5, qkv_dtype="f32", cache_dtype="f32",
                         schedule=wcfg.AnchorThen(Policy(kind=wcfg.FRAME_THRESHOLD,
                                                         max_fresh_frame_dist=1)))


def _always_reused(runs, P, g):
    """select[i, J] for groups whose every member is REUSE at every step after the first."""
    NG = (P + g - 1) // g
    sel = np.ones((P, NG), bool)
    for st in runs[1:]:
        for i in range(P):
            for J in range(NG):
                if any(st.mask[i, j] != REUSE for j in range(J * g, min(P, J * g + g))):
                    sel[i, J] = False
    return sel


def test_merged_reuse_equals_member_reuse_fp64():
    cfg = _cfg()
    P = cfg.num_partitions
    base = oracle.run_head(cfg, 0, 0, cache_mode="fp64")
    sel = _always_reused(base, P, 2)
    assert sel.sum() > 4
    merged = oracle.run_head(cfg, 0, 0, cache_mode="fp64", merges={1: [(2, sel)]})
    for a, b in zip(base, merged):
        assert np.array_equal(a.mask, b.mask)
        assert np.allclose(a.out, b.out, atol=1e-12, rtol=0)
        assert np.allclose(a.lse, b.lse, atol=1e-12, rtol=0)
    # each merged pair is read once from step 2 on
    for a, b in zip(base[1:], merged[1:]):
        assert len(b.reuse_cols) == len(a.reuse_cols) - int(sel.sum())


def test_two_level_merge_equals_direct_merge():
    cfg = _cfg()
    P = cfg.num_partitions
    base = oracle.run_head(cfg, 0, 0, cache_mode="fp64")
    s2, s4 = _always_reused(base, P, 2), _always_reused(base, P, 4)
    assert s4.sum() > 0
    two = oracle.run_head(cfg, 0, 0, cache_mode="fp64", merges={1: [(2, s2), (4, s4)]})
    one = oracle.run_head(cfg, 0, 0, cache_mode="fp64", merges={1: [(4, s4)]})
    for a, b, c in zip(two, one, base):
        assert np.allclose(a.out, b.out, atol=1e-12, rtol=0)
        assert np.allclose(a.out, c.out, atol=1e-12, rtol=0)
    # a group of 4 fully inside the selection is read once
    for a, b in zip(two[1:], one[1:]):
        assert len(a.reuse_cols) <= len(b.reuse_cols)


def test_fresh_member_recomputes_the_whole_group():
    cfg = _cfg()
    P = cfg.num_partitions
    base = oracle.run_head(cfg, 0, 0, cache_mode="fp64")
    # merge every eligible pair after step 1, then make step 3 fresh on (5, 0) only
    pol = [cfg.policy(s) for s in range(1, cfg.steps + 1)]
    M3 = np.array(base[2].mask)
    M3[5, 0] = FRESH
    pol[2] = Policy(kind=wcfg.EXPLICIT, explicit_mask=tuple(int(x) for x in M3.ravel()))
    run = oracle.run_head(cfg, 0, 0, cache_mode="fp64", merges={1: [(2, None)]}, policies=pol)
    assert run[2].mask[5, 0] == FRESH and run[2].mask[5, 1] == FRESH   # (5, 1) joins
    # the group is dissolved: at step 4 both members are reused from their own states
    assert run[3].mask[5, 0] == REUSE and run[3].mask[5, 1] == REUSE
    assert {0, 1} <= set(run[3].reuse_cols[run[3].reuse_ptr[5]:run[3].reuse_ptr[6]].tolist())


def test_groups_holding_the_diagonal_or_an_unwritten_state_are_not_merged():
    cfg = _cfg()
    P = cfg.num_partitions
    offs = partition_offsets(cfg.tokens, P)
    cache, head = {}, {}
    rng = np.random.default_rng(0)
    for i in range(P):
        for j in range(P):
            if j != 3:
                cache[(i, j)] = (rng.standard_normal((8, 16)), rng.standard_normal(8), 1)
    act = np.ones((P, P), bool)
    n = oracle.attention.merge_groups(cache, head, P, act, 2, None, lambda a: a, lambda a: a, 1)
    # per row 4 pairs; the pair holding i never merges, nor does the pair (2, 3) (no state
    # at 3) -- for rows 2 and 3 those are the same pair
    assert n == sum(4 - len({i // 2, 1}) for i in range(P))
    assert head.get((0, 3), 3) == 3 and (0, 2) not in head
