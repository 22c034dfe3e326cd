"""Pins of the oracle's block policy: closed-form counts, hand-derived masks, the
linear-in-frames active set (Efficient-vDiT abstract) and the validation rules
(DiTango, "Anchor-Guided Selection Planner": the local partition is always computed;
reuse needs a state from an earlier step)."""
import numpy as np
import pytest

from oracle.policy import (EXPLICIT, FRAME_THRESHOLD, FRESH, REUSE, SKIP, PolicyError,
                           active_mask, centroids2, partition_frames, partition_offsets,
                           policy_mask, work_lists)
from tests.golden import fixtures
from workloads import CONFIGS, Policy, custom_config
import workloads

BY_NAME = {c.name: c for c in CONFIGS.values()}


def masks_for(cfg, steps=None):
    offs = partition_offsets(cfg.tokens, cfg.num_partitions)
    P = cfg.num_partitions
    valid = np.zeros((P, P), dtype=bool)
    out = []
    for s in range(1, (steps or cfg.steps) + 1):
        M = policy_mask(offs, cfg.frame_tokens, cfg.policy(s), valid)
        valid |= M == FRESH
        out.append(M)
    return out


def test_offsets_array_split_rule():
    assert partition_offsets(26520, 16)[:3] == [0, 1658, 3316]
    offs = partition_offsets(26520, 16)
    sizes = np.diff(offs)
    assert list(sizes) == [1658] * 8 + [1657] * 8
    assert [len(a) for a in np.array_split(np.arange(26520), 16)] == list(sizes)
    for n, p in [(28800, 32), (86400, 24), (4096, 8), (256, 4), (41, 7)]:
        assert list(np.diff(partition_offsets(n, p))) == \
            [len(a) for a in np.array_split(np.arange(n), p)]
    # the workloads module's helper agrees with the oracle's own
    assert workloads.partition_offsets(26520, 16) == offs


def test_cfg_workload_partition_frames():
    cfg = CONFIGS[5]
    offs = partition_offsets(cfg.tokens, cfg.num_partitions)
    assert partition_frames(offs, cfg.frame_tokens) == \
        [0, 1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15, 16]


@pytest.mark.parametrize("key", sorted(fixtures.counts().keys()))
def test_p7_counts(key):
    name, step = key
    cfg = BY_NAME[name]
    M = masks_for(cfg, step)[step - 1]
    counts = list(work_lists(M)[4])
    assert counts == fixtures.counts()[key]


@pytest.mark.parametrize("key", sorted(fixtures.masks().keys()))
def test_p7_explicit_masks(key):
    name, step = key
    if name == "tile-sparse-6f":
        cfg = custom_config(head_dim=8, frames=6, grid_h=2, grid_w=2, num_partitions=6,
                            steps=2, schedule=CONFIGS[4].schedule)
    else:
        cfg = BY_NAME[name]
    M = masks_for(cfg, step)[step - 1]
    assert M.tolist() == fixtures.masks()[key]


@pytest.mark.parametrize("key", sorted(fixtures.fresh_columns().keys()))
def test_p7_fresh_columns(key):
    name, step, row = key
    cfg = BY_NAME[name]
    M = masks_for(cfg, step)[step - 1]
    assert [j for j in range(cfg.num_partitions) if M[row, j] == FRESH] == \
        fixtures.fresh_columns()[key]


@pytest.mark.parametrize("T", range(3, 31))
def test_p8_tile_mask_linear_in_frames(T):
    offs = partition_offsets(T * 6, T)
    act = active_mask(offs, 6, tile_sparse=True)
    assert int(act.sum()) == 4 * T - 4
    M = policy_mask(offs, 6, Policy(kind=FRAME_THRESHOLD, max_fresh_frame_dist=1,
                                    tile_sparse=True, anchor=True))
    assert int((M == FRESH).sum()) == 4 * T - 4


def test_work_lists_layout():
    M = np.array([[1, 2, 0], [2, 1, 1], [0, 0, 1]], dtype=np.uint8)
    fp, fc, rp, rc, counts = work_lists(M)
    assert fp.tolist() == [0, 1, 3, 4] and fc.tolist() == [0, 1, 2, 2]
    assert rp.tolist() == [0, 1, 2, 2] and rc.tolist() == [1, 0]
    assert counts.tolist() == [3, 4, 2]


def test_validation_rules():
    offs = partition_offsets(12, 3)
    bad_diag = Policy(kind=EXPLICIT, explicit_mask=(2, 1, 1, 1, 1, 1, 1, 1, 1))
    with pytest.raises(PolicyError):
        policy_mask(offs, 4, bad_diag, np.ones((3, 3), bool))
    reuse = Policy(kind=EXPLICIT, explicit_mask=(1, 2, 1, 1, 1, 1, 1, 1, 1))
    with pytest.raises(PolicyError):
        policy_mask(offs, 4, reuse, None)                   # nothing cached yet
    valid = np.zeros((3, 3), bool)
    valid[0, 1] = True
    assert policy_mask(offs, 4, reuse, valid)[0, 1] == REUSE
    with pytest.raises(PolicyError):
        policy_mask(offs, 4, Policy(kind=EXPLICIT, explicit_mask=(1, 3, 1, 1, 1, 1, 1, 1, 1)))
    with pytest.raises(PolicyError):
        policy_mask(offs, 4, Policy(kind=EXPLICIT, explicit_mask=(1, 1)))
    # skip outside a tile-sparse active set only
    offs6 = partition_offsets(24, 6)
    m = np.ones((6, 6), np.uint8)
    with pytest.raises(PolicyError):
        policy_mask(offs6, 4, Policy(kind=EXPLICIT, tile_sparse=True,
                                     explicit_mask=tuple(m.ravel())))


def test_centroids_and_frames_straddling():
    offs = partition_offsets(20, 3)          # sizes 7, 7, 6 over frames of 5 tokens
    assert centroids2(offs) == [6, 20, 33]
    assert partition_frames(offs, 5) == [0, 2, 3]
