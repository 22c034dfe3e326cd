"""Pins of the planner oracle, and the library's planner decision against it (CPU only).

The planner follows DiTango, "Anchor-Guided Selection Planner" (error model from importance
and temporal growth, anchor steps, online prediction from the local state, group strategy).
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle.attention import block_state
from oracle.policy import active_mask, partition_offsets, FRESH, REUSE, SKIP
from workloads import Policy, PLANNER, custom_config
import workloads.configs as wcfg


def _planner(pct=50, G=1, max_error=0.0, tile=False, anchor=False, period=0):
    return Policy(kind=PLANNER, reuse_percent=pct, group_size=G, max_error=max_error,
                  tile_sparse=tile, anchor=anchor, anchor_period=period)


# ---------------------------------------------------------------- importance

def _states_of(Q, K, offs, act, tau):
    P = len(offs) - 1
    lse = {}
    for i in range(P):
        for j in range(P):
            if act[i, j]:
                _, l = block_state(Q[offs[i]:offs[i + 1]], K[offs[j]:offs[j + 1]],
                                   K[offs[j]:offs[j + 1]], tau)
                lse[(i, j)] = l
    return lse


@pytest.mark.parametrize("tile", [False, True])
def test_importance_equals_dense_softmax_mass(tile):
    """w_ij = mean over rows of partition i of the softmax mass of keys in partition j,
    computed here from dense scores over the whole active key set."""
    rng = np.random.default_rng(3)
    T, F, P, D = 6, 10, 6, 8
    N = T * F
    offs = partition_offsets(N, P)
    act = active_mask(offs, F, tile)
    Q = rng.standard_normal((N, D)) * 1.5
    K = rng.standard_normal((N, D))
    tau = 1 / np.sqrt(D)
    w = oracle.importance(_states_of(Q, K, offs, act, tau), act)
    part = np.searchsorted(offs, np.arange(N), side="right") - 1
    for i in range(P):
        rows = np.arange(offs[i], offs[i + 1])
        z = tau * Q[rows] @ K.T
        z[:, ~act[i][part]] = -np.inf
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        for j in range(P):
            expect = p[:, part == j].sum(axis=1).mean()
            assert abs(w[i, j] - expect) < 1e-12
    assert np.all(w[~act] == 0)


def test_importance_uniform_attention_closed_form():
    """Q = 0 gives equal scores: block j's share is n_j over the active tokens."""
    N, P, D, F = 37, 5, 4, 37
    offs = partition_offsets(N, P)
    act = np.ones((P, P), bool)
    Q = np.zeros((N, D))
    K = np.random.default_rng(1).standard_normal((N, D))
    w = oracle.importance(_states_of(Q, K, offs, act, 0.5), act)
    n = np.diff(offs)
    for i in range(P):
        assert np.allclose(w[i], n / N, atol=1e-14)


def test_importance_rows_sum_to_one():
    rng = np.random.default_rng(7)
    N, P, D, F = 60, 6, 8, 10
    offs = partition_offsets(N, P)
    act = active_mask(offs, F, True)
    w = oracle.importance(_states_of(rng.standard_normal((N, D)), rng.standard_normal((N, D)),
                                     offs, act, 0.3), act)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-13)


# ---------------------------------------------------------------- growth

def test_growth_zero_and_constant_shift():
    rng = np.random.default_rng(2)
    D = 5
    old = {i: rng.standard_normal((3, 7, 8)) for i in range(3)}   # [heads, rows, DP]
    assert np.all(oracle.growth(old, old, D) == 0)
    shift = [0.25, -1.5, 3.0]
    new = {}
    for i in range(3):
        a = old[i].copy()
        a[..., :D] += shift[i]
        a[..., D:] += 100.0          # padding dims beyond D do not count
        new[i] = a
    assert np.allclose(oracle.growth(new, old, D), np.abs(shift), rtol=1e-14)


# ---------------------------------------------------------------- decision

def test_planner_mask_hand_worked_example():
    """P = 4 single-frame partitions, G = 1, 50 % reuse: A = 4, R = 2, so the diagonal and
    the one largest-error block are fresh; ties go to the smaller j.  With a cap of 0.35,
    every block above it is fresh as well."""
    offs = [0, 4, 8, 12, 16]
    E = np.array([[0.0, 0.3, 0.1, 0.5],
                  [0.2, 0.0, 0.2, 0.1],
                  [0.0, 0.9, 0.0, 0.9],
                  [0.4, 0.4, 0.4, 0.0]])
    valid = np.ones((4, 4), bool)
    F, R = FRESH, REUSE
    got = oracle.planner_mask(offs, 16, _planner(50), E, valid, False)
    assert got.tolist() == [[F, R, R, F], [F, F, R, R], [R, F, F, R], [F, R, R, F]]
    got = oracle.planner_mask(offs, 16, _planner(50, max_error=0.35), E, valid, False)
    assert got.tolist() == [[F, R, R, F], [F, F, R, R], [R, F, F, F], [F, F, F, F]]
    # an invalid slot forces its block fresh; the budget is then already used up
    v2 = valid.copy()
    v2[0, 2] = False
    got = oracle.planner_mask(offs, 16, _planner(50), E, v2, False)
    assert got[0].tolist() == [F, R, F, R]


def test_planner_mask_groups_hand_worked_example():
    """G = 2 over P = 4: groups {0,1} and {2,3}; with 50 % reuse each query group keeps its
    diagonal group fresh and reuses the other one, unless its summed error tops the cap."""
    offs = [0, 4, 8, 12, 16]
    E = np.zeros((4, 4))
    E[0, 2], E[0, 3], E[1, 2], E[1, 3] = 0.1, 0.2, 0.05, 0.05      # group (0, 1): 0.4
    E[2, 0], E[3, 1] = 0.3, 0.3                                      # group (1, 0): 0.6
    valid = np.ones((4, 4), bool)
    F, R = FRESH, REUSE
    got = oracle.planner_mask(offs, 16, _planner(50, G=2), E, valid, False)
    assert got.tolist() == [[F, F, R, R], [F, F, R, R], [R, R, F, F], [R, R, F, F]]
    got = oracle.planner_mask(offs, 16, _planner(50, G=2, max_error=0.5), E, valid, False)
    assert got.tolist() == [[F, F, R, R], [F, F, R, R], [F, F, F, F], [F, F, F, F]]


def _brute_force_check(M, offs, F_tokens, pol, E, valid):
    """Per query group: fresh groups contain the forced ones, number max(A - R, forced), and
    no other choice of the same size has a larger summed error."""
    P = len(offs) - 1
    act = active_mask(offs, F_tokens, pol.tile_sparse)
    G = pol.group_size
    groups = [list(range(g, min(P, g + G))) for g in range(0, P, G)]
    for I, gi in enumerate(groups):
        cand = {}
        for J, gj in enumerate(groups):
            mem = [(i, j) for i in gi for j in gj if act[i, j]]
            if not mem:
                continue
            states = {M[i, j] for (i, j) in mem}
            assert len(states) == 1 and states <= {FRESH, REUSE}      # group-uniform
            e = sum(E[i, j] for (i, j) in mem if i != j)
            forced = J == I or any(not valid[i, j] for (i, j) in mem) or \
                (pol.max_error > 0 and e > pol.max_error)
            cand[J] = (e, forced, states.pop() == FRESH)
        A = len(cand)
        R = min((pol.reuse_percent * A + 50) // 100, A - 1)
        n_forced = sum(f for (_, f, _) in cand.values())
        fresh = [J for J, c in cand.items() if c[2]]
        assert all(c[2] for c in cand.values() if c[1])
        assert len(fresh) == max(A - R, n_forced)
        free = [J for J, c in cand.items() if not c[1]]
        k = len(fresh) - n_forced
        best = max((sum(cand[J][0] for J in S) for S in itertools.combinations(free, k)),
                   default=0.0)
        assert sum(cand[J][0] for J in fresh if not cand[J][1]) >= best - 1e-12
    for i in range(P):
        for j in range(P):
            assert (M[i, j] == SKIP) == (not act[i, j])


@pytest.mark.parametrize("seed", range(12))
def test_planner_mask_exhaustive_small(seed):
    rng = np.random.default_rng(seed)
    T, Fr = 4, 6
    P = int(rng.integers(3, 8))
    offs = partition_offsets(T * Fr, P)
    pol = _planner(pct=int(rng.integers(0, 101)), G=int(rng.integers(1, 4)),
                   max_error=float(rng.choice([0.0, 0.5])), tile=bool(rng.integers(0, 2)))
    E = np.round(rng.random((P, P)), 1)             # ties on purpose
    valid = rng.random((P, P)) > 0.15
    M = oracle.planner_mask(offs, Fr, pol, E, valid, False)
    _brute_force_check(M, offs, Fr, pol, E, valid)


# ---------------------------------------------------------------- planner runs

def _tiny(drift=0.05):
    return custom_config(name="planner-tiny", idx=70, heads=2, head_dim=16, frames=3, grid_h=2,
                         grid_w=4, num_partitions=6, steps=5, qkv_dtype="f32",
                         cache_dtype="f32", drift=drift)


def test_planner_all_anchors_equals_all_fresh():
    cfg = _tiny()
    heads = [(0, 0), (0, 1)]
    res = oracle.run_planner(cfg, heads, _planner(60, period=1), cache_mode="fp64")
    all_fresh = [Policy(kind=wcfg.FRESH_BUDGET, anchor=True)] * cfg.steps
    for (b, h) in heads:
        ref = oracle.run_head(cfg, b, h, policies=all_fresh, cache_mode="fp64")
        for st, r in zip(res, ref):
            assert st.anchor and np.all(st.mask == FRESH)
            assert np.allclose(st.out[(b, h)], r.out, atol=1e-13, rtol=0)


def test_planner_without_drift_reuse_is_exact():
    """No drift: every cached state equals its fresh value, so whatever the planner reuses
    the output is the all-fresh one, and the measured growth is zero."""
    cfg = _tiny(drift=0.0)
    heads = [(0, 0), (0, 1)]
    res = oracle.run_planner(cfg, heads, _planner(60), cache_mode="fp64")
    assert any(np.any(st.mask == REUSE) for st in res)
    ref = oracle.run_head(cfg, 0, 1, policies=[Policy(kind=wcfg.FRESH_BUDGET, anchor=True)]
                          * cfg.steps, cache_mode="fp64")
    for st, r in zip(res, ref):
        assert np.allclose(st.out[(0, 1)], r.out, atol=1e-12, rtol=0)
        if st.step >= 2:
            assert np.all(st.delta == 0)


def test_planner_reuse_budget_and_error_ranking_in_a_run():
    cfg = _tiny()
    heads = [(0, 0), (0, 1)]
    res = oracle.run_planner(cfg, heads, _planner(60), cache_mode="emulate")
    P = cfg.num_partitions
    for st in res[1:]:
        A = P
        R = min((60 * A + 50) // 100, A - 1)
        assert np.all((st.mask == FRESH).sum(axis=1) == A - R)
        assert np.all(st.delta > 0)


# ---------------------------------------------------------------- library decision

@pytest.fixture(scope="module")
def dita():
    return pytest.importorskip("partial_state_reuse_amd")


@pytest.mark.parametrize("seed", range(20))
def test_library_planner_mask_equals_oracle(dita, seed):
    rng = np.random.default_rng(100 + seed)
    T, Fr = int(rng.integers(2, 6)), int(rng.integers(2, 9))
    N = T * Fr
    P = int(rng.integers(1, min(N, 24) + 1))
    G = int(rng.integers(1, 5))
    pct = int(rng.integers(0, 101))
    max_error = float(rng.choice([0.0, 0.3, 1e-3]))
    tile = bool(rng.integers(0, 2))
    E = rng.random((P, P)) * rng.choice([1.0, 1e-3])
    E[rng.random((P, P)) < 0.2] = 0.0                 # ties
    valid = rng.random((P, P)) > 0.1
    geom = dita.make_geometry(1, 1, N, 16, T, 1, Fr, P, dtype="f32")
    pol_c = dita.make_policy(kind=dita.POLICY_PLANNER, reuse_percent=pct, group_size=G,
                             max_error=max_error, tile_sparse=tile)
    got = dita.dita_planner_mask(geom, pol_c, E, valid.astype(np.uint8))
    offs = partition_offsets(N, P)
    exp = oracle.planner_mask(offs, Fr, _planner(pct, G, max_error, tile), E, valid, False)
    assert np.array_equal(got, exp)
    # anchor: every active block fresh
    pol_c.anchor = 1
    got = dita.dita_planner_mask(geom, pol_c, E, valid.astype(np.uint8))
    act = active_mask(offs, Fr, tile)
    assert np.array_equal(got, np.where(act, FRESH, SKIP))


def test_library_planner_argument_errors(dita):
    geom = dita.make_geometry(1, 1, 16, 16, 2, 2, 4, 4, dtype="f32")
    E = np.zeros((4, 4))
    bad = dita.make_policy(kind=dita.POLICY_FRESH_BUDGET, reuse_percent=50)
    with pytest.raises(dita.DitaError, match="INVALID_ARGUMENT"):
        dita.dita_planner_mask(geom, bad, E)
    with pytest.raises(dita.DitaError, match="INVALID_ARGUMENT"):
        dita.dita_planner_mask(geom, dita.make_policy(kind=dita.POLICY_PLANNER,
                                                      reuse_percent=101), E)
    with pytest.raises(dita.DitaError, match="INVALID_ARGUMENT"):
        dita.dita_planner_mask(geom, dita.make_policy(kind=dita.POLICY_PLANNER,
                                                      group_size=-1), E)
    # without a cache a non-anchor planner step has no errors to decide from
    with pytest.raises(dita.DitaError, match="INVALID_ARGUMENT"):
        dita.dita_policy_mask(geom, dita.make_policy(kind=dita.POLICY_PLANNER))
    M = dita.dita_policy_mask(geom, dita.make_policy(kind=dita.POLICY_PLANNER, anchor=True))
    assert np.all(M == FRESH)


def test_predicted_error_closed_form_for_constant_growth():
    """Constant growth c per step: a state last fresh at step f has drifted c (s - 1 - f)
    by step s - 1 and is predicted to drift c more, so E = w c (s - f)."""
    P, s, c = 3, 7, 0.125
    w = np.array([[0.5, 0.25, 0.25], [0.125, 0.75, 0.125], [0.0, 0.5, 0.5]], dtype=np.float32)
    delta_hist = np.full((s - 1, P), c)
    delta_hist[0] = 0.0                       # step 1 has no previous state
    fresh = np.array([[6, 1, 3], [2, 6, 5], [4, 0, 6]])
    valid = fresh > 0
    E = oracle.predicted_errors(w, delta_hist, fresh, valid, s)
    for i in range(P):
        for j in range(P):
            f = fresh[i, j]
            expect = 0.0 if f == 0 else float(w[i, j]) * c * (s - f)
            assert E[i, j] == pytest.approx(expect, abs=1e-15)
