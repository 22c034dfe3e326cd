"""GPU parity of the selection planner (DiTango, "Anchor-Guided Selection Planner"), through
the C ABI.

For every step of a planner schedule:
  * decisions: each non-anchor mask equals the oracle's decision computed from the state the
    library reports (importance, growth history, last fresh steps), bit for bit: floating
    point decides an integer here, so both sides decide from the same float inputs in the
    same float64 order;
  * measurements: the device importance and growth against the oracle replaying the same
    masks with the same cache rounding;
  * outputs: against the fp64 oracle on the same masks, within the bf16 / f32 bars.
"""
import numpy as np
import pytest

import gpu_helpers as gh
from gpu_helpers import compare, log
from workloads import Policy, PLANNER, custom_config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# importance: lse in f32 on both sides; growth: RMS of differences of bf16-rounded states,
# where a value near a rounding boundary can land one ulp apart on the two sides
W_RTOL, W_ATOL = 2e-4, 1e-7
DELTA_RTOL = {"bf16": 5e-3, "f32": 1e-4}


def fp8_delta_rtol(n):
    """Relative bar on the growth with an fp8 (e4m3) cache, over an RMS of n elements.  Both
    sides round the new and the old diagonal state to e4m3, whose spacing (1/16 to 1/8 of the
    value) is about the size of one step's change, from values that differ by their
    arithmetic error: the elements near a rounding midpoint (about a tenth) may land one
    spacing apart, in random places and directions.  Their effect on the RMS shrinks like
    1/sqrt(n), about 0.3/sqrt(n) for one standard deviation; the bar is 1/sqrt(n), and never
    under 1e-2."""
    return max(1e-2, 1.0 / np.sqrt(n))


def bf16_delta_rtol(n):
    """Relative bar on the growth with a bf16 cache, over an RMS of n elements.  The same
    rounding noise as with fp8, at bf16's spacing (1/256 to 1/128 of the value): an element
    landing one spacing apart moves its squared change by about twice the change times the
    spacing.  With the state about ten times its per-step change and, at worst, every element
    moved so in a random direction, one standard deviation of the RMS's relative error is
    about 10/(128 sqrt(n)); the bar is three of them, 0.25/sqrt(n), and never under 5e-3
    (which it exceeds for partitions of under 2500 elements)."""
    return max(DELTA_RTOL["bf16"], 0.25 / np.sqrt(n))


@pytest.fixture(scope="module")
def dita():
    import partial_state_reuse_amd as d
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return d


CASES = [
    # name, frames, gh, gw, P, D, heads, steps, dtype, reuse %, group, anchor period, cap, tile
    ("planner-bf16-d64", 4, 6, 10, 8, 64, 3, 7, "bf16", 60, 1, 4, 0.0, False),
    ("planner-bf16-groups", 4, 6, 10, 8, 64, 2, 6, "bf16", 50, 2, 0, 0.0, False),
    ("planner-bf16-cap-tile", 6, 5, 7, 6, 64, 2, 6, "bf16", 70, 1, 0, 6e-3, True),
    ("planner-bf16-d128", 3, 8, 10, 6, 128, 2, 5, "bf16", 60, 1, 3, 0.0, False),
    ("planner-f32", 3, 4, 8, 6, 64, 2, 6, "f32", 60, 2, 0, 0.0, False),
    # fp8 state cache: decisions and measurements (its outputs are checked in test_gpu_fp8)
    ("planner-fp8-cache", 4, 6, 10, 8, 64, 2, 6, "bf16/fp8", 60, 1, 3, 0.0, False),
    # many partitions: 4-row and 8-row partitions, P x P plans of 64K and 16K blocks
    ("planner-bf16-256-partitions", 4, 16, 16, 256, 64, 1, 5, "bf16", 60, 1, 3, 0.0, False),
    ("planner-fp8-128-partitions", 4, 16, 16, 128, 64, 1, 4, "bf16/fp8", 60, 2, 0, 0.0, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_planner_schedule(dita, case):
    run_planner_case(dita, case)


# Relative gap between the last block group chosen fresh and the first one reused, below which
# the device's and the oracle's own measurements could order two groups differently: each
# predicted error is importance (relative error <= 2e-4) times summed growth (<= 5e-3), so two
# errors closer than twice that sum may swap.  The bar keeps a factor of two above it.
FREE_RUN_MARGIN = 2e-2

FREE_RUN_CASES = [
    ("planner-free-d128", 3, 8, 10, 6, 128, 2, 5, "bf16", 60, 1, 3, 0.0, False),
    ("planner-free-groups", 8, 5, 6, 8, 64, 2, 6, "bf16", 60, 2, 0, 0.0, False),
]


@pytest.mark.parametrize("case", FREE_RUN_CASES, ids=[c[0] for c in FREE_RUN_CASES])
def test_planner_free_running_against_oracle(dita, case):
    """The oracle's planner deciding from its own measurements (no masks handed to it) takes
    the device's decisions at every step, on cases whose decision margins exceed what the
    measurement tolerances could move (asserted from the oracle's own predicted errors)."""
    run_planner_case(dita, case, free_running=True)


def decision_margins(offs, frame_tokens, pol, E, valid):
    """Per query group, the relative gap (e_k - e_{k+1}) / e_k between the last group chosen
    fresh by error and the first one reused, where the budget cuts the ranking; groups forced
    fresh do not take part.  A cut between two errors that are both exactly zero is exact on
    both sides and is left out."""
    from oracle.policy import active_mask
    P = len(offs) - 1
    act = active_mask(offs, frame_tokens, pol.tile_sparse)
    G = max(1, pol.group_size or 1)
    groups = [list(range(g0, min(P, g0 + G))) for g0 in range(0, P, G)]
    out = []
    for I, gi in enumerate(groups):
        cand = []
        for J, gj in enumerate(groups):
            mem = [(i, j) for i in gi for j in gj if act[i, j]]
            if not mem:
                continue
            e = sum(float(E[i, j]) for (i, j) in mem if i != j)
            forced = J == I or any(not valid[i, j] for (i, j) in mem) or \
                (pol.max_error > 0 and e > pol.max_error)
            cand.append((J, e, forced))
        A = len(cand)
        n_reuse = min((pol.reuse_percent * A + 50) // 100, A - 1)
        free = sorted([c for c in cand if not c[2]], key=lambda c: (-c[1], c[0]))
        k = max(0, A - n_reuse - sum(c[2] for c in cand))
        if 0 < k < len(free):
            a, b = free[k - 1][1], free[k][1]
            if a == 0.0 and b == 0.0:
                continue
            out.append((a - b) / a)
    return out


@pytest.mark.parametrize("seed", list(range(48)) + [103])
def test_planner_sweep(dita, seed):
    """Random small workloads under the planner: geometry (2-6 frames, 3-12 x 3-20 grid, 3-10
    partitions), head dim, path, reuse budget, group size, anchor period, error cap and the
    tile-sparse set."""
    rng = np.random.default_rng(5000 + seed)
    T, gh_, gw = int(rng.integers(2, 7)), int(rng.integers(3, 13)), int(rng.integers(3, 21))
    P = int(rng.integers(3, 11))
    dt = str(rng.choice(["bf16", "bf16", "bf16/fp8", "f32"]))
    D = int(rng.choice([64, 72, 128] if dt != "f32" else [16, 64]))
    H, S = int(rng.integers(1, 3)), int(rng.integers(3, 7))
    pct = int(rng.integers(30, 91))
    G = int(rng.integers(1, 4))
    period = int(rng.choice([0, 0, 3, 4]))
    cap = float(rng.choice([0.0, 0.0, 5e-3]))
    tile = bool(rng.random() < 0.25)
    run_planner_case(dita, (f"planner-sweep-{seed}", T, gh_, gw, P, D, H, S, dt, pct, G, period,
                            cap, tile), require_reuse=False)


def test_planner_measures_through_a_second_pass(dita):
    """Steps after the anchor run the fixed-reference pass, which measures the growth against
    a snapshot of the old diagonal states (in its 128-row groups; tail waves keep the running
    maximum, so the partitions here hold 130 rows).  One key partition's K scaled by 8 on
    step 3 (and restored on step 4) makes the pass reject its reference on both steps: the
    second pass
    computes them again, measuring the same change, and decisions, measurements and outputs
    still match the oracle on the same inputs."""
    from oracle.policy import partition_offsets
    case = ("planner-lse-jump", 4, 10, 26, 8, 64, 2, 6, "bf16", 60, 1, 0, 0.0, False)
    offs = partition_offsets(4 * 10 * 26, 8)
    j0, j1 = offs[2], offs[3]

    def modify(dev, kept):
        dev[2][1][:, :, j0:j1, :] *= 8                 # exact in bf16
        for bh in kept:
            kept[bh][2][1][j0:j1] *= 8
    run_planner_case(dita, case, modify=modify, recomputes="some")


def run_planner_case(dita, case, modify=None, recomputes=None, require_reuse=True,
                     free_running=False):
    import oracle
    from oracle.policy import active_mask, partition_offsets, FRESH, SKIP
    name, T, gh_, gw, P, D, H, S, dt, pct, G, period, cap, tile = case
    dt, cdt = dt.split("/") if "/" in dt else (dt, dt)
    cfg = custom_config(name=name, idx=80, heads=H, head_dim=D, frames=T, grid_h=gh_, grid_w=gw,
                        num_partitions=P, steps=S, qkv_dtype=dt, cache_dtype=cdt)
    pol = Policy(kind=PLANNER, reuse_percent=pct, group_size=G, anchor_period=period,
                 max_error=cap, tile_sparse=tile)
    heads = [(0, h) for h in range(H)]
    offs = partition_offsets(cfg.tokens, P)
    act = active_mask(offs, cfg.frame_tokens, tile)
    log(f"case {name}: N={cfg.tokens} P={P} D={D} H={H} steps={S} {dt} reuse={pct}% G={G} "
        f"period={period} cap={cap} tile={tile}")
    dev, kept = gh.device_inputs(cfg, S, keep_heads=set(heads))
    if modify is not None:
        modify(dev, kept)
    cache = dita.Cache(dita.geometry_from(cfg), active_mask=act.astype(np.uint8))
    masks, outs, states = [], [], []
    for s in range(S):
        cache.set_policy(dita.policy_from(pol))
        masks.append(cache.plan()["mask"].copy())
        q, k, v = dev[s]
        out, _ = cache.step(q, k, v)
        outs.append(out.cpu().numpy())
        states.append(cache.planner_state())
    recomputed = cache.stats()["device_ref_recomputes"]
    cache.free()
    log(f"steps computed a second time: {recomputed}")
    if recomputes == "some":
        assert recomputed > 0
    elif recomputes == 0:
        assert recomputed == 0

    # the last-fresh steps the library reports, against those the recorded masks imply
    fs = np.zeros((P, P), dtype=np.int64)
    for s in range(1, S + 1):
        fs[masks[s - 1] == FRESH] = s
        assert np.array_equal(states[s - 1]["fresh_step"], fs), f"step {s}: fresh_step"
        assert states[s - 1]["steps"] == s

    # decisions, bit for bit
    n_reuse_steps = 0
    for s in range(1, S + 1):
        M = masks[s - 1]
        anchor = s == 1 or (period > 0 and (s - 1) % period == 0)
        if anchor:
            assert np.array_equal(M, np.where(act, FRESH, SKIP)), f"step {s}: anchor mask"
            continue
        prev = states[s - 2]
        valid = prev["fresh_step"] > 0
        E = oracle.predicted_errors(prev["w"], prev["delta"], prev["fresh_step"], valid, s)
        want = oracle.planner_mask(offs, cfg.frame_tokens, pol, E, valid, False)
        assert np.array_equal(M, want), f"step {s}: planner decision differs"
        n_reuse_steps += int(np.any(M == 2))
    if require_reuse:
        assert n_reuse_steps > 0
    log(f"decisions: {S} steps equal, {n_reuse_steps} with reuse")

    if free_running:
        # the oracle deciding from its own measurements
        own = oracle.run_planner(cfg, heads, pol, cache_mode="emulate", inputs=kept)
        fs_o = np.zeros((P, P), dtype=np.int64)
        hist, w_o, worst = [], None, np.inf
        for s in range(1, S + 1):
            st = own[s - 1]
            if not st.anchor:
                valid = fs_o > 0
                E = oracle.predicted_errors(w_o, np.array(hist).reshape(-1, P), fs_o, valid, s)
                m = decision_margins(offs, cfg.frame_tokens, pol, E, valid)
                worst = min([worst] + m)
            assert np.array_equal(st.mask, masks[s - 1]), f"step {s}: free-running oracle"
            hist.append(st.delta if st.delta is not None else np.zeros(P))
            if st.w is not None:
                w_o = st.w.astype(np.float32)
            fs_o[st.mask == FRESH] = s
        log(f"free-running oracle: {S} steps equal; smallest decision margin {worst:.3e}")
        assert worst >= FREE_RUN_MARGIN

    # measurements against the oracle replaying the same masks (same cache rounding)
    rep = oracle.run_planner(cfg, heads, pol, masks=masks, cache_mode="emulate", inputs=kept)
    for s in range(1, S + 1):
        st, ref = states[s - 1], rep[s - 1]
        if ref.w is not None:
            err = np.abs(st["w"] - ref.w)
            assert np.all(err <= W_ATOL + W_RTOL * np.abs(ref.w)), \
                f"step {s}: importance max err {err.max():.3e}"
        if s >= 2:
            got = st["delta"][s - 1]
            rel = np.abs(got - ref.delta) / np.maximum(ref.delta, 1e-12)
            log(f"step {s}: growth {np.round(got, 5).tolist()} rel err max {rel.max():.2e}")
            rows = np.diff(np.asarray(offs, np.int64))
            sizes = [len(heads) * int(rows[i]) * cfg.head_dim for i in range(P)]
            if cdt == "fp8":
                bar = np.array([fp8_delta_rtol(n) for n in sizes])
            elif cdt == "bf16":
                bar = np.array([bf16_delta_rtol(n) for n in sizes])
            else:
                bar = DELTA_RTOL[cdt]
            assert np.all(rel <= bar), f"step {s}: growth rel err {rel.max():.3e}"

    if cdt != dt:
        return
    # outputs against the fp64 oracle on the same masks
    ref64 = oracle.run_planner(cfg, heads, pol, masks=masks, cache_mode="fp64", inputs=kept)
    ok = True
    for s in range(S):
        for (b, h) in heads:
            o, *_ = compare(outs[s][b, h], ref64[s].out[(b, h)], dt == "bf16",
                            f"step {s + 1} head {h} out")
            ok &= o
    assert ok
