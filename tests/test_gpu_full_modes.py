"""GPU parity of the widened modes at the full video workload (29 frames of a 720p latent:
N = 28800 tokens, 32 partitions, 24 heads, D = 64, 10 steps), in the launch configuration the
bench times for each mode:

  * fp8 (e4m3) state cache under the fixed schedule;
  * group composition: after the anchor step, the cached states of every aligned pair of key
    partitions that all later steps reuse are merged into one;
  * the selection planner at the schedule's reuse budget.

Every step's plan is compared bit for bit (the planner's decisions against the oracle's
decision from the importance, growth and freshness the library reports); outputs are compared
on sampled rows (the first two, last two and random rows of every partition) of two heads.
The planner's measurements cover every head and row, out of the oracle's reach at this size:
importance is checked by the properties that hold at any size (each row's shares are
non-negative, zero on inactive blocks and sum to one), growth by being finite and
non-negative; the small geometries check both against the oracle value by value."""
import dataclasses

import numpy as np
import pytest

import gpu_helpers as gh
from gpu_helpers import BF16_MAX_ABS, BF16_MEAN_ABS, compare, log
from workloads import CONFIGS, Policy, PLANNER
from workloads import configs as wcfg

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

VIDEO = 3
HEADS = [(0, 0), (0, 17)]


@pytest.fixture(scope="module")
def dita():
    import partial_state_reuse_amd as d
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return d


def _setup(cfg, seed):
    from oracle.policy import active_mask, partition_offsets
    offs = partition_offsets(cfg.tokens, cfg.num_partitions)
    act = active_mask(offs, cfg.frame_tokens, cfg.policy(1).tile_sparse)
    rows = gh.sample_rows(offs, 8, np.random.default_rng(seed))
    return offs, act, rows


def _run(dita, cfg, act, rows, policies, merges=None):
    """All steps on the GPU; returns per-step plans, sampled (out, lse) of HEADS, the
    planner state after every step, and the host copies of the HEADS inputs."""
    S = len(policies)
    log(f"case {cfg.name} cache={cfg.cache_dtype} N={cfg.tokens} P={cfg.num_partitions} "
        f"steps={S} rows={len(rows)} heads={HEADS}")
    dev, kept = gh.device_inputs(cfg, S, keep_heads=set(HEADS))
    cache = dita.Cache(dita.geometry_from(cfg), active_mask=act.astype(np.uint8))
    sel = torch.as_tensor(rows, device="cuda")
    plans, outs, states = [], [], []
    for s in range(S):
        cache.set_policy(dita.policy_from(policies[s]))
        plans.append(cache.plan())
        q, k, v = dev[s]
        out, lse = cache.step(q, k, v)
        outs.append({bh: (out[bh].index_select(0, sel).cpu().numpy(),
                          lse[bh].index_select(0, sel).cpu().numpy()) for bh in HEADS})
        if policies[s].kind == PLANNER:
            states.append(cache.planner_state())
        for (g, sl) in (merges or {}).get(s + 1, []):
            cache.merge_groups(g, select=sl)
    torch.cuda.synchronize()
    st = cache.stats()
    assert st["device_fresh_blocks"] == st["host_fresh_blocks"]
    assert st["device_reuse_blocks"] == st["host_reuse_blocks"]
    assert st["device_v_range_errors"] == 0
    cache.free()
    del dev
    return plans, outs, states, kept


def _check_plans(plans, ref, merged):
    for s, (p, r) in enumerate(zip(plans, ref)):
        assert np.array_equal(p["mask"], r.mask), f"step {s + 1}: mask"
        assert np.array_equal(p["fresh_ptr"], r.fresh_ptr), f"step {s + 1}: fresh lists"
        assert np.array_equal(p["fresh_cols"], r.fresh_cols), f"step {s + 1}: fresh lists"
        assert np.array_equal(p["reuse_ptr"], r.reuse_ptr), f"step {s + 1}: reuse lists"
        assert np.array_equal(p["reuse_cols"], r.reuse_cols), f"step {s + 1}: reuse lists"
        if not merged:
            assert np.array_equal(p["counts"], r.counts), f"step {s + 1}: counts"


def _check_outputs(outs, ref64, emu, what):
    ok_all, worst = True, (0.0, 0.0)
    for s in range(len(outs)):
        for bh in HEADS:
            o, l = outs[s][bh]
            ok, mx, mean = compare(o, ref64[bh][s].out, True, f"  {what} {bh} step {s + 1} out")
            worst = (max(worst[0], mx), max(worst[1], mean))
            ok_all &= ok
            ok_all &= float(np.mean(np.abs(o - emu[bh][s].out))) <= BF16_MEAN_ABS
            lerr = float(np.max(np.abs(l - ref64[bh][s].lse)))
            assert lerr < 2e-3, f"{what} step {s + 1} lse {lerr:.3e}"
    log(f"{what}: worst max-abs {worst[0]:.3e} mean-abs {worst[1]:.3e}")
    assert ok_all


def _spacing8(x):
    ax = np.abs(np.asarray(x, np.float64))
    k = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** -9)))
    return np.exp2(np.maximum(k, -6.0) - 3.0)


def test_full_fp8_cache_video29f(dita):
    """fp8 cache: within the bf16 bar plus, per element, one e4m3 spacing of every reused
    state weighted by its share exp(lse_r - L) (the two sides round values that differ by
    their arithmetic error)."""
    import oracle
    cfg = dataclasses.replace(CONFIGS[VIDEO], cache_dtype="fp8")
    offs, act, rows = _setup(cfg, 61)
    pols = [cfg.policy(s) for s in range(1, cfg.steps + 1)]
    plans, outs, _, kept = _run(dita, cfg, act, rows, pols)
    P = cfg.num_partitions
    ok_all = True
    for bh in HEADS:
        emu = oracle.run_head(cfg, *bh, rows=rows, cache_mode="emulate", active=act,
                              inputs=kept[bh], keep_block_lse=True)
        exact = oracle.run_head(cfg, *bh, rows=rows, cache_mode="fp64", active=act,
                                inputs=kept[bh])
        if bh == HEADS[0]:
            _check_plans(plans, emu, False)
        for s, r in enumerate(emu):
            o, l = outs[s][bh]
            bound = np.full(o.shape, BF16_MAX_ABS)
            pos = 0
            for i in range(P):
                n = int(np.count_nonzero((rows >= offs[i]) & (rows < offs[i + 1])))
                for j in range(P):
                    if r.mask[i, j] == 2:
                        wgt = np.exp(r.block_lse[(i, j)] - r.lse[pos:pos + n])
                        bound[pos:pos + n] += wgt[:, None] * _spacing8(r.block_o[(i, j)])
                pos += n
            err = np.abs(o - r.out)
            slack = float((err - bound).max())
            lerr = float(np.abs(l - r.lse).max())
            xerr = np.abs(o - exact[s].out)
            log(f"fp8 {bh} step {s + 1}: vs fp8 oracle max {err.max():.3e} mean {err.mean():.3e} "
                f"(bar slack {slack:.2e}); lse {lerr:.2e}; vs exact max {xerr.max():.3e}")
            ok_all &= slack <= 0 and lerr < 2e-3 and err.mean() <= BF16_MEAN_ABS
    assert ok_all


def test_full_group_merge_video29f(dita):
    """Pairs of key partitions merged after the anchor wherever every later step reuses the
    whole pair (the selection is taken from the oracle's masks); the merged states are then
    read once per pair."""
    import oracle
    from oracle.policy import policy_mask
    cfg = CONFIGS[VIDEO]
    offs, act, rows = _setup(cfg, 62)
    P, S, G = cfg.num_partitions, cfg.steps, 2
    pols = [cfg.policy(s) for s in range(1, S + 1)]
    later = [policy_mask(offs, cfg.frame_tokens, pols[s], np.ones((P, P), bool))
             for s in range(1, S)]
    NG = (P + G - 1) // G
    sel = np.zeros((P, NG), np.uint8)
    for i in range(P):
        for J in range(NG):
            sel[i, J] = all(M[i, j] == 2 for M in later for j in range(J * G, min(P, J * G + G)))
    assert sel.sum() > 0
    merges = {1: [(G, sel)]}
    plans, outs, _, kept = _run(dita, cfg, act, rows, pols, merges=merges)
    ref64, emu = {}, {}
    for bh in HEADS:
        ref64[bh] = oracle.run_head(cfg, *bh, rows=rows, cache_mode="fp64", active=act,
                                    inputs=kept[bh], merges=merges)
        emu[bh] = oracle.run_head(cfg, *bh, rows=rows, cache_mode="emulate", active=act,
                                  inputs=kept[bh], merges=merges)
    _check_plans(plans, emu[HEADS[0]], True)
    # reads per step: one per merged pair instead of two
    unmerged = oracle.run_head(cfg, *HEADS[0], rows=rows[:4], cache_mode="fp64", active=act,
                               inputs=kept[HEADS[0]])
    for s in range(1, S):
        assert plans[s]["reuse_ptr"][-1] < unmerged[s].reuse_ptr[-1]
    _check_outputs(outs, ref64, emu, "merged pairs")


def test_full_planner_video29f(dita):
    import oracle
    cfg = CONFIGS[VIDEO]
    offs, act, rows = _setup(cfg, 63)
    P, S = cfg.num_partitions, cfg.steps
    pl = Policy(kind=PLANNER, reuse_percent=cfg.policy(2).reuse_percent, group_size=1,
                anchor_period=0, tile_sparse=cfg.policy(1).tile_sparse)
    plans, outs, states, kept = _run(dita, cfg, act, rows, [pl] * S)
    masks = [p["mask"].copy() for p in plans]
    from oracle.policy import FRESH, SKIP
    assert np.array_equal(masks[0], np.where(act, FRESH, SKIP))
    n_reuse = 0
    for s in range(2, S + 1):
        prev = states[s - 2]
        valid = prev["fresh_step"] > 0
        E = oracle.predicted_errors(prev["w"], prev["delta"], prev["fresh_step"], valid, s)
        want = oracle.planner_mask(offs, cfg.frame_tokens, pl, E, valid, False)
        assert np.array_equal(masks[s - 1], want), f"step {s}: planner decision differs"
        n_reuse += int(np.any(masks[s - 1] == 2))
    assert n_reuse == S - 1
    w = states[0]["w"].astype(np.float64)
    assert np.all(w >= 0) and np.all(w[~act] == 0)
    assert np.allclose(w.sum(axis=1), 1.0, atol=2e-5), np.abs(w.sum(axis=1) - 1).max()
    for s in range(2, S + 1):
        d = states[s - 1]["delta"][s - 1]
        assert np.all(np.isfinite(d)) and np.all(d >= 0) and np.any(d > 0), f"step {s} growth"
    log(f"planner: {S} steps, decisions equal; importance rows sum to 1 within "
        f"{np.abs(w.sum(axis=1) - 1).max():.1e}")
    # outputs on sampled rows, replaying the decided masks
    replay = [Policy(kind=wcfg.EXPLICIT, explicit_mask=tuple(int(x) for x in M.ravel()))
              for M in masks]
    ref64, emu = {}, {}
    for bh in HEADS:
        ref64[bh] = oracle.run_head(cfg, *bh, rows=rows, cache_mode="fp64", active=act,
                                    inputs=kept[bh], policies=replay)
        emu[bh] = oracle.run_head(cfg, *bh, rows=rows, cache_mode="emulate", active=act,
                                  inputs=kept[bh], policies=replay)
    _check_plans(plans, emu[HEADS[0]], False)
    _check_outputs(outs, ref64, emu, "planner")
