"""GPU parity of group composition (DiTango, "State-Centric Parallel Runtime / Composizione
Dinamica dei Gruppi"), through the C ABI: cached states merged into coarser groups after a
step, then reused as one state.  Masks (with whole-group promotion) and reuse lists are
compared bit for bit with the oracle; outputs of every step against the fp64 oracle on the
same merges within the bf16 / f32 bars; device-counted reads against the host plan.

A merged state is rounded to the cache precision once more per merge level than a state
reused as it was written, by at most half a unit in the last place of its magnitude; every
state is a convex combination of V rows, so that magnitude is at most max |V| over the
group's keys.  The output bar therefore grows, per merged state r read with weight
w_r = exp(lse_r - L), by w_r * levels * ulp(max |V|) / 2.  Without merges it is the plain
bar."""
import numpy as np
import pytest

import gpu_helpers as gh
from gpu_helpers import BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, log
from workloads import Policy, custom_config
from workloads import configs as wcfg

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dita():
    import partial_state_reuse_amd as d
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return d


CASES = [
    # name, frames, gh, gw, P, D, heads, steps, dtype, merges {step: [(group, "sel" | None)]}
    ("groups-bf16-d64", 8, 5, 7, 8, 64, 2, 5, "bf16", {1: [(2, "sel"), (4, "sel")]}),
    ("groups-bf16-d128-all", 8, 4, 6, 8, 128, 1, 4, "bf16", {1: [(2, None)]}),
    ("groups-bf16-d72-ragged", 6, 5, 7, 6, 72, 1, 4, "bf16", {1: [(3, "sel")], 2: [(6, None)]}),
    ("groups-f32", 8, 2, 4, 8, 64, 2, 5, "f32", {2: [(2, "sel")]}),
    ("groups-bf16-128-partitions", 4, 16, 16, 128, 64, 1, 4, "bf16",
     {1: [(8, "sel")], 2: [(32, None)]}),                       # 8-row partitions
]


def _always_reused(masks, P, g):
    NG = (P + g - 1) // g
    sel = np.ones((P, NG), bool)
    for M in masks[1:]:
        for i in range(P):
            for J in range(NG):
                if any(M[i, j] != 2 for j in range(J * g, min(P, J * g + g))):
                    sel[i, J] = False
    return sel


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_group_composition(dita, case):
    run_group_case(dita, case)


@pytest.mark.parametrize("seed", list(range(48)) + [1357])
def test_group_composition_sweep(dita, seed):
    """Random small workloads (3-8 frames, 3-10 x 3-16 grid, 3-10 partitions, head dim, path)
    with a random group size merged after the anchor (every eligible group, or the groups
    every later step reuses whole) and sometimes again after step 2."""
    rng = np.random.default_rng(3000 + seed)
    T, gh_, gw = int(rng.integers(3, 9)), int(rng.integers(3, 11)), int(rng.integers(3, 17))
    P = int(rng.integers(3, 11))
    dt = "bf16" if rng.random() < 0.75 else "f32"
    D = int(rng.choice([64, 72, 128] if dt == "bf16" else [16, 64]))
    H, S = int(rng.integers(1, 3)), int(rng.integers(3, 6))
    merges = {1: [(int(rng.integers(2, 5)), "sel" if rng.random() < 0.5 else None)]}
    if rng.random() < 0.4:
        merges[2] = [(int(rng.integers(2, P + 1)), None)]
    run_group_case(dita, (f"groups-sweep-{seed}", T, gh_, gw, P, D, H, S, dt, merges),
                   require_merge=False)


def ulp(x, bf16):
    """Unit in the last place of bf16 (8 significant bits) or f32 (24) at |x|."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - (7 if bf16 else 23))


def merge_rounding_bar(r, offs, P, resolved, inputs, step, bf16):
    """Extra output allowance [N, D] at 0-based step `step` for the merged states read there:
    w_r * levels_r * ulp(max |V| over the group's keys and the steps so far) / 2, where
    levels_r counts the merge levels (group sizes g) that merged something into the state
    read at (i, j): a member without a state of its own in the same g-group."""
    levels = [g for t, lst in resolved.items() if t <= step for (g, _) in lst]
    extra = np.zeros((offs[-1], inputs[0][2].shape[1]))
    if not levels:
        return extra
    vmax = [max(float(np.abs(inputs[t][2][offs[j]:offs[j + 1]]).max()) for t in range(step + 1))
            for j in range(P)]
    for i in range(P):
        rows = slice(offs[i], offs[i + 1])
        covered = [m for m in range(P) if r.mask[i, m] == 2 and (i, m) not in r.block_o]
        for j in range(P):
            if r.mask[i, j] != 2 or (i, j) not in r.block_o:
                continue
            mine = [g for g in levels if any(m // g == j // g for m in covered)]
            if not mine:
                continue                                   # not a merged state
            members = {m for g in mine for m in range(P) if m // g == j // g}
            w = np.exp(r.block_lse[(i, j)] - r.lse[rows])
            vm = max(vmax[m] for m in members)
            extra[rows] += (w * len(mine) * 0.5 * float(ulp(vm, bf16)))[:, None]
    return extra


def run_group_case(dita, case, require_merge=True):
    import oracle
    from oracle.policy import active_mask, partition_offsets
    name, T, gh_, gw, P, D, H, S, dt, merges = case
    sched = wcfg.AnchorThen(Policy(kind=wcfg.FRAME_THRESHOLD, max_fresh_frame_dist=1))
    cfg = custom_config(name=name, idx=85, heads=H, head_dim=D, frames=T, grid_h=gh_,
                        grid_w=gw, num_partitions=P, steps=S, qkv_dtype=dt, cache_dtype=dt,
                        schedule=sched)
    heads = [(0, h) for h in range(H)]
    offs = partition_offsets(cfg.tokens, P)
    act = active_mask(offs, cfg.frame_tokens, False)
    base = oracle.run_head(cfg, 0, 0, cache_mode="fp64", rows=[0])   # masks only
    resolved = {s: [(g, _always_reused([st.mask for st in base], P, g) if sel == "sel" else None)
                    for (g, sel) in lst] for s, lst in merges.items()}
    log(f"case {name}: N={cfg.tokens} P={P} D={D} H={H} steps={S} {dt} merges="
        f"{ {s: [g for g, _ in l] for s, l in merges.items()} }")
    dev, kept = gh.device_inputs(cfg, S, keep_heads=set(heads))
    cache = dita.Cache(dita.geometry_from(cfg), active_mask=act.astype(np.uint8))
    plans, outs, lses, n_merged = [], [], [], []
    for s in range(1, S + 1):
        cache.set_policy(dita.policy_from(cfg.policy(s)))
        plans.append(cache.plan())
        q, k, v = dev[s - 1]
        out, lse = cache.step(q, k, v)
        outs.append(out.cpu().numpy())
        lses.append(lse.cpu().numpy())
        for (g, sel) in resolved.get(s, []):
            n_merged.append(cache.merge_groups(g, select=sel))
    st = cache.stats()
    cache.free()
    if require_merge:
        assert sum(n_merged) > 0
    assert st["device_reuse_blocks"] == st["host_reuse_blocks"]
    log(f"groups merged: {n_merged}; states read on device {st['device_reuse_blocks']}")

    ok = True
    bf = dt == "bf16"
    for (b, h) in heads:
        ref = oracle.run_head(cfg, b, h, cache_mode="fp64", merges=resolved, active=act,
                              inputs=kept[(b, h)], keep_block_lse=True)
        for s in range(S):
            p, r = plans[s], ref[s]
            assert np.array_equal(p["mask"], r.mask), f"step {s + 1}: mask"
            assert np.array_equal(p["reuse_ptr"], r.reuse_ptr), f"step {s + 1}: reuse_ptr"
            assert np.array_equal(p["reuse_cols"], r.reuse_cols), f"step {s + 1}: reuse_cols"
            err = np.abs(np.asarray(outs[s][b, h], np.float64) - r.out)
            extra = merge_rounding_bar(r, offs, P, resolved, kept[(b, h)], s, bf)
            bar = (BF16_MAX_ABS if bf else F32_MAX_ABS) + extra
            good = bool(np.all(err <= bar)) and (not bf or float(err.mean()) <= BF16_MEAN_ABS)
            log(f"step {s + 1} head {h} out: max-abs {err.max():.3e} mean-abs {err.mean():.3e} "
                f"(largest merge allowance {extra.max():.2e}) {'ok' if good else 'FAIL'}")
            ok &= good
            lerr = float(np.abs(lses[s][b, h] - r.lse).max())
            ok &= lerr < (2e-3 if dt == "bf16" else 1e-5)
    assert ok
