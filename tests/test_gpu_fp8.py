"""GPU parity of the fp8 (e4m3) state cache, through the C ABI.

The cache is lossy by design: the comparison is with the oracle that rounds its cached
states to e4m3 the same way (nearest even, saturating).  The GPU and the oracle round values
that differ by their arithmetic error, so a cached element can land one e4m3 spacing apart on
the two sides; each reused state r enters the output with weight w_r = exp(lse_r - L), so the
element-wise bar is the bf16 output bar plus sum over reused states of w_r * spacing(|O_r|).
A state merged from a group (group composition) is rounded twice: its members' cached states
(each possibly one spacing apart) enter the merge with their shares exp(lse_m - L_group), and
the merged result is rounded again, so its term is w_r * (spacing(|O_r|) + sum over members of
share_m * spacing(|O_m|)).  lse does not depend on the O rounding and keeps the bf16 bar.  The
distance to the exact (fp64, unrounded) result is logged: it is the accuracy the compression
costs."""
import numpy as np
import pytest

import gpu_helpers as gh
from gpu_helpers import BF16_MAX_ABS, BF16_MEAN_ABS, log
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


def spacing8(x):
    ax = np.abs(np.asarray(x, np.float64))
    k = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** -9)))
    return np.exp2(np.maximum(k, -6.0) - 3.0)


def merged_members(r, i, j, merges, P):
    """The blocks whose states the state read at (i, j) merges (j included), or [] if it is
    not a merged state.  Merges here are one level, after step 1: members of a merged group
    show REUSE in the mask without a state of their own."""
    if not merges:
        return []
    assert list(merges) == [1] and len(merges[1]) == 1, "one merge level, after step 1"
    g = merges[1][0][0]
    covered = [m for m in range(P) if m != j and m // g == j // g and r.mask[i, m] == 2
               and (i, m) not in r.block_o]
    return [j] + covered if covered else []


CASES = [
    # name, frames, gh, gw, P, D, heads, steps, schedule, merges
    ("fp8-d64-tails", 4, 10, 26, 8, 64, 2, 4, "budget", None),     # 130-row partitions
    ("fp8-d128", 3, 8, 10, 6, 128, 2, 4, "frame", None),
    ("fp8-d72", 2, 9, 11, 3, 72, 2, 3, "frame", None),
    ("fp8-d64-merged", 8, 5, 7, 8, 64, 1, 4, "frame", {1: [(2, None)]}),
    ("fp8-d64-256-partitions", 4, 16, 16, 256, 64, 1, 3, "budget", None),   # 4-row partitions
]


@pytest.mark.parametrize("seed", list(range(48)) + [270])
def test_fp8_cache_sweep(dita, seed):
    """Random small workloads with the fp8 cache (2-6 frames, 3-12 x 3-20 grid, 2-10
    partitions, head dim, schedule), sometimes with pairs or triples merged after the anchor."""
    rng = np.random.default_rng(4000 + seed)
    T, gh_, gw = int(rng.integers(2, 7)), int(rng.integers(3, 13)), int(rng.integers(3, 21))
    P = int(rng.integers(2, 11))
    D = int(rng.choice([64, 72, 128]))
    H, S = int(rng.integers(1, 3)), int(rng.integers(2, 5))
    kind = "budget" if rng.random() < 0.5 else "frame"
    merges = {1: [(int(rng.integers(2, 4)), None)]} if rng.random() < 0.4 else None
    test_fp8_cache(dita, (f"fp8-sweep-{seed}", T, gh_, gw, P, D, H, S, kind, merges))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_cache(dita, case):
    import oracle
    from oracle.policy import active_mask, partition_offsets
    name, T, gh_, gw, P, D, H, S, kind, merges = case
    if kind == "budget":
        sched = wcfg.AnchorThen(Policy(kind=wcfg.FRESH_BUDGET, reuse_percent=60))
    else:
        sched = wcfg.AnchorThen(Policy(kind=wcfg.FRAME_THRESHOLD, max_fresh_frame_dist=1))
    cfg = custom_config(name=name, idx=90, heads=H, head_dim=D, frames=T, grid_h=gh_, grid_w=gw,
                        num_partitions=P, steps=S, qkv_dtype="bf16", cache_dtype="fp8",
                        schedule=sched)
    heads = [(0, h) for h in range(H)]
    offs = partition_offsets(cfg.tokens, P)
    act = active_mask(offs, cfg.frame_tokens, False)
    log(f"case {name}: N={cfg.tokens} P={P} D={D} H={H} steps={S} cache fp8 merges={merges}")
    dev, kept = gh.device_inputs(cfg, S, keep_heads=set(heads))
    cache = dita.Cache(dita.geometry_from(cfg), active_mask=act.astype(np.uint8))
    outs, lses, plans = [], [], []
    for s in range(1, S + 1):
        cache.set_policy(dita.policy_from(cfg.policy(s)))
        plans.append(cache.plan())
        q, k, v = dev[s - 1]
        out, lse = cache.step(q, k, v)
        outs.append(out.cpu().numpy())
        lses.append(lse.cpu().numpy())
        for (g, sel) in (merges or {}).get(s, []):
            cache.merge_groups(g, select=sel)
    # cached states written at the last step, read back
    last = plans[-1]["mask"]
    slots = {}
    for (b, h) in heads[:1]:
        for i in range(P):
            for j in range(P):
                if last[i, j] == 1:
                    o_, l_ = cache.read_slot(b, h, i, j)
                    slots[(i, j)] = (o_.cpu().numpy(), l_.cpu().numpy())
    cache.free()

    ok = True
    for (b, h) in heads:
        emu = oracle.run_head(cfg, b, h, cache_mode="emulate", merges=merges, active=act,
                              inputs=kept[(b, h)], keep_block_lse=True)
        exact = oracle.run_head(cfg, b, h, cache_mode="fp64", merges=merges, active=act,
                                inputs=kept[(b, h)])
        for s in range(S):
            r = emu[s]
            assert np.array_equal(plans[s]["mask"], r.mask), f"step {s + 1}: mask"
            bound = np.full((cfg.tokens, D), BF16_MAX_ABS)
            for i in range(P):
                rows = slice(offs[i], offs[i + 1])
                for j in range(P):
                    if r.mask[i, j] == 2 and (i, j) in r.block_o:
                        wgt = np.exp(r.block_lse[(i, j)] - r.lse[rows])
                        sp = spacing8(r.block_o[(i, j)])
                        for m in merged_members(r, i, j, merges, P):
                            # members hold their anchor-step states (merged after step 1)
                            share = np.exp(emu[0].block_lse[(i, m)] - r.block_lse[(i, j)])
                            sp = sp + share[:, None] * spacing8(emu[0].block_o[(i, m)])
                        bound[rows] += wgt[:, None] * sp
            err = np.abs(outs[s][b, h] - r.out)
            slack = float((err - bound).max())
            lerr = float(np.abs(lses[s][b, h] - r.lse).max())
            xerr = np.abs(outs[s][b, h] - exact[s].out)
            log(f"step {s + 1} head {h}: vs fp8 oracle max {err.max():.3e} mean {err.mean():.3e} "
                f"(bar slack {slack:.2e}); lse {lerr:.2e}; vs exact max {xerr.max():.3e} "
                f"mean {xerr.mean():.3e}")
            ok &= slack <= 0 and lerr < 2e-3 and err.mean() <= BF16_MEAN_ABS
        if (b, h) == heads[0]:
            r = emu[-1]
            for (i, j), (o_, l_) in slots.items():
                want = oracle.round_fp8_e4m3(r.block_o[(i, j)])
                d = np.abs(o_ - want)
                assert np.all(d <= spacing8(want) + 1e-6), f"slot ({i},{j}) max {d.max():.3e}"
                assert np.abs(l_ - r.block_lse[(i, j)]).max() < 2e-3
            log(f"{len(slots)} cached fp8 states read back within one e4m3 spacing")
    assert ok
