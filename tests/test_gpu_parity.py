"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on identical seeded
inputs.  Masks, work lists, counts and device-counted blocks are compared bit for bit;
outputs within max-abs 2e-2 / mean-abs 2e-3 for bf16 inputs and 1e-5 for the f32 workload.

Small geometries compare every output element; the full-size workloads run at their real
shape in the bench's launch configuration and compare sampled rows (the first two, last two
and random rows of every partition) of a few heads over every step."""
import numpy as np
import pytest

import gpu_helpers as gh
from gpu_helpers import compare, log
from workloads import CONFIGS, Policy, custom_config
from workloads import configs as wcfg

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dita():
    import partial_state_reuse_amd as d
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return d


def oracle_mod():
    import oracle
    return oracle


def active_for(cfg):
    from oracle.policy import active_mask, partition_offsets
    offs = partition_offsets(cfg.tokens, cfg.num_partitions)
    return active_mask(offs, cfg.frame_tokens, cfg.policy(1).tile_sparse).astype(np.uint8)


def run_and_check(dita, cfg, heads, rows=None, steps=None, policies=None, offsets=None,
                  check_slots=True, modify=None, recomputes=None, layout="bhnd",
                  expect_f32_bar=None):
    """Run every step on the GPU and compare with the oracle on `heads` (and `rows`).

    layout      "bhnd", or "bnhd": Q, K, V and out handed to the library as [B, N, H, D]
    modify      optional callable(dev, kept) that edits the device inputs and the host copies
                of `heads` alike before the run
    recomputes  None, 0 (no fresh block may be computed a second time after its cached lse
                was rejected as the softmax reference) or "some" (at least one must be)
    expect_f32_bar  f32 workloads: the max-abs bar every head must be held to (checked)"""
    oracle = oracle_mod()
    S = steps or cfg.steps
    bf = cfg.qkv_dtype == "bf16"
    log(f"case {cfg.name} B={cfg.batch} H={cfg.heads} N={cfg.tokens} D={cfg.head_dim} "
        f"P={cfg.num_partitions} steps={S} heads={heads} rows={'all' if rows is None else len(rows)}")
    dev, kept = gh.device_inputs(cfg, S, keep_heads=set(heads))
    if modify is not None:
        modify(dev, kept)
    g = dita.geometry_from(cfg, offsets=offsets)
    if layout == "bnhd":
        g.layout = dita.LAYOUT_BNHD
    cache = dita.Cache(g, active_mask=active_for(cfg) if offsets is None else None)
    pols = policies or [cfg.policy(s) for s in range(1, S + 1)]
    outs = []
    plans = []
    for s in range(S):
        cache.set_policy(dita.policy_from(pols[s]))
        plans.append(cache.plan())
        q, k, v = dev[s]
        if layout == "bnhd":
            q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
        out, lse = cache.step(q, k, v)
        if layout == "bnhd":
            out = out.transpose(1, 2)
        sel = torch.as_tensor(rows, device=out.device) if rows is not None else None
        per_head = {}
        for (b, h) in heads:
            o = out[b, h] if sel is None else out[b, h].index_select(0, sel)
            l = lse[b, h] if sel is None else lse[b, h].index_select(0, sel)
            per_head[(b, h)] = (o.cpu().numpy(), l.cpu().numpy())
        outs.append(per_head)
        if check_slots and s == S - 1:
            slot_checks = {}
            for (b, h) in heads[:1]:
                for (i, j) in [(0, 0), (cfg.num_partitions - 1, cfg.num_partitions - 1)]:
                    slot_checks[(b, h, i, j)] = [t.cpu().numpy() for t in cache.read_slot(b, h, i, j)]
    torch.cuda.synchronize()
    st = cache.stats()
    ok_all = True
    worst = (0.0, 0.0)
    offs_used = oracle.partition_offsets(cfg.tokens, cfg.num_partitions) \
        if offsets is None else offsets
    n_max = int(np.max(np.diff(np.asarray(offs_used))))
    for (b, h) in heads:
        # f32: the bar for blocks of this length (gpu_helpers.f32_bar)
        f32_max = gh.f32_bar(n_max, max(float(np.abs(x[2]).max()) for x in kept[(b, h)][:S]))
        if expect_f32_bar is not None and not bf:
            assert f32_max == expect_f32_bar, (f32_max, expect_f32_bar)
        # the bar is against fp64 (no cache rounding); the reference that also rounds its
        # cache to the workload's precision must agree on average
        ref = oracle.run_head(cfg, b, h, steps=S, rows=rows, policies=pols,
                              inputs=kept[(b, h)], offsets=offsets, cache_mode="fp64")
        emu = oracle.run_head(cfg, b, h, steps=S, rows=rows, policies=pols,
                              inputs=kept[(b, h)], offsets=offsets, cache_mode="emulate")
        for s in range(S):
            r = ref[s]
            p = plans[s]
            assert np.array_equal(p["mask"], r.mask), f"mask step {s + 1}"
            assert np.array_equal(p["fresh_ptr"], r.fresh_ptr)
            assert np.array_equal(p["fresh_cols"], r.fresh_cols)
            assert np.array_equal(p["reuse_ptr"], r.reuse_ptr)
            assert np.array_equal(p["reuse_cols"], r.reuse_cols)
            assert np.array_equal(p["counts"], r.counts)
            o, l = outs[s][(b, h)]
            ok, mx, mean = compare(o, r.out, bf, f"  b={b} h={h} step {s + 1} out", f32_max)
            worst = (max(worst[0], mx), max(worst[1], mean))
            ok_all &= ok
            emean = float(np.mean(np.abs(o - emu[s].out)))
            ok_all &= emean <= (gh.BF16_MEAN_ABS if bf else gh.F32_MAX_ABS)
            lerr = float(np.max(np.abs(l - r.lse)))
            assert lerr < (2e-3 if bf else 1e-5), f"lse step {s + 1}: {lerr}"
        if check_slots and (b, h) == heads[0]:
            # the last step's cached states of two diagonal blocks (fresh every step)
            for (bb, hh, i, j), (o_slot, l_slot) in slot_checks.items():
                offs = oracle.partition_offsets(cfg.tokens, cfg.num_partitions) \
                    if offsets is None else offsets
                Qs, Ks, Vs = (np.asarray(x, np.float64) for x in kept[(b, h)][S - 1])
                sl_i, sl_j = slice(offs[i], offs[i + 1]), slice(offs[j], offs[j + 1])
                O_ref, l_ref = oracle.block_state(Qs[sl_i], Ks[sl_j], Vs[sl_j],
                                                  1.0 / np.sqrt(cfg.head_dim))
                rnd = oracle.round_bf16 if bf else oracle.round_f32
                ok = gh.compare_cached(o_slot, rnd(O_ref), O_ref, bf, f"  cached state ({i},{j})",
                                       f32_max)
                assert ok, f"slot ({i},{j})"
                assert np.max(np.abs(l_slot - l_ref)) < (2e-3 if bf else 1e-5)
    bh = cfg.batch * cfg.heads
    assert st["steps_done"] == S
    assert st["device_fresh_blocks"] == st["host_fresh_blocks"]
    assert st["device_reuse_blocks"] == st["host_reuse_blocks"]
    assert st["device_v_range_errors"] == 0
    assert st["host_fresh_blocks"] == bh * sum(int(p["counts"][1]) for p in plans)
    if recomputes == 0:
        assert st["device_ref_recomputes"] == 0, st["device_ref_recomputes"]
    elif recomputes == "some":
        assert st["device_ref_recomputes"] > 0
    log(f"case {cfg.name}: worst max-abs {worst[0]:.3e} mean-abs {worst[1]:.3e}; "
        f"blocks recomputed after a rejected reference: {st['device_ref_recomputes']}")
    assert ok_all
    cache.free()
    return outs


# --------------------------------------------------------------------------------------
# small geometries: every element
# --------------------------------------------------------------------------------------
def test_tiny_f32_workload_all_heads(dita):
    """The small fp32 workload (64-key blocks) is held to exactly the stated 1e-5."""
    cfg = CONFIGS[1]
    assert gh.f32_bar(64, 100.0) == 1e-5
    run_and_check(dita, cfg, heads=[(0, 0), (0, 1)], expect_f32_bar=1e-5)


def test_image_bf16_d72_workload(dita):
    """Every head of the image workload, every element."""
    cfg = CONFIGS[2]
    run_and_check(dita, cfg, heads=[(0, h) for h in range(cfg.heads)])


RAGGED_CASES = [
    # (name, frames, gh, gw, P, D, heads, steps, policy kind)
    ("ragged-d64", 3, 10, 13, 5, 64, 2, 3, "budget"),
    ("ragged-d72", 2, 9, 11, 3, 72, 2, 3, "frame"),
    ("ragged-d128", 2, 15, 20, 7, 128, 2, 3, "budget"),
    ("single-partition-d64", 1, 7, 9, 1, 64, 1, 2, "frame"),
    ("tiny-partitions-d64", 1, 3, 11, 11, 64, 1, 3, "budget"),
    ("tile-sparse-d64", 6, 5, 7, 6, 64, 2, 4, "tile"),
    ("video-slice-d64", 2, 45, 80, 8, 64, 2, 3, "budget"),
    ("many-partitions-d64", 4, 16, 16, 256, 64, 1, 2, "tile"),     # 4-row partitions
    ("max-partitions-d64", 4, 16, 16, 1024, 64, 1, 2, "budget"),   # 1024 one-row partitions
    ("many-partitions-d72", 4, 16, 16, 128, 72, 1, 2, "frame"),     # 8-row partitions
    ("many-partitions-d128", 4, 16, 16, 200, 128, 1, 3, "budget"),  # 5- and 6-row partitions
]


@pytest.mark.parametrize("case", RAGGED_CASES, ids=[c[0] for c in RAGGED_CASES])
def test_ragged_bf16_geometries(dita, case):
    name, T, gh_, gw, P, D, H, S, kind = case
    if kind == "budget":
        sched = wcfg.AnchorThen(Policy(kind=wcfg.FRESH_BUDGET, reuse_percent=60))
    elif kind == "frame":
        sched = wcfg.AnchorThen(Policy(kind=wcfg.FRAME_THRESHOLD, max_fresh_frame_dist=0))
    else:
        sched = wcfg.AnchorThen(Policy(kind=wcfg.FRAME_THRESHOLD, max_fresh_frame_dist=1,
                                       tile_sparse=True))
    cfg = custom_config(name=name, idx=40, heads=H, head_dim=D, frames=T, grid_h=gh_,
                        grid_w=gw, num_partitions=P, steps=S, qkv_dtype="bf16",
                        cache_dtype="bf16", schedule=sched)
    run_and_check(dita, cfg, heads=[(0, h) for h in range(H)])


def _sweep_case(seed):
    """A random small workload: geometry (1-4 frames, 3-16 x 3-24 grid, 1-10 partitions, so
    partitions range from a few rows, handled by tail workgroups alone, to several row
    groups), head dim, heads, steps, path (bf16 three times in four) and block policy."""
    rng = np.random.default_rng(1000 + seed)
    T, gh_, gw = int(rng.integers(1, 5)), int(rng.integers(3, 17)), int(rng.integers(3, 25))
    N = T * gh_ * gw
    P = int(rng.integers(1, min(10, N) + 1))
    bf = bool(rng.random() < 0.75)
    D = int(rng.choice([64, 72, 128] if bf else [16, 40, 64]))
    H, S = int(rng.integers(1, 3)), int(rng.integers(2, 5))
    kind = int(rng.integers(0, 4))
    if kind == 0:
        pol = Policy(kind=wcfg.FRESH_BUDGET, reuse_percent=int(rng.integers(0, 101)))
    elif kind == 1:
        pol = Policy(kind=wcfg.FRAME_THRESHOLD, max_fresh_frame_dist=int(rng.integers(0, 3)))
    elif kind == 2:
        pol = Policy(kind=wcfg.CENTROID_THRESHOLD, max_fresh_centroid2=int(rng.integers(0, 2 * N)))
    else:
        pol = Policy(kind=wcfg.FRAME_THRESHOLD, max_fresh_frame_dist=1, tile_sparse=True)
    dt = "bf16" if bf else "f32"
    return custom_config(name=f"sweep-{seed}", idx=200 + seed, heads=H, head_dim=D, frames=T,
                         grid_h=gh_, grid_w=gw, num_partitions=P, steps=S, qkv_dtype=dt,
                         cache_dtype=dt, schedule=wcfg.AnchorThen(pol))


@pytest.mark.parametrize("seed", list(range(48)) + [1242])
def test_random_geometry_sweep(dita, seed):
    """Random small workloads, every element and every step against the oracle; odd seeds
    hand Q, K, V and out over as [B, N, H, D]."""
    cfg = _sweep_case(seed)
    run_and_check(dita, cfg, heads=[(0, h) for h in range(cfg.heads)],
                  layout="bnhd" if seed % 2 else "bhnd")


def test_explicit_masks_and_custom_offsets_bf16(dita):
    """Explicit masks with skips and ragged hand-picked offsets (including a 1-token and a
    33-token partition)."""
    offs = [0, 1, 34, 100, 161, 257, 300]
    P = 6
    rng = np.random.default_rng(5)
    masks = []
    valid = np.zeros((P, P), bool)
    for s in range(4):
        M = rng.integers(0, 3, (P, P)).astype(np.uint8)
        M[(M == 2) & ~valid] = 1
        np.fill_diagonal(M, 1)
        valid |= M == 1
        masks.append(Policy(kind=wcfg.EXPLICIT, explicit_mask=tuple(int(x) for x in M.ravel())))
    cfg = custom_config(name="explicit-offsets", idx=41, heads=2, head_dim=64, frames=3,
                        grid_h=10, grid_w=10, num_partitions=P, steps=4, qkv_dtype="bf16",
                        cache_dtype="bf16")
    run_and_check(dita, cfg, heads=[(0, 0), (0, 1)], policies=masks, offsets=offs)


def test_fixed_reference_fallback_bf16(dita):
    """A fresh block whose slot holds an earlier state takes that state's lse as its softmax
    reference.  Here one key partition's K is scaled by 4 on step 2 and restored on step 3,
    so the lse of its blocks jumps up, then down, far beyond the accepted window: those
    blocks are computed a second time with the running maximum (counted on the device),
    and the outputs still match the oracle on the same inputs.  Two 130-row partitions
    exercise the tail waves too."""
    from oracle.policy import partition_offsets
    sched = wcfg.AnchorThen(Policy(kind=wcfg.FRESH_BUDGET, reuse_percent=0))
    cfg = custom_config(name="ref-jump", idx=47, heads=2, head_dim=64, frames=4, grid_h=10,
                        grid_w=26, num_partitions=8, steps=3, qkv_dtype="bf16",
                        cache_dtype="bf16", schedule=sched)
    offs = partition_offsets(cfg.tokens, cfg.num_partitions)
    j0, j1 = offs[3], offs[4]

    def modify(dev, kept):
        dev[1][1][:, :, j0:j1, :] *= 4                 # exact in bf16
        for bh in kept:
            kept[bh][1][1][j0:j1] *= 4
    run_and_check(dita, cfg, heads=[(0, 0), (0, 1)], modify=modify, recomputes="some")


def test_fixed_reference_smooth_drift_bf16(dita):
    """With the seeded drift between steps every fresh block keeps its cached lse as the
    reference: no block is computed twice."""
    sched = wcfg.AnchorThen(Policy(kind=wcfg.FRESH_BUDGET, reuse_percent=40))
    cfg = custom_config(name="ref-drift", idx=48, heads=2, head_dim=64, frames=4, grid_h=10,
                        grid_w=26, num_partitions=8, steps=4, qkv_dtype="bf16",
                        cache_dtype="bf16", schedule=sched)
    run_and_check(dita, cfg, heads=[(0, 0), (0, 1)], recomputes=0)


def test_f32_random_geometries(dita):
    for seed, (T, gh_, gw, P, D) in enumerate([(2, 5, 7, 3, 16), (3, 4, 9, 5, 64),
                                               (1, 10, 10, 7, 40)]):
        sched = wcfg.AnchorThen(Policy(kind=wcfg.FRESH_BUDGET, reuse_percent=50))
        cfg = custom_config(name=f"f32-{seed}", idx=42 + seed, heads=2, head_dim=D, frames=T,
                            grid_h=gh_, grid_w=gw, num_partitions=P, steps=3,
                            qkv_dtype="f32", cache_dtype="f32", schedule=sched)
        run_and_check(dita, cfg, heads=[(0, 0), (0, 1)])


def test_no_drift_reuse_is_noop_on_gpu(dita):
    """With unchanged inputs, a reuse step reproduces the all-fresh step (f32 path: within
    the f32 tolerance; the cached states are the fresh ones)."""
    cfg = custom_config(name="nodrift", idx=45, heads=2, head_dim=64, frames=4, grid_h=4,
                        grid_w=8, num_partitions=4, steps=3, qkv_dtype="f32",
                        cache_dtype="f32", drift=0.0, schedule=CONFIGS[1].schedule)
    dev, _ = gh.device_inputs(cfg, 3)
    c = dita.Cache(dita.geometry_from(cfg))
    res = []
    for s in range(3):
        c.set_policy(dita.policy_from(cfg.policy(min(s + 1, 2))))
        out, _ = c.step(*dev[s])
        res.append(out.cpu().numpy())
    assert np.max(np.abs(res[1] - res[0])) <= gh.F32_MAX_ABS
    assert np.max(np.abs(res[2] - res[0])) <= gh.F32_MAX_ABS


def test_determinism_and_side_stream(dita):
    cfg = CONFIGS[2]
    dev, _ = gh.device_inputs(cfg, 2)
    outs = []
    for use_side in (False, True, True):
        c = dita.Cache(dita.geometry_from(cfg))
        stream = torch.cuda.Stream() if use_side else torch.cuda.current_stream()
        with torch.cuda.stream(stream):
            for s in range(2):
                c.set_policy(dita.policy_from(cfg.policy(s + 1)))
                out, lse = c.step(*dev[s])
        stream.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
        c.free()
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])


def test_error_paths_on_device(dita):
    cfg = CONFIGS[1]
    dev, _ = gh.device_inputs(cfg, 2)
    c = dita.Cache(dita.geometry_from(cfg))
    with pytest.raises(dita.DitaError) as e:
        c.step(*dev[0])
    assert e.value.name == "NO_POLICY"
    c.set_policy(dita.policy_from(cfg.policy(1)))
    c.step(*dev[0])
    c.set_policy(dita.policy_from(cfg.policy(2)))
    c.step(*dev[1])
    c.reset()
    with pytest.raises(dita.DitaError) as e:
        c.set_policy(dita.policy_from(cfg.policy(2)))
    assert e.value.name == "CACHE_MISS"
    with pytest.raises(dita.DitaError) as e:
        c.read_slot(0, 0, 0, 3)
    assert e.value.name == "CACHE_MISS"
    # recovery: anchor step, then reuse works again
    c.set_policy(dita.policy_from(cfg.policy(1)))
    c.step(*dev[0])
    c.set_policy(dita.policy_from(cfg.policy(2)))
    c.step(*dev[1])
    torch.cuda.synchronize()
    assert c.stats()["steps_done"] == 4


# --------------------------------------------------------------------------------------
# full-size workloads, sampled rows
# --------------------------------------------------------------------------------------
def _full(dita, idx, heads, per_part, layout="bhnd"):
    from oracle.policy import partition_offsets
    cfg = CONFIGS[idx]
    rows = gh.sample_rows(partition_offsets(cfg.tokens, cfg.num_partitions), per_part,
                          np.random.default_rng(idx))
    run_and_check(dita, cfg, heads=heads, rows=rows, recomputes=0, layout=layout)


def test_full_video29f_720p(dita):
    _full(dita, 3, heads=[(0, 0), (0, 13), (0, 23)], per_part=12)


def test_full_video29f_720p_every_row_of_one_head(dita):
    """The 29-frame workload at full size in the bench's launch configuration, every row and
    every element of one head over the whole 10-step schedule (the anchor's running-maximum
    kernel, then nine fixed-reference passes with 608 of 1024 states reused), against the fp64
    oracle: the row groups, the packed tail sub-tiles (4 rows of every partition) and the
    split row groups all write rows of this head."""
    run_and_check(dita, CONFIGS[3], heads=[(0, 11)], rows=None, recomputes=0)


def test_full_video93f_every_row_of_one_head(dita):
    """The 93-frame tile-sparse workload at full size (86400 tokens, 24 partitions of 3600,
    92 of 576 blocks active), every element of one head over its anchor and first reuse step,
    against the fp64 oracle."""
    run_and_check(dita, CONFIGS[4], heads=[(0, 7)], rows=None, steps=2, recomputes=0)


def test_full_cfg_long_video_every_row_of_one_head(dita):
    """The CFG workload at full size (B = 2, 40 heads, 26520 tokens, D = 128, 16 partitions of
    1658/1657), every element of one head of the second branch over its two anchor steps (the
    running-maximum kernel, then the fixed-reference pass with every block fresh) and its first
    step with 70 % of the states reused, against the fp64 oracle."""
    run_and_check(dita, CONFIGS[5], heads=[(1, 39)], rows=None, steps=3, recomputes=0)


def test_full_video29f_720p_token_major(dita):
    """The same workload with Q, K, V and out as [B, N, H, D] (a token stride of H D = 1536)."""
    _full(dita, 3, heads=[(0, 5), (0, 18)], per_part=8, layout="bnhd")


def test_full_video93f_tile_sparse(dita):
    _full(dita, 4, heads=[(0, 0), (0, 23)], per_part=8)


def test_full_cfg_long_video_d128(dita):
    _full(dita, 5, heads=[(0, 0), (0, 39), (1, 0), (1, 39)], per_part=8)
