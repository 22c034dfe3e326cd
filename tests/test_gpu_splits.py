"""GPU: split row groups, through the C ABI.

On the bf16 path the row groups dispatched last on each XCD run as two (or more) workgroups,
consecutive shares of the row's fresh blocks and reused states, each leaving its partial
merge of the rows in a workspace, and merge_splits combines the parts and writes the rows.  The merge is the same log-sum-exp merge as the one over blocks (DiTango, "State-Centric
Parallel Runtime / Composizione dello Stato": attention states, output and log-sum-exp,
combine associatively and commutatively), so a split run must meet the fp64 oracle's bars
like any other, and agree with the unsplit run up to the association of the sums.

The default splits only grids of two rounds of workgroups and more (the full-size parity
tests run it); here DITA_SPLITS_PER_XCD forces splits on small workloads, whose every row
is then compared: bf16 with tail workgroups (in 2 and in 3 parts), D = 128, a bf16 output, a
fixed reference that is rejected (the second pass re-runs the splits), the allocation-free
step, and the workspace's size in the cache's bytes.  With an fp8 cache the split run is
held to the unsplit one (the fp8 cache's own bars are those of its tests)."""
import numpy as np
import pytest

import gpu_helpers as gh
from gpu_helpers import log
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


def _cfg(name, idx, **kw):
    d = dict(heads=3, head_dim=64, frames=4, grid_h=20, grid_w=26, num_partitions=8, steps=3,
             qkv_dtype="bf16", cache_dtype="bf16",
             schedule=wcfg.AnchorThen(Policy(kind=wcfg.FRESH_BUDGET, reuse_percent=50)))
    d.update(kw)
    return custom_config(name=name, idx=idx, **d)


def _split_bytes(cfg, splits, parts=2):
    dp = 64 if cfg.head_dim <= 64 else (96 if cfg.head_dim <= 96 else 128)
    return splits * parts * 256 * (2 + dp // 2) * 4


def _required(dita, cfg):
    from test_gpu_parity import active_for
    c = dita.Cache(dita.geometry_from(cfg), active_mask=active_for(cfg))
    n = c.required_bytes
    c.free()
    return n


@pytest.mark.parametrize("case", ["bf16-d64-tails", "bf16-d64-3-parts", "bf16-d128",
                                  "bf16-out"])
def test_forced_splits_meet_the_oracle(dita, monkeypatch, case):
    from test_gpu_parity import run_and_check
    parts = 3 if case == "bf16-d64-3-parts" else 2
    monkeypatch.setenv("DITA_SPLIT_PARTS", str(parts))
    if case.startswith("bf16-d64"):
        # 260-row partitions: two row groups and a 4-row tail each, 17 workgroups per head
        cfg = _cfg("split-d64", 95, steps=3 if parts == 2 else 4)
    elif case == "bf16-d128":
        cfg = _cfg("split-d128", 96, heads=2, head_dim=128, grid_h=24, grid_w=24,
                   num_partitions=6)
    else:
        cfg = _cfg("split-bf16-out", 97, heads=2, grid_h=16, grid_w=32, num_partitions=4)
    monkeypatch.setenv("DITA_SPLITS_PER_XCD", "0")
    plain = _required(dita, cfg)
    monkeypatch.setenv("DITA_SPLITS_PER_XCD", "2")
    split = _required(dita, cfg)
    # 2 row groups split on each of the 8 XCD ranges: 16 sets of partial merges, and the
    # work lists of the 4 plan slots longer by 2 words per added workgroup and per split
    # group (each slot rounded up to 256 bytes)
    want = _split_bytes(cfg, 16, parts)
    plan_words = 2 * 16 * (parts - 1) + 2 * 16
    slack = 4 * (-(-plan_words * 4 // 256) + 1) * 256
    assert want <= split - plain <= want + slack, (split, plain)
    log(f"case {cfg.name}: 16 row groups split in {parts}, workspace {split - plain} bytes")
    if case == "bf16-out":
        _bf16_out_against_f32(dita, monkeypatch, cfg)
        return
    run_and_check(dita, cfg, heads=[(0, 0), (0, cfg.heads - 1)], recomputes=0)


def _bf16_out_against_f32(dita, monkeypatch, cfg):
    """bf16 output of a split run: the f32 output of the same run rounded to nearest even."""
    from test_gpu_parity import active_for
    dev, _ = gh.device_inputs(cfg, cfg.steps)
    res = {}
    for od in ("f32", "bf16"):
        c = dita.Cache(dita.geometry_from(cfg, out_dtype=od), active_mask=active_for(cfg))
        outs = []
        for s in range(cfg.steps):
            c.set_policy(dita.policy_from(cfg.policy(s + 1)))
            out, _ = c.step(*dev[s])
            outs.append(out.float().cpu().numpy())
        res[od] = outs
        c.free()
    for s in range(cfg.steps):
        want = torch.from_numpy(res["f32"][s]).to(torch.bfloat16).float().numpy()
        assert np.array_equal(res["bf16"][s], want), f"step {s + 1}"


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_split_run_agrees_with_the_unsplit_run(dita, monkeypatch, cache):
    """The same steps with and without splits: the same block counts, outputs and lse equal
    up to the rounding of the sums' association (the cached states, fp8 included, are the
    same in both), and the allocation-free step with splits bit for bit equal to the step
    with splits."""
    from test_gpu_parity import active_for
    cfg = _cfg("split-vs-plain-" + cache, 98, steps=4, cache_dtype=cache,
               head_dim=64 if cache == "bf16" else 128)
    dev, _ = gh.device_inputs(cfg, cfg.steps)

    def run(k, static=False):
        monkeypatch.setenv("DITA_SPLITS_PER_XCD", str(k))
        c = dita.Cache(dita.geometry_from(cfg), active_mask=active_for(cfg))
        res = []
        for s in range(cfg.steps):
            c.set_policy(dita.policy_from(cfg.policy(s + 1)))
            out, lse = c.step(*dev[s], static_scratch=static)
            res.append((out.cpu().numpy(), lse.cpu().numpy()))
        st = c.stats()
        c.free()
        return res, st

    plain, st_p = run(0)
    split, st_s = run(2)
    stat, st_t = run(2, static=True)
    for key in ("device_fresh_blocks", "device_reuse_blocks", "host_fresh_blocks"):
        assert st_s[key] == st_p[key] == st_t[key], key
    worst = 0.0
    for s in range(cfg.steps):
        d = np.abs(split[s][0] - plain[s][0])
        scale = np.maximum(np.abs(plain[s][0]), 1.0)
        worst = max(worst, float(np.max(d / scale)))
        assert np.max(np.abs(split[s][1] - plain[s][1])) < 1e-5
        assert np.array_equal(stat[s][0], split[s][0]), f"static step {s + 1}: out"
        assert np.array_equal(stat[s][1], split[s][1]), f"static step {s + 1}: lse"
    log(f"split vs unsplit: worst relative difference {worst:.2e}")
    assert worst < 1e-5


def test_rejected_reference_with_splits(dita, monkeypatch):
    """A key partition's K scaled by 4 on step 2 and restored on step 3: the fixed-reference
    pass rejects, the second pass recomputes every workgroup, split halves included, and
    merge_splits runs again after it."""
    from oracle.policy import partition_offsets
    from test_gpu_parity import run_and_check
    monkeypatch.setenv("DITA_SPLITS_PER_XCD", "2")
    cfg = _cfg("split-ref-jump", 99, heads=2,
               schedule=wcfg.AnchorThen(Policy(kind=wcfg.FRESH_BUDGET, reuse_percent=0)))
    offs = partition_offsets(cfg.tokens, cfg.num_partitions)
    j0, j1 = offs[3], offs[4]

    def modify(dev, kept):
        dev[1][1][:, :, j0:j1, :] *= 4                 # exact in bf16
        for bh in kept:
            kept[bh][1][1][j0:j1] *= 4
    run_and_check(dita, cfg, heads=[(0, 0), (0, 1)], modify=modify, recomputes="some")


def _split_sweep_case(seed, sub):
    """A random workload meant to hold split row groups: 2-3 heads, 2-4 frames of a 16-24 x
    20-30 grid, 2-8 partitions (a few row groups each, ragged tails), head dim 64, 72, 96 or
    128, 2-4 steps and a random policy kind; with K in 1-3 split groups per XCD range and 2-4
    parts."""
    rng = np.random.default_rng(7000 + 100 * seed + sub)
    T, gh_, gw = int(rng.integers(2, 5)), int(rng.integers(16, 25)), int(rng.integers(20, 31))
    P = int(rng.integers(2, 9))
    D = int(rng.choice([64, 72, 96, 128]))
    H, S = int(rng.integers(2, 4)), int(rng.integers(2, 5))
    N = T * gh_ * gw
    kind = int(rng.integers(0, 3))
    if kind == 0:
        pol = Policy(kind=wcfg.FRESH_BUDGET, reuse_percent=int(rng.integers(0, 101)))
    elif kind == 1:
        pol = Policy(kind=wcfg.FRAME_THRESHOLD, max_fresh_frame_dist=int(rng.integers(0, 3)))
    else:
        pol = Policy(kind=wcfg.CENTROID_THRESHOLD, max_fresh_centroid2=int(rng.integers(0, 2 * N)))
    cfg = custom_config(name=f"split-sweep-{seed}", idx=300 + seed, heads=H, head_dim=D,
                        frames=T, grid_h=gh_, grid_w=gw, num_partitions=P, steps=S,
                        qkv_dtype="bf16", cache_dtype="bf16", schedule=wcfg.AnchorThen(pol))
    return cfg, int(rng.integers(1, 4)), int(rng.integers(2, 5))


@pytest.mark.parametrize("seed", list(range(16)))
def test_split_sweep(dita, monkeypatch, seed):
    """Random workloads with forced splits, every element of every head and step against
    the oracle; odd seeds hand Q, K, V and out over as [B, N, H, D].  A drawn workload whose
    XCD ranges cannot all give K row groups (the library then splits none) is redrawn."""
    from test_gpu_parity import active_for, run_and_check

    def required(cfg, k, parts):
        monkeypatch.setenv("DITA_SPLITS_PER_XCD", str(k))
        monkeypatch.setenv("DITA_SPLIT_PARTS", str(parts))
        return dita.dita_cache_required_bytes(dita.geometry_from(cfg), active_for(cfg))

    for sub in range(20):
        cfg, k, parts = _split_sweep_case(seed, sub)
        if required(cfg, k, parts) - required(cfg, 0, parts) >= _split_bytes(cfg, 8 * k, parts):
            break
    else:
        pytest.fail("no drawn workload splits")
    required(cfg, k, parts)                        # leaves the variables set for the run
    log(f"case {cfg.name} (draw {sub}): {8 * k} row groups split in {parts}")
    run_and_check(dita, cfg, heads=[(0, h) for h in range(cfg.heads)],
                  layout="bnhd" if seed % 2 else "bhnd")
