"""GPU: compaction of merged groups (DiTango, "State-Centric Parallel Runtime / Composizione
Dinamica dei Gruppi": merging stored states into coarser groups relieves memory pressure),
through the C ABI.

A run that merges cached states and compacts the cache onto one slot per stored state must
continue exactly as the same run without compaction: outputs, lse and device counts bit for
bit, at every step, through a second merge and compaction.  After an expansion back to the
full slot table, the anchor step that recomputes the merged groups matches the uncompacted
run up to rounding: the compacted members' own states are gone, so their cached lse no longer
serves as the softmax reference and the step keeps the running maximum, where the uncompacted
run (whose member slots still hold their own states) takes the fixed-reference pass.  The
bytes the cache needs fall by g - 1 slots per merged group of g (the group factor on the
merged states).  Both runs are held to the fp64 oracle with the merge bars of the
group-composition tests."""
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
    # name, frames, gh, gw, P, D, heads, steps, dtype, merges {after step: [group sizes]}
    ("compact-bf16-d64", 8, 5, 7, 8, 64, 2, 6, "bf16", {1: [2], 2: [4]}),
    ("compact-fp8-d128", 8, 4, 6, 8, 128, 1, 5, "bf16/fp8", {1: [2, 4]}),
    ("compact-f32", 8, 2, 4, 8, 64, 2, 5, "f32", {1: [2], 3: [8]}),
    ("compact-bf16-64-partitions", 4, 16, 16, 64, 64, 1, 5, "bf16", {1: [4], 2: [16]}),
]


def _always_reused(masks, P, g):
    NG = (P + g - 1) // g
    sel = np.ones((P, NG), np.uint8)
    for M in masks:
        for i in range(P):
            for J in range(NG):
                if any(M[i, j] != 2 for j in range(J * g, min(P, J * g + g))):
                    sel[i, J] = 0
    return sel


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_compaction_continues_bit_identically(dita, case):
    import oracle
    from oracle.policy import active_mask, partition_offsets
    name, T, gh_, gw, P, D, H, S, dt, merges = case
    dt, cdt = dt.split("/") if "/" in dt else (dt, dt)
    sched = wcfg.AnchorThen(Policy(kind=wcfg.FRAME_THRESHOLD, max_fresh_frame_dist=1))
    cfg = custom_config(name=name, idx=86, heads=H, head_dim=D, frames=T, grid_h=gh_,
                        grid_w=gw, num_partitions=P, steps=S, qkv_dtype=dt, cache_dtype=cdt,
                        schedule=sched)
    heads = [(0, h) for h in range(H)]
    offs = partition_offsets(cfg.tokens, P)
    act = active_mask(offs, cfg.frame_tokens, False).astype(np.uint8)
    log(f"case {name}: N={cfg.tokens} P={P} D={D} H={H} steps={S} {dt}/{cdt} merges={merges}")
    dev, kept = gh.device_inputs(cfg, S, keep_heads=set(heads))
    g = dita.geometry_from(cfg)
    # steps 1 .. S-1 follow the schedule; step S is an anchor (after the expansion)
    pols = [dita.policy_from(cfg.policy(s)) for s in range(1, S)]
    pols.append(dita.policy_from(cfg.policy(1).as_anchor()))
    later = [dita.dita_policy_mask(g, pols[s], np.ones((P, P), np.uint8)) for s in range(1, S - 1)]
    sels = {gs: _always_reused([M for k, M in enumerate(later) if k + 1 >= t], P, gs)
            for t, lst in merges.items() for gs in lst}
    per_slot = cfg.batch * H * (-(-max(np.diff(offs)) // 64) * 64) * (
        4 + {"bf16": 2, "fp8": 1, "f32": 4}[cdt] * (64 if D <= 64 else (96 if D <= 96 else 128)))

    runs = {}
    for compact in (False, True):
        c = dita.Cache(g, active_mask=act)
        full = c.required_bytes
        outs, lses, merged_total = [], [], 0
        for s in range(S):
            if compact and s == S - 1:
                c.expand()
                c.release_old_buffer()
                assert c.buffer.numel() == full
            c.set_policy(pols[s])
            out, lse = c.step(*dev[s])
            outs.append(out.cpu().numpy())
            lses.append(lse.cpu().numpy())
            for gs in merges.get(s + 1, []):
                n = c.merge_groups(gs, select=sels[gs])
                merged_total += n
                log(f"  after step {s + 1}: {n} groups of {gs} merged")
                if compact:
                    before = c.buffer.numel()
                    need = c.compact_bytes()
                    c.compact()
                    c.release_old_buffer()
                    log(f"  compacted: {before} -> {need} bytes "
                        f"(full table {full}, {(full - need) // per_slot} slots freed)")
            if compact and merged_total:
                assert c.buffer.numel() <= full
        st = c.stats()
        runs[compact] = (outs, lses, st)
        c.free()
    ref, got = runs[False], runs[True]
    for s in range(S - 1):
        assert np.array_equal(got[0][s], ref[0][s]), f"step {s + 1}: out differs"
        assert np.array_equal(got[1][s], ref[1][s]), f"step {s + 1}: lse differs"
    # after the expansion: the same attention state, rounded differently on the bf16 path
    # (fixed reference against running maximum: a few bf16 roundings of the P values); the
    # f32 path keeps the running maximum either way
    d_out = float(np.max(np.abs(got[0][S - 1] - ref[0][S - 1])))
    d_lse = float(np.max(np.abs(got[1][S - 1] - ref[1][S - 1])))
    log(f"  anchor after the expansion: out differs by {d_out:.2e}, lse by {d_lse:.2e}")
    assert d_out <= (4e-3 if dt == "bf16" else 1e-5), d_out
    assert d_lse <= (1e-3 if dt == "bf16" else 1e-5), d_lse
    for key in ("device_fresh_blocks", "device_reuse_blocks", "host_fresh_blocks",
                "host_reuse_blocks"):
        assert got[2][key] == ref[2][key], key
    assert got[2]["device_fresh_blocks"] == got[2]["host_fresh_blocks"]
    assert got[2]["device_reuse_blocks"] == got[2]["host_reuse_blocks"]

    # the uncompacted run against the fp64 oracle with the same merges (as the group tests)
    from test_gpu_groups import merge_rounding_bar
    omerges = {t: [(gs, sels[gs].astype(bool)) for gs in lst] for t, lst in merges.items()}
    bf = dt == "bf16"
    ok = True
    for (b, h) in heads:
        r64 = oracle.run_head(cfg, b, h, steps=S, inputs=kept[(b, h)], cache_mode="fp64",
                              policies=[cfg.policy(s) for s in range(1, S)]
                              + [cfg.policy(1).as_anchor()],
                              merges=omerges, keep_block_lse=True)
        for s in range(S):
            if cdt == "fp8":
                break                          # the fp8 cache's own bars: test_gpu_fp8
            extra = merge_rounding_bar(r64[s], offs, P, omerges, kept[(b, h)], s, bf)
            bar = (BF16_MAX_ABS if bf else F32_MAX_ABS) + extra
            for name, run in (("uncompacted", ref), ("compacted", got)):
                if name == "compacted" and s < S - 1:
                    continue                   # bit-identical to the uncompacted run
                err = np.abs(run[0][s][b, h].astype(np.float64) - r64[s].out)
                good = bool(np.all(err <= bar)) and (not bf or float(err.mean()) <= BF16_MEAN_ABS)
                ok &= good
                log(f"  oracle b={b} h={h} step {s + 1} ({name}): max-abs {err.max():.3e} "
                    f"{'ok' if good else 'FAIL'}")
    assert ok


def test_compaction_bytes_and_rules(dita):
    """The compacted table frees exactly g - 1 slots per merged group of g; a compacted group
    cannot be recomputed (POLICY) until the cache is expanded; a reset keeps the groups."""
    from oracle.policy import active_mask, partition_offsets
    sched = wcfg.AnchorThen(Policy(kind=wcfg.FRAME_THRESHOLD, max_fresh_frame_dist=1))
    cfg = custom_config(name="compact-rules", idx=87, heads=2, head_dim=64, frames=8, grid_h=4,
                        grid_w=8, num_partitions=8, steps=3, qkv_dtype="bf16",
                        cache_dtype="bf16", schedule=sched)
    P = cfg.num_partitions
    offs = partition_offsets(cfg.tokens, P)
    act = active_mask(offs, cfg.frame_tokens, False).astype(np.uint8)
    dev, _ = gh.device_inputs(cfg, 3)
    c = dita.Cache(dita.geometry_from(cfg), active_mask=act)
    full = c.required_bytes
    assert c.compact_bytes() == full
    c.set_policy(dita.policy_from(cfg.policy(1)))
    c.step(*dev[0])
    g = dita.geometry_from(cfg)
    step2 = dita.dita_policy_mask(g, dita.policy_from(cfg.policy(2)), np.ones((P, P), np.uint8))
    n = c.merge_groups(2, select=_always_reused([step2], P, 2))   # the pairs step 2 reuses
    assert n > 0
    per_slot = cfg.batch * cfg.heads * 64 * (4 + 64 * 2)
    need = c.compact_bytes()
    assert full - need == n * per_slot, (full, need, n)
    log(f"{n} pairs merged: {full} -> {need} bytes; the merged states' bytes halve")
    c.compact()
    c.release_old_buffer()
    with pytest.raises(dita.DitaError) as e:
        c.set_policy(dita.policy_from(cfg.policy(1).as_anchor()))
    assert e.value.name == "POLICY"
    c.set_policy(dita.policy_from(cfg.policy(2)))  # reuse of every merged group: allowed
    c.step(*dev[1])
    c.reset()
    with pytest.raises(dita.DitaError) as e:
        c.set_policy(dita.policy_from(cfg.policy(1).as_anchor()))
    assert e.value.name == "POLICY"
    c.expand()
    c.release_old_buffer()
    assert c.buffer.numel() == full
    c.set_policy(dita.policy_from(cfg.policy(1).as_anchor()))
    c.step(*dev[2])
    torch.cuda.synchronize()
    with pytest.raises(dita.DitaError) as e:
        c.expand()                                 # not compacted
    assert e.value.name == "INVALID_ARGUMENT"
    c.free()


def test_compaction_with_split_row_groups(dita, monkeypatch):
    """The same continuation with split row groups forced (two per XCD range, in 3 parts):
    the split workspace moves with the rest of the buffer's regions on compaction and
    expansion."""
    monkeypatch.setenv("DITA_SPLITS_PER_XCD", "2")
    monkeypatch.setenv("DITA_SPLIT_PARTS", "3")
    test_compaction_continues_bit_identically(
        dita, ("compact-bf16-splits", 4, 20, 26, 8, 64, 3, 5, "bf16", {1: [2], 2: [4]}))
