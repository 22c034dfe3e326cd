"""The allocation-free step, dita_attn_step_static, through the C ABI on the GPU.

It must give exactly what dita_attn_step gives on the same inputs (the two share their
kernels; only where the per-step scratch lives differs), and so meet the fp64 oracle's bars.
The cases run back to back through the one static scratch array of the GPU, each smaller
than the one before (bf16 D = 64 over many rows, bf16 D = 72, then the small fp32
workload), so that every call finds the previous, larger call's contents in the array."""
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


def _cases():
    budget = wcfg.AnchorThen(Policy(kind=wcfg.FRESH_BUDGET, reuse_percent=60))
    return [
        custom_config(name="static-bf16-d64", idx=91, heads=3, head_dim=64, frames=2, grid_h=45,
                      grid_w=40, num_partitions=6, steps=3, qkv_dtype="bf16",
                      cache_dtype="bf16", schedule=budget),
        custom_config(name="static-bf16-d72", idx=92, heads=2, head_dim=72, frames=1, grid_h=16,
                      grid_w=20, num_partitions=3, steps=2, qkv_dtype="bf16",
                      cache_dtype="bf16", schedule=budget),
        CONFIGS[1],
    ]


def _run(dita, cfg, dev, static):
    import oracle
    g = dita.geometry_from(cfg)
    offs = oracle.partition_offsets(cfg.tokens, cfg.num_partitions)
    from oracle.policy import active_mask
    act = active_mask(offs, cfg.frame_tokens, cfg.policy(1).tile_sparse).astype(np.uint8)
    cache = dita.Cache(g, active_mask=act)
    res = []
    for s in range(cfg.steps):
        cache.set_policy(dita.policy_from(cfg.policy(s + 1)))
        out, lse = cache.step(*dev[s], static_scratch=static)
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    st = cache.stats()
    cache.free()
    return res, st


def test_static_step_equals_the_step_on_back_to_back_shrinking_calls(dita):
    import oracle
    cases = _cases()
    sizes = [c.batch * c.heads * c.tokens * c.head_dim for c in cases]
    assert sizes == sorted(sizes, reverse=True)
    for cfg in cases:
        bf = cfg.qkv_dtype == "bf16"
        log(f"case {cfg.name}: B={cfg.batch} H={cfg.heads} N={cfg.tokens} D={cfg.head_dim} "
            f"P={cfg.num_partitions} steps={cfg.steps} {cfg.qkv_dtype}")
        dev, kept = gh.device_inputs(cfg, cfg.steps, keep_heads={(0, 0)})
        ref, st_ref = _run(dita, cfg, dev, static=False)
        got, st_got = _run(dita, cfg, dev, static=True)
        for s in range(cfg.steps):
            assert np.array_equal(got[s][0], ref[s][0]), f"{cfg.name} step {s + 1}: out"
            assert np.array_equal(got[s][1], ref[s][1]), f"{cfg.name} step {s + 1}: lse"
        for key in ("device_fresh_blocks", "device_reuse_blocks", "host_fresh_blocks",
                    "host_reuse_blocks", "device_v_range_errors", "steps_done"):
            assert st_got[key] == st_ref[key], key
        assert st_got["device_fresh_blocks"] == st_got["host_fresh_blocks"]
        assert st_got["profiled_steps"] == 0
        # and both against the fp64 oracle, on head (0, 0)
        want = oracle.run_head(cfg, 0, 0, steps=cfg.steps, inputs=kept[(0, 0)],
                               cache_mode="fp64")
        for s in range(cfg.steps):
            ok, _, _ = compare(got[s][0][0, 0], want[s].out, bf,
                               f"  {cfg.name} step {s + 1} static out")
            assert ok
            lerr = float(np.max(np.abs(got[s][1][0, 0] - want[s].lse)))
            assert lerr < (2e-3 if bf else 1e-5), lerr
        log(f"case {cfg.name}: static step bit-identical to dita_attn_step over "
            f"{cfg.steps} steps")
