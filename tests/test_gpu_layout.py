"""GPU tests of the token-major layout: Q, K, V and out given as [B, N, H, D] (layout BNHD)
instead of [B, H, N, D].  The same logical inputs in both layouts must give bit-identical
outputs and lse (the kernels do the same arithmetic on other addresses), and the BNHD run is
held to the fp64 oracle's bars like every other run."""
import numpy as np
import pytest

import gpu_helpers as gh
from gpu_helpers import compare, log
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
    # name, batch, frames, gh, gw, P, D, heads, steps, dtype
    ("layout-bf16-d64-tails", 2, 4, 10, 26, 8, 64, 3, 3, "bf16"),    # 130-row partitions
    ("layout-bf16-d72", 1, 3, 8, 10, 5, 72, 2, 3, "bf16"),
    ("layout-bf16-d128", 1, 3, 8, 10, 6, 128, 2, 3, "bf16"),
    ("layout-f32-d64", 2, 4, 4, 6, 4, 64, 3, 2, "f32"),
    ("layout-bf16-d64-16heads", 1, 4, 10, 26, 8, 64, 16, 2, "bf16"),  # token stride 1024
]


def _run(dita, cfg, act, steps_qkv, layout):
    g = dita.geometry_from(cfg)
    g.layout = dita.LAYOUT_BNHD if layout == "bnhd" else dita.LAYOUT_BHND
    cache = dita.Cache(g, active_mask=act.astype(np.uint8))
    outs, lses = [], []
    for s in range(cfg.steps):
        cache.set_policy(dita.policy_from(cfg.policy(s + 1)))
        q, k, v = steps_qkv[s]
        if layout == "bnhd":
            q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
        out, lse = cache.step(q, k, v)
        if layout == "bnhd":
            out = out.transpose(1, 2).contiguous()
        outs.append(out)
        lses.append(lse.clone())
    torch.cuda.synchronize()
    cache.free()
    return outs, lses


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bnhd_layout_matches_bhnd(dita, case):
    import oracle
    from oracle.policy import active_mask, partition_offsets
    name, B, T, gh_, gw, P, D, H, S, dt = case
    sched = wcfg.AnchorThen(Policy(kind=wcfg.FRAME_THRESHOLD, max_fresh_frame_dist=1))
    cfg = custom_config(name=name, idx=87, batch=B, heads=H, head_dim=D, frames=T, grid_h=gh_,
                        grid_w=gw, num_partitions=P, steps=S, qkv_dtype=dt, cache_dtype=dt,
                        schedule=sched)
    offs = partition_offsets(cfg.tokens, P)
    act = active_mask(offs, cfg.frame_tokens, False)
    heads = [(b, h) for b in range(B) for h in range(H)]
    log(f"case {name}: B={B} H={H} N={cfg.tokens} P={P} D={D} steps={S} {dt}")
    dev, kept = gh.device_inputs(cfg, S, keep_heads=set(heads))
    o1, l1 = _run(dita, cfg, act, dev, "bhnd")
    o2, l2 = _run(dita, cfg, act, dev, "bnhd")
    for s in range(S):
        assert torch.equal(o1[s], o2[s]), f"step {s + 1}: out differs between layouts"
        assert torch.equal(l1[s], l2[s]), f"step {s + 1}: lse differs between layouts"
    bf = dt == "bf16"
    ok = True
    for (b, h) in heads:
        ref = oracle.run_head(cfg, b, h, cache_mode="fp64", active=act, inputs=kept[(b, h)])
        for s in range(S):
            good, *_ = compare(o2[s][b, h].cpu().numpy(), ref[s].out, bf,
                               f"bnhd step {s + 1} head ({b},{h}) out")
            ok &= good
            ok &= float(np.abs(l2[s][b, h].cpu().numpy() - ref[s].lse).max()) < \
                (2e-3 if bf else 1e-5)
    assert ok
