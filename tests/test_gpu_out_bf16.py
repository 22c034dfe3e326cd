"""GPU: the bf16 output (geometry out_dtype = BF16), through the C ABI.

The kernel forms the same f32 result as with an f32 output and rounds it to bf16 (nearest
even), so every element must equal torch's round-to-nearest-even of the f32 output of an
identical run, bit for bit; against the fp64 oracle it must meet the f32 output's bars widened
by that rounding (gpu_helpers.bf16_out_bars)."""
import numpy as np
import pytest

import gpu_helpers as gh
from gpu_helpers import log
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


BUDGET = wcfg.AnchorThen(Policy(kind=wcfg.FRESH_BUDGET, reuse_percent=60))
CASES = [
    # name, frames, gh, gw, P, D, heads, steps, layout
    ("out-bf16-d64", 3, 10, 13, 5, 64, 2, 3, "bhnd"),
    ("out-bf16-d72", 2, 9, 11, 3, 72, 2, 3, "bhnd"),
    ("out-bf16-d128", 2, 15, 20, 7, 128, 2, 3, "bhnd"),
    ("out-bf16-d64-token-major", 2, 45, 20, 6, 64, 3, 3, "bnhd"),
]


def run_pair(dita, cfg, heads, rows=None, layout="bhnd"):
    """The schedule with an f32 and a bf16 output on identical inputs; per step the bf16
    output must be the f32 one rounded to bf16.  Returns the bf16 outputs of `heads`
    (at `rows`) and the host inputs."""
    from oracle.policy import active_mask, partition_offsets
    S = cfg.steps
    dev, kept = gh.device_inputs(cfg, S, keep_heads=set(heads))
    if layout == "bnhd":
        dev = [[t.transpose(1, 2).contiguous() for t in st] for st in dev]
    offs = partition_offsets(cfg.tokens, cfg.num_partitions)
    act = active_mask(offs, cfg.frame_tokens, cfg.policy(1).tile_sparse).astype(np.uint8)
    caches = {dt: dita.Cache(dita.geometry_from(cfg, out_dtype=dt, layout=layout),
                             active_mask=act) for dt in ("f32", "bf16")}
    got = []
    sel = torch.as_tensor(rows, device="cuda") if rows is not None else None
    for s in range(S):
        res = {}
        for dt, c in caches.items():
            c.set_policy(dita.policy_from(cfg.policy(s + 1)))
            out, lse = c.step(*dev[s])
            res[dt] = (out, lse)
        o32, o16 = res["f32"][0], res["bf16"][0]
        assert o16.dtype == torch.bfloat16
        assert torch.equal(o16, o32.to(torch.bfloat16)), f"step {s + 1}: bf16 != rne(f32)"
        assert torch.equal(res["bf16"][1], res["f32"][1]), f"step {s + 1}: lse differs"
        if layout == "bnhd":
            o16 = o16.transpose(1, 2)
        per = {}
        for (b, h) in heads:
            o = o16[b, h] if sel is None else o16[b, h].index_select(0, sel)
            per[(b, h)] = o.float().cpu().numpy()
        got.append(per)
    for c in caches.values():
        c.free()
    return got, kept


def check_against_oracle(cfg, heads, got, kept, rows=None):
    import oracle
    ok = True
    for (b, h) in heads:
        ref = oracle.run_head(cfg, b, h, steps=cfg.steps, rows=rows, inputs=kept[(b, h)],
                              cache_mode="fp64")
        for s in range(cfg.steps):
            o, want = got[s][(b, h)], ref[s].out
            err = np.abs(o.astype(np.float64) - want)
            elem_bar, mean_bar = gh.bf16_out_bars(want)
            good = bool(np.all(err <= elem_bar)) and float(err.mean()) <= mean_bar
            log(f"  {cfg.name} b={b} h={h} step {s + 1}: max-abs {err.max():.3e} "
                f"(bar {elem_bar.max():.3e}) mean-abs {err.mean():.3e} (bar {mean_bar:.3e}) "
                f"{'ok' if good else 'FAIL'}")
            ok &= good
    assert ok


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bf16_output(dita, case):
    name, T, gh_, gw, P, D, H, S, layout = case
    cfg = custom_config(name=name, idx=93, heads=H, head_dim=D, frames=T, grid_h=gh_,
                        grid_w=gw, num_partitions=P, steps=S, qkv_dtype="bf16",
                        cache_dtype="bf16", schedule=BUDGET)
    heads = [(0, h) for h in range(H)]
    got, kept = run_pair(dita, cfg, heads, layout=layout)
    check_against_oracle(cfg, heads, got, kept)


def test_bf16_output_full_video29f_720p(dita):
    """The 29-frame 720p workload at full size: every step bit-equal to the rounded f32
    output over all heads and rows; sampled rows of two heads against the oracle."""
    from oracle.policy import partition_offsets
    cfg = CONFIGS[3]
    rows = gh.sample_rows(partition_offsets(cfg.tokens, cfg.num_partitions), 6,
                          np.random.default_rng(31))
    heads = [(0, 2), (0, 21)]
    got, kept = run_pair(dita, cfg, heads, rows=rows)
    check_against_oracle(cfg, heads, got, kept, rows=rows)

