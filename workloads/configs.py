"""The five synthetic workloads of partitioned video-DiT attention with state reuse.

Each workload fixes a token geometry (frames x grid_h x grid_w, flattened frame-major,
row-major inside a frame), a contiguous split into context partitions, the head shape,
the number of denoising steps, the input and cache precision, and a per-step block policy.

The policies are plain parameter records (kind + thresholds); how a policy turns into a
fresh/reuse/skip mask is defined twice, independently: once in the fp64 oracle and once in
the native host library.  Nothing in this module computes attention or a mask.

Sources for the shapes and schedules (the pages give no numbers for them; the shapes below
are readings consistent with them):
  * DiTango (gist.science 2607.15650), "Metodologia / Anchor-Guided Selection Planner":
    partitions are computed fresh or reuse an earlier step's attention state; anchor steps
    recompute everything; the local partition is always computed.
  * Efficient-vDiT (chatpaper abstract): tile-style sparse 3D attention whose cost is linear
    in the number of frames (self + first frame + neighbouring frames).
  * Hybridiff (gist.science 2602.21760), "Metodologia B": warm-up / parallel /
    full-connection phases, used only as the shape of the CFG workload's reuse schedule.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, Optional, Tuple

# Policy kinds (same numbering as the C header's dita_policy_kind).
EXPLICIT = 0
FRAME_THRESHOLD = 1
FRESH_BUDGET = 2
CENTROID_THRESHOLD = 3
PLANNER = 4


@dataclass(frozen=True)
class Policy:
    """Parameters of one step's block policy.

    kind                 EXPLICIT / FRAME_THRESHOLD / FRESH_BUDGET / CENTROID_THRESHOLD
    max_fresh_frame_dist FRAME_THRESHOLD: a block is fresh iff its frame distance <= this
    reuse_percent        FRESH_BUDGET: per row, R = min(floor((pct*A + 50)/100), A - 1)
    max_fresh_centroid2  CENTROID_THRESHOLD: fresh iff |C_i - C_j| <= this (doubled tokens)
    tile_sparse          restrict the active set to {own frame, frame 0, own frame +- 1}
    anchor               every active block is fresh this step
    explicit_mask        EXPLICIT: P*P values in {0 skip, 1 fresh, 2 reuse}, row-major
    group_size           PLANNER: partitions per group (decisions per block group)
    anchor_period        PLANNER: steps between anchors (0: only the first)
    max_error            PLANNER: block groups above this predicted error are fresh (0: off)
    """

    kind: int = FRAME_THRESHOLD
    max_fresh_frame_dist: int = 0
    reuse_percent: int = 0
    max_fresh_centroid2: int = 0
    tile_sparse: bool = False
    anchor: bool = False
    explicit_mask: Optional[Tuple[int, ...]] = None
    group_size: int = 1
    anchor_period: int = 0
    max_error: float = 0.0

    def as_anchor(self) -> "Policy":
        return Policy(kind=self.kind, max_fresh_frame_dist=self.max_fresh_frame_dist,
                      reuse_percent=self.reuse_percent,
                      max_fresh_centroid2=self.max_fresh_centroid2,
                      tile_sparse=self.tile_sparse, anchor=True,
                      explicit_mask=self.explicit_mask, group_size=self.group_size,
                      anchor_period=self.anchor_period, max_error=self.max_error)


@dataclass(frozen=True)
class Config:
    idx: int                    # 1-based workload number; also the first seed word
    name: str
    batch: int
    heads: int
    head_dim: int
    frames: int
    grid_h: int
    grid_w: int
    num_partitions: int
    steps: int
    qkv_dtype: str              # "f32" | "bf16"
    cache_dtype: str            # "f32" | "bf16"   (cache lse is always f32)
    pe_mode: str                # "3d" | "2d"
    pe_scale: float = 2.0
    drift: float = 0.05
    cfg_v_offset: float = 0.0   # b >= 1: V = V[b=0] + offset * eps (eps fixed over steps)
    schedule: Callable[[int], Policy] = field(default=None, compare=False, repr=False)

    @property
    def tokens(self) -> int:
        return self.frames * self.grid_h * self.grid_w

    @property
    def frame_tokens(self) -> int:
        return self.grid_h * self.grid_w

    def policy(self, step: int) -> Policy:
        """Policy for 1-indexed denoising step `step`."""
        if not 1 <= step <= self.steps:
            raise ValueError(f"step {step} outside 1..{self.steps}")
        return self.schedule(step)


@dataclass(frozen=True)
class AnchorThen:
    """Schedule: the first `anchors` steps are anchors (everything fresh), then `policy`."""
    policy: Policy
    anchors: int = 1

    def __call__(self, step: int) -> Policy:
        return self.policy.as_anchor() if step <= self.anchors else self.policy


def _anchor_then(p: Policy, anchors: int = 1) -> AnchorThen:
    return AnchorThen(p, anchors)


def _cfg_schedule(step: int) -> Policy:
    # steps 1-2 anchor (0 % reuse), 3-18 at 70 % reuse, 19-20 at 30 % reuse
    if step <= 2:
        return Policy(kind=FRESH_BUDGET, reuse_percent=0, anchor=True)
    if step <= 18:
        return Policy(kind=FRESH_BUDGET, reuse_percent=70)
    return Policy(kind=FRESH_BUDGET, reuse_percent=30)


CONFIGS: Dict[int, Config] = {
    1: Config(1, "tiny-f32", batch=1, heads=2, head_dim=64, frames=4, grid_h=8, grid_w=8,
              num_partitions=4, steps=2, qkv_dtype="f32", cache_dtype="f32", pe_mode="3d",
              schedule=_anchor_then(Policy(kind=FRAME_THRESHOLD, max_fresh_frame_dist=1))),
    2: Config(2, "image-bf16-d72", batch=1, heads=16, head_dim=72, frames=1, grid_h=64,
              grid_w=64, num_partitions=8, steps=5, qkv_dtype="bf16", cache_dtype="bf16",
              pe_mode="2d",
              # 2 patch rows x 64 patches = 128 tokens = 256 in doubled-centroid units
              schedule=_anchor_then(Policy(kind=CENTROID_THRESHOLD, max_fresh_centroid2=256))),
    3: Config(3, "video29f-720p-bf16", batch=1, heads=24, head_dim=64, frames=8, grid_h=45,
              grid_w=80, num_partitions=32, steps=10, qkv_dtype="bf16", cache_dtype="bf16",
              pe_mode="3d",
              schedule=_anchor_then(Policy(kind=FRESH_BUDGET, reuse_percent=60))),
    4: Config(4, "video93f-tile-sparse-bf16", batch=1, heads=24, head_dim=64, frames=24,
              grid_h=45, grid_w=80, num_partitions=24, steps=8, qkv_dtype="bf16",
              cache_dtype="bf16", pe_mode="3d",
              schedule=_anchor_then(Policy(kind=FRAME_THRESHOLD, max_fresh_frame_dist=1,
                                           tile_sparse=True))),
    5: Config(5, "cfg-long-video-bf16-d128", batch=2, heads=40, head_dim=128, frames=17,
              grid_h=30, grid_w=52, num_partitions=16, steps=20, qkv_dtype="bf16",
              cache_dtype="bf16", pe_mode="3d", cfg_v_offset=0.1, schedule=_cfg_schedule),
}


def partition_offsets(tokens: int, parts: int):
    """Contiguous split of `tokens` into `parts` ranges; the first tokens % parts ranges get
    one extra token (the numpy array_split rule).  Returns a list of parts + 1 offsets."""
    if parts <= 0 or parts > tokens:
        raise ValueError("need 1 <= parts <= tokens")
    base, extra = divmod(tokens, parts)
    offs = [0]
    for p in range(parts):
        offs.append(offs[-1] + base + (1 if p < extra else 0))
    return offs


def custom_config(**kw) -> Config:
    """A small ad-hoc workload (tests); unspecified fields take tiny defaults."""
    d = dict(idx=99, name="custom", batch=1, heads=1, head_dim=16, frames=2, grid_h=4,
             grid_w=4, num_partitions=4, steps=2, qkv_dtype="f32", cache_dtype="f32",
             pe_mode="3d", schedule=_anchor_then(Policy(kind=FRAME_THRESHOLD,
                                                        max_fresh_frame_dist=0)))
    d.update(kw)
    return Config(**d)
