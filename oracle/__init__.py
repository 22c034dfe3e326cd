"""fp64 CPU oracle for partitioned attention with selective attention-state reuse.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline leg
may import this package.  The native library never calls it, and it shares no code with the
native path: it builds its own partition map, block policy and work lists from the
definitions, computes every block state with numpy in float64, and merges them by
log-sum-exp.  Only the seeded input generator (package `workloads`) is common to both.

What it follows (DiTango, gist.science 2607.15650):
  * "State-Centric Parallel Runtime / Composizione dello Stato": the unit that is cached and
    combined is an attention state made of an output and its log-sum-exp, and states
    combine associatively and commutatively;
  * "Anchor-Guided Selection Planner": per step each partition is either computed fresh or
    reuses a state from an earlier step; anchor steps compute everything; the local
    partition is always computed;
  * Efficient-vDiT (chatpaper abstract): tile-style sparse 3D attention, linear in frames,
    read as a block-selection policy.

Pins (tests/test_oracle_pins.py): dense softmax attention from torch's SDPA (all-fresh),
masked SDPA (tile mask), brute-force scalar loops over the closed "mixed-time" form,
split/merge-order invariance, reuse-with-no-drift no-op, merge weights summing to one,
closed-form mask counts and printed masks (tests/golden/), linear-in-frames active count,
head-permutation equivariance and the CFG constant-shift identity.  Planner
(tests/test_planner_oracle.py): importance against a dense-softmax brute force and the
uniform-attention closed form, rows summing to one, growth zero without drift and equal to a
planted constant shift, the group decision against an exhaustive search on small cases and a
hand-worked example, and the planner reducing to the all-fresh run when every step is an
anchor.
"""
from .policy import (partition_offsets, centroids2, partition_frames, active_mask,
                     policy_mask, work_lists, PolicyError, SKIP, FRESH, REUSE)
from .attention import (block_state, merge_states, round_bf16, round_f32, round_fp8_e4m3,
                        run_head, OracleStep)
from .planner import (importance, growth, predicted_errors, planner_mask, run_planner,
                      PlannerStep, PLANNER)

__all__ = ["partition_offsets", "centroids2", "partition_frames", "active_mask",
           "policy_mask", "work_lists", "PolicyError", "SKIP", "FRESH", "REUSE",
           "block_state", "merge_states", "round_bf16", "round_f32", "round_fp8_e4m3", "run_head",
           "OracleStep", "importance", "growth", "predicted_errors", "planner_mask",
           "run_planner", "PlannerStep", "PLANNER"]
