"""Synthetic workloads (shapes, schedules) and the seeded input generator.

This package is shared by the oracle's tests, the GPU tests and the bench.  It draws
inputs only; it contains no attention arithmetic and no mask construction."""
from .configs import (CONFIGS, Config, Policy, EXPLICIT, FRAME_THRESHOLD, FRESH_BUDGET,
                      CENTROID_THRESHOLD, PLANNER, partition_offsets, custom_config)
from .gen import HeadStream, head_steps, all_steps, position_term

__all__ = ["CONFIGS", "Config", "Policy", "EXPLICIT", "FRAME_THRESHOLD", "FRESH_BUDGET",
           "CENTROID_THRESHOLD", "PLANNER", "partition_offsets", "custom_config", "HeadStream",
           "head_steps", "all_steps", "position_term"]
