"""Seeded synthetic inputs for the vision-tower forward.

This package only *draws* inputs: tower shapes, image/video sizes, uint8
pixels and random weights.  It holds none of the tower's arithmetic, so both
the CPU oracle (``oracle/``) and the HIP library's tests and bench may import
it without sharing any computation.
"""

from .configs import (  # noqa: F401
    TowerConfig,
    Item,
    Workload,
    CONFIG_IDS,
    tower_config,
    draw_items,
    make_workload,
    make_custom_workload,
    weight_specs,
    make_weights,
    pack_pixels,
    bf16_representable,
)
