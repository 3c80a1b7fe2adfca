"""Seeded synthetic inputs for the DFlash draft step.

This package holds the workload descriptions (model dimensions, batch and
context shapes) and the seeded generators that draw weights, target-layer
features, token ids and planted target ids.  It contains none of the method's
arithmetic: both the CPU oracle (``oracle/``) and the HIP library
(``block_diffusion_drafter_layers_amd``) consume what it produces, and neither
is imported here.
"""

from .configs import CONFIGS, DrafterDims, Workload, get_workload  # noqa: F401
from .inputs import (  # noqa: F401
    SEED,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    geometric_prefix_lengths,
    make_rng,
    planted_targets,
    target_layer_ids,
    DrafterInputs,
)
