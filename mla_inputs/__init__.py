"""Seeded synthetic inputs for the MLA decode step.

This package only draws random numbers and lays them out in memory: the paged
latent-cache pool, the block table, the query and the two up-projection
weights.  It performs none of the attention arithmetic.  Both the HIP library's
tests and the CPU oracle's tests take their inputs from here; neither side
imports the other.
"""
from .configs import CONFIGS, MLAConfig, config_by_name  # noqa: F401
from .generate import MLAInputs, generate, make_inputs  # noqa: F401
