"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package only draws random numbers and lays out coordinates; it holds
none of the attention or clustering arithmetic, so both the HIP path and the
oracle can consume its arrays without sharing any of the method's code.
"""

from .configs import CONFIGS, WorkloadConfig, get_config  # noqa: F401
from .synth import (  # noqa: F401
    make_case,
    make_coords,
    perlin_visible_cells,
    stress_duplicate_slots,
    stress_copy_rows,
    to_dtype,
)
from .sampler import SAMPLER_CONFIGS, SamplerConfig, make_sampler_case  # noqa: F401
from .merge import MERGE_CONFIGS, MergeConfig, make_merge_case  # noqa: F401
from .ragged import RAGGED_CONFIGS, RaggedConfig, make_varlen_case  # noqa: F401
from .volume import VOLUME_CONFIGS, VolumeConfig, make_volume_case  # noqa: F401
