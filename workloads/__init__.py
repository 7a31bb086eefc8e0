"""Seeded synthetic inputs for paged-attention decode.

This package is the only code shared by the CPU oracle and the GPU path. It
draws random numbers, builds block tables, context lengths and slot mappings,
and holds none of the attention arithmetic. Caches are returned as flat arrays
of i.i.d. values; each consumer applies its own view of the physical layout.
"""

from .configs import CONFIGS, CONFIG_ORDER, EXTRA_CONFIGS, Config, get_config  # noqa: F401
from .gen import Inputs, make_inputs, nan_of, poison_blocks, to_storage  # noqa: F401
