"""Seeded synthetic inputs for paged E5M2 decode attention.

This package only makes inputs: it draws query vectors and K/V values, rounds
K/V to FP8 E5M2 bytes, assigns physical pages through a block table and fills
everything unreferenced with a poison code. It holds none of the attention
arithmetic and imports neither the oracle nor the HIP library, so both sides
of a parity test can consume the same inputs.
"""

from .quantize import quantize_e5m2, E5M2_MAX_FINITE, POISON_CODE
from .configs import Workload, make_config, make_custom, CONFIG_NAMES
from .select import make_selection

__all__ = [
    "quantize_e5m2",
    "E5M2_MAX_FINITE",
    "POISON_CODE",
    "Workload",
    "make_config",
    "make_custom",
    "CONFIG_NAMES",
    "make_selection",
]
