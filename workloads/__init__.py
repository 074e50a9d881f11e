"""Seeded synthetic workloads for block-sparse attention prefill.

This module only draws inputs: it holds the workload shapes and the seeded
generators that both the GPU path and the CPU oracle consume, byte for byte.
It contains none of the method's arithmetic (no pooling, scoring, selection or
attention).  Where a structure is "planted" (a needle block, a near-tied pair,
a wide block hiding an outlier key) it is built from plain random draws and the
mean query direction of the generated data.
"""

from .configs import CONFIGS, EXTRA_CONFIGS, WorkloadConfig, config_by_name, scaled  # noqa: F401
from .generate import Inputs, generate  # noqa: F401
