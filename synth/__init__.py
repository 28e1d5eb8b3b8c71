"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks.

This package draws random inputs (weights, activations, KV caches, token trees,
logits, Gumbel noise) and describes the five workload shapes. It holds none of
the method's arithmetic: no quantization, no attention, no acceptance logic.
Both the HIP path and the oracle receive the same bytes from here.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from . import gen  # noqa: F401
