"""Seeded synthetic inputs shared by the tests, ``bench.py`` and the oracle.

This package holds geometry and random numbers only: no slot mapping, no
window selection, no masking, no attention, no quantisation.  Both the HIP
library and the oracle derive everything else from what is generated here,
each with its own code.
"""

from .configs import CONFIGS, Geometry, Workload, LayerInputs, make_workload, small_variant  # noqa: F401
