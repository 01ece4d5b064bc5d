"""Seeded synthetic layers shaped like the pages' workloads.

This package only makes inputs (weights and calibration activations); it
holds none of the quantization method's arithmetic.  Both the oracle side and
the HIP side of every test and benchmark consume the same bytes produced here.
"""

from .workloads import *  # noqa: F401,F403
