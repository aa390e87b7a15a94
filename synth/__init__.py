"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's
checks: counter-based random numbers, packed-weight containers, the encoders
that produce packed codes, and MoE routing.  Nothing here dequantizes or
multiplies; that arithmetic lives separately in the oracle and in the HIP
library.
"""

from . import formats, quant, rng, routing  # noqa: F401
from .formats import AFFINE4_G64, MXFP4, NVFP4, Q6_K, BLOCK, NAMES, BY_NAME, Packed  # noqa: F401
