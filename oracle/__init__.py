"""CPU oracle for the fused fp32 convolutions -- TEST INFRASTRUCTURE ONLY.

A slow, literal, double-precision reference (C, loaded with ctypes).  Only the
tests, the smoke check and the benchmark's CPU-baseline leg may use it; the
HIP library never calls it and shares no code with it.
"""

from .oracle import (  # noqa: F401
    POOL_AVG,
    POOL_MAX,
    conv2d_pool_sigmoid_sum,
    conv2d_pooled_at,
    conv2d_sizes,
    dwsep_conv1d,
    dwsep_conv1d_at,
    dwsep_tout,
    load,
)
