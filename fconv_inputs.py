"""Seeded synthetic inputs for the two fused fp32 convolutions.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It holds only shapes, distributions and random-number generation:
none of the arithmetic of either convolution lives here.

Workloads (names say what they are; shapes follow the problem statements on the
two POPCORNBENCH pages, "Kimi-K2.6 l2_p65" for Conv2d -> AvgPool2d -> Sigmoid ->
Sum and "Kimi-K2.6 l2_p7" for the depthwise-separable Conv1d):

* ``conv2d_tiny``  x[2,3,16,16],     Conv2d 3->4,    k=3, AvgPool k=s=4 (14 -> 3)
* ``conv2d_full``  x[128,8,384,384], Conv2d 8->64,   k=3, AvgPool k=s=4 (382 -> 95)
* ``conv2d_tail``  x[64,16,257,257], Conv2d 16->128, k=5, AvgPool k=s=3 (253 -> 84)
* ``dwsep_small``  x[4,16,256],      depthwise k=9 pad 4, pointwise 16->32
* ``dwsep_full``   x[32,256,4096],   depthwise k=9 pad 4, pointwise 256->512

Distributions: the input is N(0, 1); every weight and bias is
U(-1/sqrt(fan_in), +1/sqrt(fan_in)), PyTorch's default initialisation bound,
where fan_in is Cin*K*K for the Conv2d weight and bias, K for the depthwise
filter, and C for the pointwise weight and its bias.

Random streams: numpy PCG64, seeded with SeedSequence([seed, tensor_id]) so
that every tensor has its own stream (x = 0, conv/depthwise weight = 1,
conv bias/pointwise weight = 2, pointwise bias = 3).
"""

from __future__ import annotations

import math

import numpy as np

WORKLOADS = {
    "conv2d_tiny": dict(kind="conv2d", B=2, Cin=3, H=16, W=16, Cout=4, K=3, pool=4),
    "conv2d_full": dict(kind="conv2d", B=128, Cin=8, H=384, W=384, Cout=64, K=3, pool=4),
    "conv2d_tail": dict(kind="conv2d", B=64, Cin=16, H=257, W=257, Cout=128, K=5, pool=3),
    "dwsep_small": dict(kind="dwsep", B=4, C=16, T=256, O=32, K=9, pad=4),
    "dwsep_full": dict(kind="dwsep", B=32, C=256, T=4096, O=512, K=9, pad=4),
}


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)])))


def normal(shape, seed: int, tensor_id: int) -> np.ndarray:
    """Standard-normal float32 array of ``shape`` from stream (seed, tensor_id)."""
    return _rng(seed, tensor_id).standard_normal(shape, dtype=np.float32)


def uniform(shape, bound: float, seed: int, tensor_id: int) -> np.ndarray:
    """U(-bound, +bound) float32 array of ``shape`` from stream (seed, tensor_id)."""
    r = _rng(seed, tensor_id).random(shape, dtype=np.float64)
    return ((2.0 * r - 1.0) * bound).astype(np.float32)


def conv2d_inputs(B, Cin, H, W, Cout, K, seed=0, **_unused):
    """x[B,Cin,H,W] ~ N(0,1); w[Cout,Cin,K,K], b[Cout] ~ U(+-1/sqrt(Cin*K*K))."""
    bound = 1.0 / math.sqrt(Cin * K * K)
    x = normal((B, Cin, H, W), seed, 0)
    w = uniform((Cout, Cin, K, K), bound, seed, 1)
    b = uniform((Cout,), bound, seed, 2)
    return x, w, b


def dwsep_inputs(B, C, T, O, K, seed=0, **_unused):
    """x[B,C,T] ~ N(0,1); w_dw[C,K] ~ U(+-1/sqrt(K)); w_pw[O,C], b_pw[O] ~ U(+-1/sqrt(C))."""
    x = normal((B, C, T), seed, 0)
    w_dw = uniform((C, K), 1.0 / math.sqrt(K), seed, 1)
    w_pw = uniform((O, C), 1.0 / math.sqrt(C), seed, 2)
    b_pw = uniform((O,), 1.0 / math.sqrt(C), seed, 3)
    return x, w_dw, w_pw, b_pw


def make(name: str, seed: int = 0):
    """Inputs of a named workload as a tuple of float32 numpy arrays."""
    cfg = WORKLOADS[name]
    if cfg["kind"] == "conv2d":
        return conv2d_inputs(seed=seed, **cfg)
    return dwsep_inputs(seed=seed, **cfg)
