"""Floating-point primitives of the oracle (fp32 step-by-step arithmetic).

Every numpy elementwise operation on float32 arrays below is one IEEE-754
binary32 operation with round-to-nearest-even and no fused multiply-add, which
is what makes the encoders reproducible operation by operation.
"""

import numpy as np

F32 = np.float32


def f16_bits(x):
    """fp32 -> fp16 round-to-nearest-even (subnormals kept), as uint16 bits."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_value(bits):
    """fp16 bit patterns -> their exact value as float32."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def rhaz(v):
    """Round half away from zero of float32 values, returned as int64.

    Evaluated as copysign(floor(|v| + 0.5), v) in float64, where |v| + 0.5 is
    exact for every float32 the codecs produce (|v| < 2**28).  Doing it in
    float32 instead would round 0.49999997 up to 1.
    """
    v64 = np.asarray(v, dtype=np.float32).astype(np.float64)
    r = np.floor(np.abs(v64) + 0.5)
    return np.copysign(r, v64).astype(np.int64)


def tree_sum(v):
    """Stride-halving fp32 sum over the last axis: v <- v[:n/2] + v[n/2:].

    The last axis length must be a power of two.  This is the summation order
    the codecs define (it matches a butterfly over lanes l and l + n/2).
    """
    v = np.asarray(v, dtype=np.float32)
    n = v.shape[-1]
    assert n & (n - 1) == 0, "tree_sum needs a power-of-two length"
    while n > 1:
        h = n // 2
        v = v[..., :h] + v[..., h:n]
        n = h
    return v[..., 0]


def safe_recip(d):
    """1.0f / d where d != 0, else 0 (fp32, correctly rounded)."""
    d = np.asarray(d, dtype=np.float32)
    out = np.zeros_like(d)
    nz = d != 0
    out[nz] = F32(1.0) / d[nz]
    return out
