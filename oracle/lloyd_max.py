"""Lloyd-Max quantizers (16 and 8 levels) for a standard normal source.

The rot4 codec stores, per value, the index of one of 16 reconstruction
levels; the rot3 codec one of 8.  The pages name a scalar quantizer applied after the random-sign FWHT
rotation (buun-llama-cpp page, "How it works", step 1, and the rotated
"turbo4" row of its "Codecs" table); the rotation makes entries close to
i.i.d. N(0,1), and the minimum-MSE scalar quantizer for that source is the
Lloyd-Max quantizer (J. Max, "Quantizing for minimum distortion", IRE Trans.
Inf. Theory 6(1), 1960; S. Lloyd, "Least squares quantization in PCM", 1957/1982).

Reading taken (the pages give no codebook): levels are the 16-level (rot4) or
8-level (rot3, the 3-bit "tq3_0 / turbo3" class) Lloyd-Max levels for N(0,1),
solved here in fp64, then stored at fp16 precision (the same precision as
every other stored field).  The encoder's decision
thresholds are the fp32 midpoints of adjacent stored levels, so nearest-level
coding and threshold counting agree.
"""

import math

import numpy as np

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _pdf(x):
    return _INV_SQRT_2PI * math.exp(-0.5 * x * x) if math.isfinite(x) else 0.0


def _upper_tail(x):
    """P(X > x) for X ~ N(0,1), accurate in the tail."""
    if x == math.inf:
        return 0.0
    return 0.5 * math.erfc(x / _SQRT2)


def _centroid(a, b):
    """E[X | a < X < b] for X ~ N(0,1), 0 <= a < b <= inf."""
    mass = _upper_tail(a) - _upper_tail(b)
    return (_pdf(a) - _pdf(b)) / mass


def solve_positive_half(n_levels=16, tol=1e-15, max_iter=2_000_000):
    """Lloyd iteration on the positive half of a symmetric quantizer.

    Alternates the two optimality conditions until the levels stop moving:
    (1) each threshold is the midpoint of its two neighbouring levels;
    (2) each level is the conditional mean of N(0,1) over its cell.
    By symmetry the middle threshold is exactly 0, so only n_levels/2 levels
    are solved.  Returns (levels, thresholds, iterations) in fp64, where
    ``thresholds`` are the n_levels/2 - 1 positive interior thresholds.
    """
    half = n_levels // 2
    # start from equally probable cells
    c = [0.0] * half
    for i in range(half):
        c[i] = 0.5 + i  # any increasing start converges
    it = 0
    for it in range(1, max_iter + 1):
        t = [0.0] + [0.5 * (c[i] + c[i + 1]) for i in range(half - 1)] + [math.inf]
        new = [_centroid(t[i], t[i + 1]) for i in range(half)]
        delta = max(abs(new[i] - c[i]) for i in range(half))
        c = new
        if delta < tol:
            break
    thr = [0.5 * (c[i] + c[i + 1]) for i in range(half - 1)]
    return np.array(c), np.array(thr), it


def full_levels_fp64(n_levels=16):
    """All n_levels levels in increasing order (fp64): c[n-1-k] = -c[k]."""
    pos, _, _ = solve_positive_half(n_levels)
    return np.concatenate([-pos[::-1], pos])


def mse_fp64(levels, thresholds):
    """Mean squared error of a quantizer on N(0,1), by exact cell integrals.

    For a cell (a, b) with level y:  E[(X - y)^2; a<X<b]
      = [Phi - x phi]_a^b - 2 y [ -phi ]_a^b + y^2 [Phi]_a^b.
    ``levels`` has n entries, ``thresholds`` the n-1 interior thresholds.
    """
    edges = [-math.inf] + list(thresholds) + [math.inf]
    total = 0.0
    for k, y in enumerate(levels):
        a, b = edges[k], edges[k + 1]
        mass = _upper_tail(a) - _upper_tail(b)
        first = _pdf(a) - _pdf(b)                      # integral of x phi
        xa = 0.0 if not math.isfinite(a) else a * _pdf(a)
        xb = 0.0 if not math.isfinite(b) else b * _pdf(b)
        second = mass + xa - xb                        # integral of x^2 phi
        total += second - 2.0 * y * first + y * y * mass
    return total


def codebook(n_levels=16):
    """The stored codebook and thresholds (16 levels: rot4; 8 levels: rot3).

    Returns (levels_f32, thresholds_f32, levels_fp16_bits):
      levels_f32[k]     -- level k rounded to fp16 (RNE), as its exact fp32 value
      thresholds_f32[k] -- fp32((levels_f32[k] + levels_f32[k+1]) * 0.5), k < n-1
      levels_fp16_bits  -- the fp16 bit patterns of the levels
    The fp32 sum of two fp16 values is exact and * 0.5 is exact, so every
    threshold is the exact midpoint of its two stored levels.
    """
    lv = full_levels_fp64(n_levels)
    bits = lv.astype(np.float32).astype(np.float16).view(np.uint16)
    # fp64 -> fp16 through fp32: the two roundings cannot differ from a direct
    # fp64 -> fp16 rounding for these values (checked by a test).
    lv16 = bits.view(np.float16).astype(np.float32)
    thr = ((lv16[:-1] + lv16[1:]) * np.float32(0.5)).astype(np.float32)
    return lv16, thr, bits
