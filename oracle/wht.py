"""Walsh-Hadamard transform used by the rotated codec.

The rotation is the one the buun-llama-cpp page names in step 1 of "How it
works" (FWHT with random sign flips, which turns correlated KV vectors into
near-i.i.d. Gaussian entries) and that the Randozart/VITRIOL page calls
"Walsh-Hadamard-rotated quantizers" ("How It Works -- Resident mode").  The
pages give no normalisation or stage order; the reading taken here is the
Sylvester (natural) order, stages h = 1, 2, 4, ..., n/2, unnormalised, so that
H is symmetric and H @ H = n I.
"""

import numpy as np


def wht(x, dtype=np.float32):
    """Unnormalised fast WHT over the last axis, in ``dtype`` arithmetic.

    For h = 1, 2, 4, ..., n/2 and every index i with (i & h) == 0 the pair
    (w_i, w_{i+h}) becomes (w_i + w_{i+h}, w_i - w_{i+h}).  Each add and
    subtract is one rounding in ``dtype``; the stage order is part of the
    rot4 format.
    """
    w = np.array(x, dtype=dtype, copy=True)
    n = w.shape[-1]
    assert n & (n - 1) == 0
    lead = w.shape[:-1]
    h = 1
    while h < n:
        v = w.reshape(lead + (n // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        w = v.reshape(lead + (n,))
        h *= 2
    return w


def sylvester(n):
    """The n x n Sylvester Hadamard matrix (entries +-1), built by doubling."""
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def sign_vector(mask16):
    """Expand a 16-byte sign mask into +-1 (int64) for 128 channels.

    Bit (j & 7) of byte (j >> 3) set means channel j is negated.
    """
    m = np.asarray(mask16, dtype=np.uint8)
    assert m.shape == (16,)
    bits = (m[np.arange(128) >> 3] >> (np.arange(128) & 7)) & 1
    return np.where(bits == 1, -1, 1).astype(np.int64)
