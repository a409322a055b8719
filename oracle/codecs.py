"""The four KV codecs, written step by step (encoders in fp32, decoders in fp64).

A row is one (token, KV head) vector of D = 128 fp32 values.  Blocks are 32
consecutive channels (4 per row).  The codec family and its sizes are the
buun-llama-cpp page's "Codecs" table (f16 16 bpv, q8_0 8.5 bpv, q4_0 4.5 bpv,
and the rotated scalar "turbo" codecs); the K=f16 / V=q8_0 pairing is the
serving contract in the serverAppConfigs commit log (tests/frank_small_unit.bats
page).  The pages print no encoder arithmetic, so each encoder below states
its reading.  Shared rules (readings):

* codes are computed from the fp32 scale through its fp32 reciprocal; only the
  stored scale is rounded to fp16 (round-to-nearest-even);
* integer rounding is round-half-away-from-zero;
* a block whose largest magnitude is 0 stores scale +0.0 and the zero code.

Domain: finite inputs; every nonzero 32-value block has largest magnitude at
least 2^-100 (below that the fp32 reciprocal of the scale overflows and
0 * inf leaves the codes undefined) and the stored fp16 fields do not overflow.
The encoders assert the first two conditions.

Logical outputs (what parity compares, bit for bit):
  f16   codes uint16[N,128]              (fp16 bits)
  q8_0  codes int8[N,128], scales uint16[N,4]
  q4_0  codes uint8[N,128] in 0..15, scales uint16[N,4]
  rot4  idx uint8[N,128] in 0..15, scales uint16[N,4], norms uint16[N]
  rot3  idx uint8[N,128] in 0..7, scales uint16[N,4]
For q4_0 and rot4 the canonical byte packing of block b is
byte j (0..15) = code[32b + j] | code[32b + j + 16] << 4   (``pack_nibbles``).
"""

import numpy as np

from .fp import F32, f16_bits, f16_value, rhaz, safe_recip, tree_sum
from .lloyd_max import codebook
from .wht import sign_vector, wht

D = 128
QK = 32
NB = D // QK

CODECS = ("f16", "q8_0", "q4_0", "rot4", "rot3")


MIN_BLOCK_MAX = np.float32(2.0 ** -100)


def _rows(x):
    x = np.asarray(x, dtype=np.float32)
    assert x.ndim == 2 and x.shape[1] == D, x.shape
    assert np.all(np.isfinite(x)), "codec inputs must be finite"
    return x


def _check_block_domain(xb):
    amax = np.max(np.abs(xb), axis=-1)
    assert np.all((amax == 0) | (amax >= MIN_BLOCK_MAX)), "block maximum below 2^-100 is outside the domain"


# ----------------------------------------------------------------------- f16
def quantize_f16(x):
    """code_j = fp16(x_j), round-to-nearest-even."""
    return {"codes": f16_bits(_rows(x))}


def dequant_f16(q):
    return f16_value(q["codes"]).astype(np.float64)


# ---------------------------------------------------------------------- q8_0
def quantize_q8_0(x):
    """q8_0, per 32-value block (scale amax/127, int8 codes).

    amax = max_j |x_j|; d = amax / 127 (fp32 division); id = 1/d (0 if d = 0);
    c_j = clamp(RHAZ(x_j * id), -127, 127); stored scale D = fp16(d).
    """
    x = _rows(x)
    xb = x.reshape(-1, NB, QK)
    _check_block_domain(xb)
    amax = np.max(np.abs(xb), axis=-1)
    d = (amax / F32(127.0)).astype(np.float32)
    inv = safe_recip(d)
    prod = (xb * inv[..., None]).astype(np.float32)
    c = np.clip(rhaz(prod), -127, 127).astype(np.int8)
    return {"codes": c.reshape(-1, D), "scales": f16_bits(d)}


def dequant_q8_0(q):
    s = f16_value(q["scales"]).astype(np.float64)
    c = q["codes"].astype(np.float64).reshape(-1, NB, QK)
    return (c * s[..., None]).reshape(-1, D)


# ---------------------------------------------------------------------- q4_0
def quantize_q4_0(x):
    """q4_0, per 32-value block (signed-max / -8, offset +8, clamp 0..15).

    j* = first j with |x_j| = amax; m = x_{j*};
    d = +0.0 if amax == 0 else m / -8 (fp32); id = 1/d (0 if d == 0);
    c_j = min(15, max(0, RHAZ(x_j * id) + 8)); stored scale D = fp16(d).
    The clamp only acts on elements within |d|/2 of -m (they would round to +8).
    """
    x = _rows(x)
    xb = x.reshape(-1, NB, QK)
    _check_block_domain(xb)
    a = np.abs(xb)
    amax = a.max(axis=-1)
    jstar = np.argmax(a, axis=-1)  # numpy returns the first maximal index
    m = np.take_along_axis(xb, jstar[..., None], axis=-1)[..., 0]
    d = np.where(amax == 0, F32(0.0), (m / F32(-8.0)).astype(np.float32)).astype(np.float32)
    inv = safe_recip(d)
    prod = (xb * inv[..., None]).astype(np.float32)
    c = np.clip(rhaz(prod) + 8, 0, 15).astype(np.uint8)
    return {"codes": c.reshape(-1, D), "scales": f16_bits(d)}


def dequant_q4_0(q):
    s = f16_value(q["scales"]).astype(np.float64)
    c = q["codes"].astype(np.float64).reshape(-1, NB, QK) - 8.0
    return (c * s[..., None]).reshape(-1, D)


# ---------------------------------------------------------------------- rot4
def level_index(t, thr):
    """Level index of whitened fp32 values ``t`` against ascending thresholds
    ``thr`` (the midpoints of adjacent levels): the number of thresholds below
    t, where a value lying exactly on a threshold goes to the level farther
    from zero, and 0 (either sign) to the first non-negative level.

    Equivalently: the nearest level, exact midpoints resolved away from zero.
    Both rotated codecs (rot4 with 15 thresholds, rot3 with 7) use this rule.
    Counted as: for t >= 0 (-0 included) the thresholds at or below t, for
    t < 0 the thresholds strictly below t.
    """
    t = np.asarray(t, dtype=np.float32)
    thr = np.asarray(thr, dtype=np.float32)
    at_or_below = np.searchsorted(thr, t, side="right")
    strictly_below = np.searchsorted(thr, t, side="left")
    return np.where(t >= 0, at_or_below, strictly_below)


def whiten_rot4(x, signs16):
    """Steps 1-7 of the rot4 encoder (see ``quantize_rot4``), all fp32.

    Returns (t [N,4,32], r_b [N,4], n [N]): the whitened values whose level
    index is stored, the per-block RMS and the row norm before fp16 rounding.
    """
    x = _rows(x)
    s = sign_vector(signs16)
    r = np.where(s < 0, -x, x).astype(np.float32)
    w = wht(r, np.float32)
    n = np.sqrt(tree_sum((x * x).astype(np.float32))).astype(np.float32)
    g = safe_recip(n)
    u = (w * g[:, None]).astype(np.float32)
    ub = u.reshape(-1, NB, QK)
    ms = (tree_sum((ub * ub).astype(np.float32)) * F32(0.03125)).astype(np.float32)
    rb = np.sqrt(ms).astype(np.float32)
    ib = safe_recip(rb)
    t = (ub * ib[..., None]).astype(np.float32)
    return t, rb, n


def quantize_rot4(x, signs16):
    """Rotated 4-bit codec (random signs, WHT, fp16 norm, per-32 fp16 RMS scale,
    16-level Lloyd-Max indices).

    Steps, all fp32, in this order:
      1. r_j = s_j x_j                      (s = +-1 from the 16-byte sign mask)
      2. w = WHT(r)                         (unnormalised; stages h = 1..64)
      3. n = sqrt(tree(x_j * x_j))          (norm of the model-domain row)
      4. N = fp16(n)
      5. g = 1/n (0 if n == 0);  u_j = w_j * g        (u has mean square ~1)
      6. per block b: r_b = sqrt(tree32(u_j * u_j) * 0.03125);  S_b = fp16(r_b)
      7. ib = 1/r_b (0 if r_b == 0);  t_j = u_j * ib
      8. idx_j = level_index(t_j) over the 15 thresholds
         (a tie goes to the level farther from zero; 0 -> 8)
    Reading for the two fp16 fields: the norm is ||x||_2 of the input row and
    the block scale is the RMS of the norm-whitened rotated block, so N*S_b is
    the per-block magnitude and the Lloyd-Max levels see unit-variance input.
    """
    t, rb, n = whiten_rot4(x, signs16)
    _, thr, _ = codebook()
    idx = level_index(t, thr)
    return {
        "codes": idx.astype(np.uint8).reshape(-1, D),
        "scales": f16_bits(rb),
        "norms": f16_bits(n),
    }


def dequant_rot4_rotated(q):
    """Rotated-domain reconstruction y_j = N * S_b * level[idx_j] / sqrt(128)."""
    lv, _, _ = codebook()
    N = f16_value(q["norms"]).astype(np.float64)
    S = f16_value(q["scales"]).astype(np.float64)
    c = lv.astype(np.float64)[q["codes"].astype(np.int64)].reshape(-1, NB, QK)
    y = c * S[..., None] * N[:, None, None] / np.sqrt(128.0)
    return y.reshape(-1, D)


def dequant_rot4(q, signs16):
    """Model-domain reconstruction x = s * (H y) / sqrt(128), in fp64."""
    y = dequant_rot4_rotated(q)
    s = sign_vector(signs16).astype(np.float64)
    return s * wht(y, np.float64) / np.sqrt(128.0)


# ---------------------------------------------------------------------- rot3
def whiten_rot3(x, signs16):
    """Steps 1-3 of the rot3 encoder (see ``quantize_rot3``), all fp32.

    Returns (t [N,4,32], r_b [N,4]).
    """
    x = _rows(x)
    s = sign_vector(signs16)
    r = np.where(s < 0, -x, x).astype(np.float32)
    w = wht(r, np.float32)
    wb = w.reshape(-1, NB, QK)
    ms = (tree_sum((wb * wb).astype(np.float32)) * F32(0.03125)).astype(np.float32)
    rb = np.sqrt(ms).astype(np.float32)
    ib = safe_recip(rb)
    t = (wb * ib[..., None]).astype(np.float32)
    return t, rb


def quantize_rot3(x, signs16):
    """Rotated 3-bit codec, 3.5 bits/value (the "tq3_0 / turbo3" class of the
    Randozart/VITRIOL page's "What sets VITRIOL apart" table and the
    buun-llama-cpp page's "Codecs" table: WHT-rotated, 3-bit scalar codes).

    Steps, all fp32, in this order:
      1. r_j = s_j x_j;  w = WHT(r)          (as rot4, unnormalised)
      2. per block b: r_b = sqrt(tree32(w_j * w_j) * 0.03125);  S_b = fp16(r_b)
      3. ib = 1/r_b (0 if r_b == 0);  t_j = w_j * ib
      4. idx_j = level_index(t_j) over the 7 thresholds of the 8-level
         codebook (a tie goes to the level farther from zero; 0 -> 4)
    Reading: with one fp16 per 32 values (3 + 16/32 = 3.5 bits/value) the
    block scale is the RMS of the rotated block itself (no row norm), so the
    rotated-domain reconstruction is S_b * level, i.e. y = w / sqrt(128)
    reconstructs as S_b * level / sqrt(128), the domain rot4 uses.
    """
    t, rb = whiten_rot3(x, signs16)
    _, thr, _ = codebook(8)
    idx = level_index(t, thr)
    return {"codes": idx.astype(np.uint8).reshape(-1, D), "scales": f16_bits(rb)}


def dequant_rot3_rotated(q):
    """Rotated-domain reconstruction y_j = S_b * level[idx_j] / sqrt(128)."""
    lv, _, _ = codebook(8)
    S = f16_value(q["scales"]).astype(np.float64)
    c = lv.astype(np.float64)[q["codes"].astype(np.int64)].reshape(-1, NB, QK)
    return (c * S[..., None] / np.sqrt(128.0)).reshape(-1, D)


def dequant_rot3(q, signs16):
    """Model-domain reconstruction x = s * (H y) / sqrt(128), in fp64."""
    y = dequant_rot3_rotated(q)
    s = sign_vector(signs16).astype(np.float64)
    return s * wht(y, np.float64) / np.sqrt(128.0)


# ------------------------------------------------------------------ dispatch
def quantize(codec, x, signs16=None):
    if codec == "f16":
        return quantize_f16(x)
    if codec == "q8_0":
        return quantize_q8_0(x)
    if codec == "q4_0":
        return quantize_q4_0(x)
    if codec == "rot4":
        return quantize_rot4(x, signs16)
    if codec == "rot3":
        return quantize_rot3(x, signs16)
    raise ValueError(codec)


def dequant(codec, q, signs16=None):
    if codec == "f16":
        return dequant_f16(q)
    if codec == "q8_0":
        return dequant_q8_0(q)
    if codec == "q4_0":
        return dequant_q4_0(q)
    if codec == "rot4":
        return dequant_rot4(q, signs16)
    if codec == "rot3":
        return dequant_rot3(q, signs16)
    raise ValueError(codec)


def pack_nibbles(codes):
    """Canonical 4-bit packing of a [N,128] code array into [N,64] bytes:
    byte 16b + j = code[32b + j] | code[32b + j + 16] << 4."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1, NB, QK)
    return (c[..., :16] | (c[..., 16:] << 4)).reshape(-1, D // 2)


def unpack_nibbles(packed):
    p = np.asarray(packed, dtype=np.uint8).reshape(-1, NB, 16)
    return np.concatenate([p & 15, p >> 4], axis=-1).reshape(-1, D)
