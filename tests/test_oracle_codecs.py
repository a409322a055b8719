"""Pins of the oracle's encoders and decoders (CPU only).

Each test checks the oracle against something other than itself: hand-built
blocks with exact ties, an integer search that re-derives round-half-away,
bit-level fp16 rounding written from the IEEE definition, closed-form
round-trip bounds, and codebook statistics.
"""

import numpy as np
import pytest

from oracle import codecs, fp, lloyd_max

D = 128


def _row(block_values, fill=0.0):
    """A 128-value row whose first block starts with ``block_values``."""
    x = np.full(D, fill, dtype=np.float32)
    x[: len(block_values)] = block_values
    return x[None, :]


def _fp16_bits_by_definition(v):
    """fp32 -> fp16 RNE written from the format definition (integers only)."""
    v = float(np.float32(v))
    if v == 0.0:
        return 0x8000 if np.signbit(v) else 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    from fractions import Fraction

    f = Fraction(a)
    e = 15  # find exponent with 1 <= a / 2^(e-15) < 2 for normals
    while f >= Fraction(2) ** (e - 14) and e < 31:
        e += 1
    while f < Fraction(2) ** (e - 15) and e > 1:
        e -= 1
    if f < Fraction(2) ** -14:  # subnormal: m * 2^-24
        m = f * 2**24
        e_field = 0
    else:
        m = (f / Fraction(2) ** (e - 15) - 1) * 1024
        e_field = e
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if e_field == 0:
        return sign | fl  # fl may carry into the normal range; bits still right
    if fl == 1024:
        fl = 0
        e_field += 1
    return sign | (e_field << 10) | fl


# ------------------------------------------------------------------ helpers
def test_rhaz_definition():
    v = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 0.49999997, -0.49999997, 126.5, -126.5, 0.0, -0.0],
                 dtype=np.float32)
    assert list(fp.rhaz(v)) == [1, 2, 3, -1, -2, -3, 0, 0, 127, -127, 0, 0]


def test_tree_sum_order():
    # the stride-halving order: ((a0+a2)+(a1+a3)); pick values where order matters
    v = np.array([1e8, 1.0, -1e8, 1.0], dtype=np.float32)
    # (1e8 + -1e8) + (1 + 1) = 2 exactly; left-to-right would lose a 1
    assert fp.tree_sum(v) == np.float32(2.0)


@pytest.mark.parametrize("v", [0.0, 1.0, -2.5, 65504.0, 6.1e-5, 5.96e-8, 1e-6, 0.333333, 1234.5678,
                               2.9802322e-08, 3.0e-08, 6.0975552e-05])
def test_f16_rounding_matches_ieee_definition(v):
    assert int(fp.f16_bits(np.float32(v))) == _fp16_bits_by_definition(v)


# ---------------------------------------------------------------------- f16
def test_f16_codec_roundtrip_exact_on_f16_values(rng):
    x = rng.standard_normal((7, D)).astype(np.float16).astype(np.float32)
    q = codecs.quantize_f16(x)
    assert np.array_equal(codecs.dequant_f16(q), x.astype(np.float64))


# --------------------------------------------------------------------- q8_0
@pytest.mark.parametrize("k", [0, 3, 10])
def test_q8_exact_ties_round_away(k):
    u = 2.0 ** -k
    blk = [127 * u, 2.5 * u, -2.5 * u, 1.5 * u, -0.5 * u, 0.5 * u, 126.5 * u]
    q = codecs.quantize_q8_0(_row(blk))
    c = q["codes"][0, : len(blk)].tolist()
    assert c == [127, 3, -3, 2, -1, 1, 127]
    assert int(q["scales"][0, 0]) == _fp16_bits_by_definition(u)


def test_q8_zero_block_and_sign():
    q = codecs.quantize_q8_0(_row([0.0] * 32, fill=0.0))
    assert np.all(q["scales"] == 0) and np.all(q["codes"] == 0)
    q = codecs.quantize_q8_0(_row([-3.0] + [0.0] * 31))
    assert q["codes"][0, 0] == -127 and int(q["scales"][0, 0]) == _fp16_bits_by_definition(3.0 / 127.0)


def test_q8_codes_equal_integer_search(rng):
    x = (rng.standard_normal((64, D)) * rng.lognormal(0, 2, (64, 1))).astype(np.float32)
    q = codecs.quantize_q8_0(x)
    xb = x.reshape(-1, 4, 32)
    d = (np.abs(xb).max(-1) / np.float32(127)).astype(np.float32)
    inv = (np.float32(1) / d).astype(np.float32)
    prod = (xb * inv[..., None]).astype(np.float64)
    # nearest integer by search; exact halves go away from zero
    cand = np.arange(-127, 128, dtype=np.float64)
    dist = np.abs(prod[..., None] - cand)
    best = dist.min(-1, keepdims=True)
    ties = dist == best
    pick = np.where(prod >= 0, np.where(ties, cand, -1e9).max(-1), np.where(ties, cand, 1e9).min(-1))
    assert np.array_equal(q["codes"].reshape(-1, 4, 32).astype(np.float64), pick)


def test_q8_roundtrip_bound(rng):
    x = (rng.standard_normal((256, D)) * rng.lognormal(0, 1.5, (256, 1))).astype(np.float32)
    q = codecs.quantize_q8_0(x)
    xh = codecs.dequant_q8_0(q).reshape(-1, 4, 32)
    xb = x.reshape(-1, 4, 32).astype(np.float64)
    d = (np.abs(x.reshape(-1, 4, 32)).max(-1) / np.float32(127)).astype(np.float64)
    D16 = fp.f16_value(q["scales"]).astype(np.float64)
    bound = 0.5 * d + 127 * np.abs(d - D16) + 1e-6 * d * 127
    assert np.all(np.abs(xb - xh) <= bound[..., None] + 1e-30)


def test_q8_subnormal_scale():
    amax = np.float32(127.0 * 1e-6)  # d = 1e-6 -> fp16 subnormal
    q = codecs.quantize_q8_0(_row([amax, -amax / 2]))
    d = np.float32(amax / np.float32(127))
    assert int(q["scales"][0, 0]) == _fp16_bits_by_definition(d)
    assert int(q["scales"][0, 0]) < 0x0400  # subnormal field


# --------------------------------------------------------------------- q4_0
@pytest.mark.parametrize("a", [1.0, 0.75, 3.0e-3])
def test_q4_opposite_sign_tie_first_index_and_clamp(a):
    q = codecs.quantize_q4_0(_row([a, -a, 0.0]))
    assert int(q["scales"][0, 0]) == _fp16_bits_by_definition(np.float32(a) / np.float32(-8))
    assert q["codes"][0, 0] == 0  # +a -> -8 -> 0
    assert q["codes"][0, 1] == 15  # -a -> +8 -> clamped to 15
    assert q["codes"][0, 2] == 8
    q = codecs.quantize_q4_0(_row([-a, a]))
    assert q["codes"][0, 0] == 0 and q["codes"][0, 1] == 15
    assert int(q["scales"][0, 0]) == _fp16_bits_by_definition(np.float32(a) / np.float32(8))


def test_q4_exact_ties_round_away():
    u = 2.0 ** -4
    q = codecs.quantize_q4_0(_row([-8 * u, 2.5 * u, -2.5 * u, 0.5 * u, -0.5 * u, 7.5 * u]))
    # d = -8u / -8 = u ; codes = RHAZ(x/u) + 8
    assert q["codes"][0, :6].tolist() == [0, 11, 5, 9, 7, 15]


def test_q4_zero_block_positive_zero_scale():
    q = codecs.quantize_q4_0(np.zeros((1, D), np.float32))
    assert np.all(q["scales"] == 0x0000) and np.all(q["codes"] == 8)


def test_q4_roundtrip_bound(rng):
    x = (rng.standard_normal((256, D)) * rng.lognormal(0, 1.5, (256, 1))).astype(np.float32)
    q = codecs.quantize_q4_0(x)
    xh = codecs.dequant_q4_0(q).reshape(-1, 4, 32)
    xb = x.reshape(-1, 4, 32).astype(np.float64)
    a = np.abs(x.reshape(-1, 4, 32)).max(-1).astype(np.float64)
    d = a / 8.0
    D16 = np.abs(fp.f16_value(q["scales"]).astype(np.float64))
    err = np.abs(xb - xh)
    bound = 0.5 * d + 8 * np.abs(d - D16) + 1e-6 * a
    # code 15 is also where RHAZ gave +8 (elements within |d|/2 of -m): error <= |d|
    clamped = q["codes"].reshape(-1, 4, 32) == 15
    ok = np.where(clamped, err <= (d + 8 * np.abs(d - D16) + 1e-6 * a)[..., None],
                  err <= bound[..., None] + 1e-30)
    assert np.all(ok)


def test_nibble_pack_roundtrip(rng):
    c = rng.integers(0, 16, (5, D)).astype(np.uint8)
    p = codecs.pack_nibbles(c)
    assert p.shape == (5, 64)
    assert p[0, 0] == (c[0, 0] | (c[0, 16] << 4))
    assert p[0, 16] == (c[0, 32] | (c[0, 48] << 4))
    assert np.array_equal(codecs.unpack_nibbles(p), c)


# --------------------------------------------------------------------- rot4
def _signs(rng):
    return rng.integers(0, 256, 16, dtype=np.uint8)


def test_rot4_zero_row():
    q = codecs.quantize_rot4(np.zeros((1, D), np.float32), np.zeros(16, np.uint8))
    assert q["norms"][0] == 0 and np.all(q["scales"] == 0) and np.all(q["codes"] == 8)


def test_rot4_norm_field_is_row_norm(rng):
    x = rng.standard_normal((32, D)).astype(np.float32)
    q = codecs.quantize_rot4(x, _signs(rng))
    n = np.linalg.norm(x.astype(np.float64), axis=1)
    N = fp.f16_value(q["norms"]).astype(np.float64)
    assert np.all(np.abs(N - n) <= n * 2.0 ** -11 * 1.001)


def test_rot4_index_is_nearest_level(rng):
    """Away from exact midpoints the threshold count equals argmin |t - c_k|."""
    x = rng.standard_normal((512, D)).astype(np.float32)
    s = _signs(rng)
    q = codecs.quantize_rot4(x, s)
    # recompute t independently in fp64 (the fp32 path differs only in the last ulps)
    from oracle.wht import sign_vector, sylvester

    H = sylvester(D).astype(np.float64)
    w = (x.astype(np.float64) * sign_vector(s)) @ H.T
    u = w / np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True)
    ub = u.reshape(-1, 4, 32)
    t = ub / np.sqrt((ub * ub).mean(-1, keepdims=True))
    lv, thr, _ = lloyd_max.codebook()
    near = np.argmin(np.abs(t[..., None] - lv.astype(np.float64)), axis=-1)
    gap = np.min(np.abs(t[..., None] - thr.astype(np.float64)), axis=-1)
    safe = gap > 1e-5
    assert safe.mean() > 0.99
    assert np.array_equal(q["codes"].reshape(-1, 4, 32)[safe], near[safe])


def test_rot4_statistics_match_lloyd_max_mse(rng):
    x = rng.standard_normal((20000, D)).astype(np.float32)
    s = _signs(rng)
    q = codecs.quantize_rot4(x, s)
    lv, _, _ = lloyd_max.codebook()
    # normalized-domain MSE E(t - c[idx])^2 with fp64 t
    from oracle.wht import sign_vector, sylvester

    H = sylvester(D).astype(np.float64)
    u = ((x.astype(np.float64) * sign_vector(s)) @ H.T) / np.linalg.norm(x, axis=1, keepdims=True)
    ub = u.reshape(-1, 4, 32)
    t = ub / np.sqrt((ub * ub).mean(-1, keepdims=True))
    e = t - lv.astype(np.float64)[q["codes"].reshape(-1, 4, 32)]
    mse = (e * e).mean()
    assert 0.008 < mse < 0.012
    xh = codecs.dequant_rot4(q, s)
    rel = ((xh - x) ** 2).sum(1) / (x.astype(np.float64) ** 2).sum(1)
    assert 0.008 < rel.mean() < 0.013


def test_rot4_decoder_inverts_rotation_exactly():
    """With every whitened value exactly a level, only fp16 rounding of N and
    S separates the decode from the input."""
    lv, _, _ = lloyd_max.codebook()
    from oracle.wht import wht

    rng = np.random.default_rng(5)
    idx = rng.integers(0, 16, (8, D))
    y = lv[idx].astype(np.float64)  # rotated domain values
    s = rng.integers(0, 256, 16, dtype=np.uint8)
    from oracle.wht import sign_vector

    x = sign_vector(s) * wht(y, np.float64) / np.sqrt(128.0)
    q = {"codes": idx.astype(np.uint8),
         "scales": fp.f16_bits(np.ones((8, 4), np.float32)),
         "norms": fp.f16_bits(np.full(8, np.sqrt(128.0), np.float32))}
    xh = codecs.dequant_rot4(q, s)
    n16 = float(fp.f16_value(fp.f16_bits(np.float32(np.sqrt(128.0)))))
    assert np.allclose(xh, x * n16 / np.sqrt(128.0), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------- rot3
def test_rot3_impulse_closed_form():
    """x = a e_j rotates to w = +-a on every channel: each block's RMS is |a|,
    every t is +-1 (index 5 or 2), and the decode is exactly L5 * a * e_j
    with L5 the stored level 0.756 (a fp16-exact, any signs)."""
    lv, _, _ = lloyd_max.codebook(8)
    rng = np.random.default_rng(8)
    for j, a in ((0, 3.0), (77, -0.375), (127, 1.25)):
        s = rng.integers(0, 256, 16, dtype=np.uint8)
        x = np.zeros((1, D), np.float32)
        x[0, j] = a
        q = codecs.quantize_rot3(x, s)
        assert np.all(fp.f16_value(q["scales"]) == abs(a))
        assert set(np.unique(q["codes"]).tolist()) <= {2, 5}
        xh = codecs.dequant_rot3(q, s)
        expect = np.zeros((1, D))
        expect[0, j] = float(lv[5]) * a
        assert np.allclose(xh, expect, rtol=0, atol=1e-12)


def test_rot3_zero_row():
    q = codecs.quantize_rot3(np.zeros((1, D), np.float32), np.zeros(16, np.uint8))
    assert np.all(q["scales"] == 0) and np.all(q["codes"] == 4) and "norms" not in q


def test_rot3_index_is_nearest_level(rng):
    x = rng.standard_normal((512, D)).astype(np.float32)
    s = _signs(rng)
    q = codecs.quantize_rot3(x, s)
    from oracle.wht import sign_vector, sylvester

    H = sylvester(D).astype(np.float64)
    wb = ((x.astype(np.float64) * sign_vector(s)) @ H.T).reshape(-1, 4, 32)
    t = wb / np.sqrt((wb * wb).mean(-1, keepdims=True))
    lv, thr, _ = lloyd_max.codebook(8)
    near = np.argmin(np.abs(t[..., None] - lv.astype(np.float64)), axis=-1)
    gap = np.min(np.abs(t[..., None] - thr.astype(np.float64)), axis=-1)
    safe = gap > 1e-5
    assert safe.mean() > 0.99
    assert np.array_equal(q["codes"].reshape(-1, 4, 32)[safe], near[safe])


def test_rot3_thresholds_symmetric():
    """The 8-level thresholds are symmetric with a zero middle threshold (the
    tie rule itself is pinned on crafted rows in test_oracle_crafted.py)."""
    _, thr, _ = lloyd_max.codebook(8)
    assert thr[3] == 0.0 and all(thr[k] == -thr[6 - k] for k in range(7))


def test_rot3_statistics_match_lloyd_max_mse(rng):
    x = rng.standard_normal((20000, D)).astype(np.float32)
    s = _signs(rng)
    q = codecs.quantize_rot3(x, s)
    xh = codecs.dequant_rot3(q, s)
    rel = ((xh - x) ** 2).sum(1) / (x.astype(np.float64) ** 2).sum(1)
    assert 0.030 < rel.mean() < 0.040  # the 8-level Lloyd-Max MSE is 0.0345


def test_rot3_bits_per_value():
    from oracle import bytes_model

    assert bytes_model.BPV["rot3"] == 3.5
    assert 1.0 - bytes_model.BPV["rot3"] / bytes_model.BPV["q4_0"] == pytest.approx(0.2222, abs=1e-4)  # ~22% smaller


# -------------------------------------------------- planted mistakes (oracle)
def test_planted_fp32_floor_rounding_is_caught(monkeypatch):
    """A plausible mistake (fp32 floor(x + 0.5)) must fail the q8 tie pin."""
    def bad_rhaz(v):
        v = np.asarray(v, np.float32)
        return (np.sign(v) * np.floor(np.abs(v) + np.float32(0.5))).astype(np.int64)

    x = _row([127.0, 0.49999997 * 127.0 / 127.0 * 1.0])
    good = codecs.quantize_q8_0(x)["codes"][0, 1]
    monkeypatch.setattr(codecs, "rhaz", bad_rhaz)
    bad = codecs.quantize_q8_0(x)["codes"][0, 1]
    assert good == 0 and bad == 1


def test_planted_q4_sign_mistake_is_caught(rng, monkeypatch):
    """Dividing by +8 instead of -8 breaks the round-trip bound."""
    x = rng.standard_normal((16, D)).astype(np.float32)
    good = codecs.dequant_q4_0(codecs.quantize_q4_0(x))
    orig = np.float32

    def bad_quant(xx):
        q = codecs.quantize_q4_0(xx)
        q = dict(q)
        q["scales"] = fp.f16_bits(-fp.f16_value(q["scales"]))
        return q

    bad = codecs.dequant_q4_0(bad_quant(x))
    # a correct round trip errs by at most |d| per block (|d|/2 from rounding,
    # |d| at the clamped -m), plus the fp16 rounding of d times |code| <= 8;
    # a sign-flipped scale errs by ~2|x| at the block maximum |x| = 8|d|
    d = np.abs(fp.f16_value(codecs.quantize_q4_0(x)["scales"]).astype(np.float64))  # [16, 4]
    bound = np.repeat(d * (1.0 + 8 * 2.0 ** -10), 32, axis=1)
    assert np.all(np.abs(good - x) <= bound)
    assert np.all(np.max(np.abs(bad - x).reshape(-1, 4, 32), axis=-1) >= 15.0 * d)
    del orig, monkeypatch


def test_domain_guard_rejects_tiny_blocks():
    x = np.zeros((1, D), np.float32)
    x[0, 3] = np.float32(3.0e-39)
    with pytest.raises(AssertionError):
        codecs.quantize_q8_0(x)
    with pytest.raises(AssertionError):
        codecs.quantize_q4_0(x)
    x[0, 3] = np.float32(2.0 ** -100)
    assert codecs.quantize_q8_0(x)["codes"][0, 3] == 127
