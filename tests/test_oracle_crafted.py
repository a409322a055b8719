"""Pins of the encoders' rounding rules and operation order on crafted rows (CPU only).

The rows in ``golden/crafted_rows.txt`` (inputs only, found by
``golden/make_crafted_rows.py`` with the oracle) are ones where a rule decides
a stored field:

* tie rows: a whitened rot4 / rot3 value lands exactly on a nonzero
  threshold, so the index is set by the tie rule;
* recip rows: rounding x * (1/d) and rounding x / d give different codes;
* order rows: reversing the WHT stage order, or summing the row norm or a
  block's mean square with numpy's pairwise ``np.sum`` instead of the
  stride-halving tree, moves a stored field.

Expected values come from a reference written here from the codec
definitions in exact rational arithmetic: every step is computed exactly with
``fractions.Fraction`` and rounded to the nearest binary32 value (ties to
even) by the rounding rule written out below, and the level index is the
nearest level with exact midpoints sent to the level farther from zero (the
oracle counts thresholds instead).  The tie indices are also stated by hand.
The planted-mistake tests at the end swap one rule or order in the oracle
and show that a pin here fails.
"""

import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import codecs, fp, lloyd_max

D = 128
HERE = os.path.dirname(os.path.abspath(__file__))


# ------------------------------------------------------------------ fixture
def _load():
    rows, signs = [], None
    with open(os.path.join(HERE, "golden", "crafted_rows.txt")) as f:
        for line in f:
            if line.startswith("# signs "):
                signs = np.frombuffer(bytes.fromhex(line.split()[2]), dtype=np.uint8).copy()
                continue
            if line.startswith("#") or not line.strip():
                continue
            head, body = line.split(":")
            kind, codec, ch, detail = head.split()
            x = np.array([int(w, 16) for w in body.split()], dtype=np.uint32).view(np.float32)
            assert x.shape == (D,)
            rows.append(dict(kind=kind, codec=codec, ch=int(ch), detail=detail, x=x))
    assert signs is not None and signs.shape == (16,)
    return rows, signs


ROWS, SIGNS = _load()


def _of(kind, codec=None):
    return [r for r in ROWS if r["kind"] == kind and (codec is None or r["codec"] == codec)]


# ------------------------------------------ exact arithmetic, fp32 rounding
def r32(v):
    """The binary32 value nearest to the rational v (ties to even; subnormal
    quantum 2^-149).  Signed zero is not tracked (no stored field here
    depends on it)."""
    v = Fr(v)
    if v == 0:
        return Fr(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    if Fr(2) ** e > a:
        e -= 1
    if Fr(2) ** (e + 1) <= a:
        e += 1
    q = Fr(2) ** (max(e, -126) - 23)  # spacing of binary32 values at a
    m = a / q
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * q
    assert r < Fr(2) ** 128, "overflow"
    return r if v > 0 else -r


def sqrt32(a):
    """The binary32 value nearest to sqrt(a), a >= 0 rational: start from a
    float guess, then move to the neighbour on the side of sqrt(a) while
    sqrt(a) lies beyond the midpoint (compared exactly through squares)."""
    a = Fr(a)
    assert a >= 0
    if a == 0:
        return Fr(0)
    r = np.float32(math.sqrt(float(a)))
    while True:
        up = np.nextafter(r, np.float32(np.inf))
        dn = np.nextafter(r, np.float32(0))
        if a > ((Fr(float(r)) + Fr(float(up))) / 2) ** 2:
            r = up
        elif a < ((Fr(float(r)) + Fr(float(dn))) / 2) ** 2:
            r = dn
        else:
            return Fr(float(r))


def recip32(d):
    return Fr(0) if d == 0 else r32(1 / d)


def rhaz(v):
    """Round half away from zero of an exact rational."""
    a = abs(v)
    n = math.floor(a + Fr(1, 2))
    return n if v >= 0 else -n


def f16_bits(v):
    """fp16 bit pattern of the rational v (RNE, subnormals kept), by the format's definition."""
    from test_oracle_codecs import _fp16_bits_by_definition

    return _fp16_bits_by_definition(float(v))


def tree(vals):
    """Stride-halving sum, one binary32 rounding per addition."""
    v = list(vals)
    while len(v) > 1:
        h = len(v) // 2
        v = [r32(v[i] + v[i + h]) for i in range(h)]
    return v[0]


def wht_ref(r):
    """Unnormalised Sylvester WHT: for h = 1, 2, ..., 64, every pair (i, i+h)
    with i & h == 0 becomes (a + b, a - b), each rounded to binary32."""
    w = list(r)
    h = 1
    while h < D:
        for i in range(D):
            if i & h == 0:
                a, b = w[i], w[i + h]
                w[i], w[i + h] = r32(a + b), r32(a - b)
        h *= 2
    return w


def nearest_level(t, levels):
    """Index of the level nearest to t; an exact midpoint goes to the level of
    larger magnitude (farther from zero); t = 0 to the non-negative level."""
    dist = [abs(t - L) for L in levels]
    best = min(dist)
    cand = [k for k, dd in enumerate(dist) if dd == best]
    return max(cand, key=lambda k: (abs(levels[k]), levels[k]))


def _levels(n):
    lv, _, _ = lloyd_max.codebook(n)
    return [Fr(float(v)) for v in lv]


def _signs(mask):
    bits = (mask[np.arange(D) >> 3] >> (np.arange(D) & 7)) & 1
    return [-1 if b else 1 for b in bits]


# ----------------------------------------------------- reference encoders
def ref_q8_0(x):
    X = [Fr(float(v)) for v in x]
    codes, scales = [], []
    for b in range(4):
        blk = X[32 * b:32 * b + 32]
        amax = max(abs(v) for v in blk)
        d = r32(amax / 127)
        inv = recip32(d)
        codes += [max(-127, min(127, rhaz(r32(v * inv)))) for v in blk]
        scales.append(f16_bits(d))
    return {"codes": codes, "scales": scales}


def ref_q4_0(x):
    X = [Fr(float(v)) for v in x]
    codes, scales = [], []
    for b in range(4):
        blk = X[32 * b:32 * b + 32]
        amax = max(abs(v) for v in blk)
        m = next(v for v in blk if abs(v) == amax)  # the first of largest magnitude
        d = Fr(0) if amax == 0 else r32(m / -8)
        inv = recip32(d)
        codes += [max(0, min(15, rhaz(r32(v * inv)) + 8)) for v in blk]
        scales.append(f16_bits(d))
    return {"codes": codes, "scales": scales}


def ref_rot4(x, mask):
    """Returns the stored fields and the whitened values t (exact binary32 values)."""
    X = [Fr(float(v)) for v in x]
    s = _signs(mask)
    w = wht_ref([X[j] * s[j] for j in range(D)])
    n = sqrt32(tree([r32(v * v) for v in X]))
    g = recip32(n)
    u = [r32(v * g) for v in w]
    t, scales = [], []
    for b in range(4):
        ub = u[32 * b:32 * b + 32]
        rb = sqrt32(r32(tree([r32(v * v) for v in ub]) * Fr(1, 32)))
        ib = recip32(rb)
        t += [r32(v * ib) for v in ub]
        scales.append(f16_bits(rb))
    lv = _levels(16)
    return {"codes": [nearest_level(v, lv) for v in t], "scales": scales, "norms": [f16_bits(n)]}, t


def ref_rot3(x, mask):
    X = [Fr(float(v)) for v in x]
    s = _signs(mask)
    w = wht_ref([X[j] * s[j] for j in range(D)])
    t, scales = [], []
    for b in range(4):
        wb = w[32 * b:32 * b + 32]
        rb = sqrt32(r32(tree([r32(v * v) for v in wb]) * Fr(1, 32)))
        ib = recip32(rb)
        t += [r32(v * ib) for v in wb]
        scales.append(f16_bits(rb))
    lv = _levels(8)
    return {"codes": [nearest_level(v, lv) for v in t], "scales": scales}, t


REF = {"q8_0": lambda x: ref_q8_0(x), "q4_0": lambda x: ref_q4_0(x),
       "rot4": lambda x: ref_rot4(x, SIGNS)[0], "rot3": lambda x: ref_rot3(x, SIGNS)[0]}

_REF_CACHE = {}


def _ref(codec, i):
    key = (codec, i)
    if key not in _REF_CACHE:
        _REF_CACHE[key] = REF[codec](ROWS[i]["x"])
    return _REF_CACHE[key]


# ------------------------------------------------------------- the checks
def check_ties(rows, quantize=codecs.quantize):
    """On a tie row the whitened value at the row's channel equals threshold
    k, the exact midpoint of levels k and k+1; the stored index is then the
    level farther from zero: k+1 for a positive threshold, k for a negative
    one (stated by hand, not computed by the rule under test)."""
    for r in rows:
        codec, j, k = r["codec"], r["ch"], int(r["detail"][3:])
        n = 16 if codec == "rot4" else 8
        lv = _levels(n)
        mid = (lv[k] + lv[k + 1]) / 2
        assert mid != 0
        _, t = (ref_rot4 if codec == "rot4" else ref_rot3)(r["x"], SIGNS)
        assert t[j] == mid, f"{codec} row does not land on threshold {k}"
        want = k + 1 if mid > 0 else k
        got = int(quantize(codec, r["x"][None], SIGNS)["codes"][0, j])
        assert got == want, f"{codec} tie on threshold {k} (t = {float(mid):+.6f}): index {got}, want {want}"


def check_recip(rows, quantize):
    """The crafted element x of a recip row: code from x * (1/d) (exact
    arithmetic, each step rounded to binary32), which differs from the code
    x / d would give."""
    for r in rows:
        codec, j, x = r["codec"], r["ch"], r["x"]
        blk = [Fr(float(v)) for v in x[:32]]
        amax = max(abs(v) for v in blk)
        if codec == "q8_0":
            d = r32(amax / 127)
            code = lambda p: max(-127, min(127, rhaz(p)))
        else:
            m = next(v for v in blk if abs(v) == amax)
            d = r32(m / -8)
            code = lambda p: max(0, min(15, rhaz(p) + 8))
        xj = blk[j]
        want = code(r32(xj * r32(1 / d)))
        other = code(r32(xj / d))
        assert want != other, "row does not separate the two rules"
        got = int(quantize(x[None])["codes"][0, j])
        assert got == want, f"{codec}: code {got}, want {want} (x / d would give {other})"


def check_reference(codec, indices, quantize=codecs.quantize):
    """Every stored field of the oracle's encoding equals the exact reference."""
    for i in indices:
        ref = _ref(codec, i)
        q = quantize(codec, ROWS[i]["x"][None], SIGNS if codec in ("rot4", "rot3") else None)
        for key, want in ref.items():
            got = [int(v) for v in np.asarray(q[key]).reshape(-1)]
            if codec == "q8_0" and key == "codes":
                got = [int(np.int8(v)) for v in got]
            assert got == [int(v) for v in want], (
                f"{codec} {key} differs from the exact reference on crafted row {i} "
                f"({ROWS[i]['kind']} {ROWS[i]['detail']})")


# ---------------------------------------------------------------- pins
def test_fixture_has_every_kind():
    assert len(_of("tie", "rot4")) >= 8 and len(_of("tie", "rot3")) >= 6
    for codec in ("q8_0", "q4_0"):
        assert {r["detail"] for r in _of("recip", codec)} == {"pos", "neg"}
    for codec, muts in (("rot4", {"wht_reversed", "norm_np_sum", "block_np_sum"}),
                        ("rot3", {"wht_reversed", "block_np_sum"})):
        assert {r["detail"] for r in _of("order", codec)} == muts
    # ties at both signs
    for codec, n in (("rot4", 16), ("rot3", 8)):
        ks = [int(r["detail"][3:]) for r in _of("tie", codec)]
        assert min(ks) < n // 2 - 1 < max(ks)


def test_level_index_rule_by_hand():
    """Thresholds, their float neighbours and zero, through the oracle's index
    rule; expected indices stated by hand from the levels' order."""
    for n in (16, 8):
        lv, thr, _ = lloyd_max.codebook(n)
        half = n // 2
        assert thr[half - 1] == 0.0
        for k, th in enumerate(thr):
            th = np.float32(th)
            up, dn = np.nextafter(th, np.float32(np.inf)), np.nextafter(th, np.float32(-np.inf))
            got = codecs.level_index(np.array([dn, th, up], np.float32), thr).tolist()
            if th > 0:
                assert got == [k, k + 1, k + 1], (n, k, got)
            elif th < 0:
                assert got == [k, k, k + 1], (n, k, got)
            else:
                assert got == [half - 1, half, half], (n, k, got)
        assert codecs.level_index(np.array([-0.0], np.float32), thr).tolist() == [half]
        assert codecs.level_index(np.array([-1e30, 1e30], np.float32), thr).tolist() == [0, n - 1]


@pytest.mark.parametrize("codec", ["rot4", "rot3"])
def test_crafted_ties_go_away_from_zero(codec):
    check_ties(_of("tie", codec))


@pytest.mark.parametrize("codec", ["q8_0", "q4_0"])
def test_crafted_codes_use_the_fp32_reciprocal(codec):
    check_recip(_of("recip", codec), getattr(codecs, f"quantize_{codec}"))


@pytest.mark.parametrize("codec", ["q8_0", "q4_0", "rot4", "rot3"])
def test_crafted_rows_match_exact_reference(codec):
    """All crafted rows through each quantized codec: every stored field
    equals the exact-arithmetic reference (WHT stage order, tree sums,
    reciprocals, correctly rounded square roots, nearest-level indices)."""
    check_reference(codec, range(len(ROWS)))


def test_exact_reference_on_random_rows():
    """The reference and the oracle agree on ordinary rows too."""
    global ROWS
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((3, D)) * rng.lognormal(0, 1.5, (3, 1))).astype(np.float32)
    extra = [dict(kind="random", codec="-", ch=-1, detail="-", x=x[i]) for i in range(3)]
    saved = ROWS
    ROWS = saved + extra
    try:
        for codec in ("q8_0", "q4_0", "rot4", "rot3"):
            check_reference(codec, range(len(saved), len(ROWS)))
    finally:
        ROWS = saved
        for key in [k for k in _REF_CACHE if k[1] >= len(saved)]:
            del _REF_CACHE[key]


# ------------------------------------------ planted mistakes (in the oracle)
def test_planted_tie_rule_toward_zero_is_caught(monkeypatch):
    """Counting thresholds with >= sends negative ties toward zero."""
    monkeypatch.setattr(codecs, "level_index",
                        lambda t, thr: (np.asarray(t, np.float32)[..., None] >= thr).sum(-1))
    for codec in ("rot4", "rot3"):
        with pytest.raises(AssertionError):
            check_ties(_of("tie", codec))


def test_planted_strict_count_is_caught(monkeypatch):
    """Counting only thresholds strictly below sends positive ties toward zero."""
    monkeypatch.setattr(codecs, "level_index",
                        lambda t, thr: (np.asarray(t, np.float32)[..., None] > thr).sum(-1))
    for codec in ("rot4", "rot3"):
        with pytest.raises(AssertionError):
            check_ties(_of("tie", codec))


def _q8_by_division(x):
    xb = np.asarray(x, np.float32).reshape(-1, 4, 32)
    d = (np.abs(xb).max(-1) / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        prod = np.where(d[..., None] != 0, xb / d[..., None], 0).astype(np.float32)
    return {"codes": np.clip(fp.rhaz(prod), -127, 127).astype(np.int8).reshape(-1, D), "scales": fp.f16_bits(d)}


def _q4_by_division(x):
    xb = np.asarray(x, np.float32).reshape(-1, 4, 32)
    a = np.abs(xb)
    m = np.take_along_axis(xb, np.argmax(a, -1)[..., None], -1)[..., 0]
    d = np.where(a.max(-1) == 0, np.float32(0), (m / np.float32(-8)).astype(np.float32)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        prod = np.where(d[..., None] != 0, xb / d[..., None], 0).astype(np.float32)
    return {"codes": np.clip(fp.rhaz(prod) + 8, 0, 15).astype(np.uint8).reshape(-1, D), "scales": fp.f16_bits(d)}


@pytest.mark.parametrize("codec,mutant", [("q8_0", _q8_by_division), ("q4_0", _q4_by_division)])
def test_planted_division_instead_of_reciprocal_is_caught(codec, mutant):
    with pytest.raises(AssertionError):
        check_recip(_of("recip", codec), mutant)


def _wht_reversed(x, dtype=np.float32):
    w = np.array(x, dtype=dtype, copy=True)
    n = w.shape[-1]
    lead = w.shape[:-1]
    h = n // 2
    while h >= 1:
        v = w.reshape(lead + (n // (2 * h), 2, h))
        a, b = v[..., 0, :].copy(), v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        w = v.reshape(lead + (n,))
        h //= 2
    return w


def _np_sum_at(length):
    real = fp.tree_sum

    def mixed(v):
        v = np.asarray(v, np.float32)
        return np.sum(v, axis=-1, dtype=np.float32) if v.shape[-1] == length else real(v)

    return mixed


@pytest.mark.parametrize("codec", ["rot4", "rot3"])
def test_planted_reversed_wht_stage_order_is_caught(codec, monkeypatch):
    monkeypatch.setattr(codecs, "wht", _wht_reversed)
    idx = [i for i, r in enumerate(ROWS) if r["kind"] == "order" and r["codec"] == codec]
    with pytest.raises(AssertionError):
        check_reference(codec, idx)


def test_planted_pairwise_norm_sum_is_caught(monkeypatch):
    monkeypatch.setattr(codecs, "tree_sum", _np_sum_at(128))
    idx = [i for i, r in enumerate(ROWS) if r["kind"] == "order" and r["codec"] == "rot4"]
    with pytest.raises(AssertionError):
        check_reference("rot4", idx)


@pytest.mark.parametrize("codec", ["rot4", "rot3"])
def test_planted_pairwise_block_sum_is_caught(codec, monkeypatch):
    monkeypatch.setattr(codecs, "tree_sum", _np_sum_at(32))
    idx = [i for i, r in enumerate(ROWS) if r["kind"] == "order" and r["codec"] == codec]
    with pytest.raises(AssertionError):
        check_reference(codec, idx)
