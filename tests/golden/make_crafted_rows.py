"""Write tests/golden/crafted_rows.txt: encoder input rows on which a rounding
rule or an operation order decides a stored field.

    python tests/golden/make_crafted_rows.py

Calls only ``oracle/`` (and numpy).  The rows are inputs; no stored value here
is an expected output -- the tests derive those independently.  Three kinds:

tie    rot4 / rot3 rows whose whitened fp32 value t at one channel lands
       exactly on a nonzero threshold (the midpoint of two adjacent levels), at
       both signs, so the stored index is decided by the tie rule (the level
       farther from zero).  Found by solving for one input coordinate with a
       secant step, then scanning its fp32 neighbours for an exact hit.
recip  q8_0 / q4_0 blocks holding one element x for which rounding
       x * (1/d) and rounding x / d give different codes, so the stored code is
       decided by the reciprocal rule (codes from the fp32 reciprocal).
order  rot4 / rot3 rows on which a plausible change of operation order moves a
       stored field: the WHT stages run h = 64 .. 1 instead of 1 .. 64, the row
       norm or the block mean square summed by numpy's pairwise ``np.sum``
       instead of the stride-halving tree.  Found by a seeded random search
       that swaps that one step of the oracle and compares the stored fields.

All rotated rows use the one sign mask written in the file's header.
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import codecs, fp  # noqa: E402
from oracle.lloyd_max import codebook  # noqa: E402

OUT = os.path.join(HERE, "crafted_rows.txt")
D = 128
SIGNS = np.random.default_rng(20261202).integers(0, 256, 16, dtype=np.uint8)


def _hex_row(x):
    return " ".join(f"{int(v):08x}" for v in np.asarray(x, np.float32).view(np.uint32))


# ---------------------------------------------------------------- tie rows
def _whitened(codec, X):
    if codec == "rot4":
        t, _, _ = codecs.whiten_rot4(X, SIGNS)
    else:
        t, _ = codecs.whiten_rot3(X, SIGNS)
    return t.reshape(-1, D)


def find_tie(codec, k, rng):
    """A row whose whitened value at some channel equals threshold k exactly."""
    _, thr, _ = codebook(16 if codec == "rot4" else 8)
    target = np.float32(thr[k])
    for _ in range(400):
        x = rng.standard_normal(D).astype(np.float32)
        t = _whitened(codec, x[None])[0]
        j = int(np.argmin(np.abs(t.astype(np.float64) - float(target))))
        i = int(np.argmax(np.abs(x) * (np.abs(x) < 1.5)))  # a coordinate of moderate size

        def f(xi):
            y = x.copy()
            y[i] = np.float32(xi)
            return float(_whitened(codec, y[None])[0, j]) - float(target)

        a, b = float(x[i]), float(x[i]) + 0.01
        fa, fb = f(a), f(b)
        for _ in range(30):  # secant steps toward the threshold
            if fb == fa:
                break
            a, b, fa = b, b - fb * (b - a) / (fb - fa), fb
            fb = f(b)
            if abs(fb) < 1e-6:
                break
        if not np.isfinite(b) or abs(fb) > 1e-4 or np.sign(b) != np.sign(x[i]):
            continue
        base = np.array([b], np.float32).view(np.int32)[0]
        steps = np.arange(-4096, 4097, dtype=np.int64)
        cand = (base + steps).astype(np.int32).view(np.float32)
        X = np.repeat(x[None], len(cand), 0)
        X[:, i] = cand
        hit = np.nonzero(_whitened(codec, X)[:, j] == target)[0]
        if hit.size:
            return X[hit[len(hit) // 2]], j
    raise RuntimeError(f"no tie row found for {codec} threshold {k}")


# -------------------------------------------------------------- recip rows
def _rhaz(v):
    return fp.rhaz(np.asarray(v, np.float32))


def find_recip(codec, rng, negative):
    """A block (channels 0..31 of a row) with one element whose code differs
    between x * (1/d) and x / d."""
    for _ in range(20000):
        if codec == "q8_0":
            amax = np.float32(rng.uniform(0.5, 50.0))
            d = np.float32(amax / np.float32(127.0))
            lo, hi = 1, 126
            lead = amax
        else:
            amax = np.float32(rng.uniform(0.5, 50.0))
            lead = amax  # positive first maximum: d = m / -8 < 0
            d = np.float32(lead / np.float32(-8.0))
            lo, hi = 0, 7
        inv = np.float32(np.float32(1.0) / d)
        kk = int(rng.integers(lo, hi + 1))
        half = (kk + 0.5) * (-1.0 if negative else 1.0)
        x0 = np.float32(half * float(d))
        base = np.array([x0], np.float32).view(np.int32)[0]
        cand = (base + np.arange(-64, 65)).astype(np.int32).view(np.float32)
        cand = cand[np.abs(cand) < amax]
        a = _rhaz((cand * inv).astype(np.float32))
        b = _rhaz((cand / d).astype(np.float32))
        diff = np.nonzero(a != b)[0]
        if diff.size:
            x = np.zeros(D, np.float32)
            x[0] = lead
            x[1] = cand[diff[0]]
            x[2:32] = (rng.standard_normal(30) * 0.25 * amax).astype(np.float32)
            x[2:32] = np.clip(x[2:32], -0.9 * amax, 0.9 * amax)
            x[32:] = rng.standard_normal(96).astype(np.float32)
            return x, 1
    raise RuntimeError(f"no reciprocal row found for {codec}")


# -------------------------------------------------------------- order rows
def _wht_reversed(x, dtype=np.float32):
    w = np.array(x, dtype=dtype, copy=True)
    n = w.shape[-1]
    lead = w.shape[:-1]
    h = n // 2
    while h >= 1:
        v = w.reshape(lead + (n // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        w = v.reshape(lead + (n,))
        h //= 2
    return w


def _np_sum_for(length):
    real = fp.tree_sum

    def mixed(v):
        v = np.asarray(v, np.float32)
        if v.shape[-1] == length:
            return np.sum(v, axis=-1, dtype=np.float32)
        return real(v)

    return mixed


MUTANTS = {
    "wht_reversed": ("wht", _wht_reversed),
    "norm_np_sum": ("tree_sum", _np_sum_for(128)),
    "block_np_sum": ("tree_sum", _np_sum_for(32)),
}


def _fields(q):
    return np.concatenate([q[k].reshape(len(q["codes"]), -1).astype(np.int64) for k in sorted(q)], axis=1)


def find_order(codec, mutant, rng, want=2):
    name, fn = MUTANTS[mutant]
    found = []
    for _ in range(20):
        X = (rng.standard_normal((50000, D)) * rng.lognormal(0, 1.0, (50000, 1))).astype(np.float32)
        good = _fields(codecs.quantize(codec, X, SIGNS))
        saved = getattr(codecs, name)
        setattr(codecs, name, fn)
        try:
            bad = _fields(codecs.quantize(codec, X, SIGNS))
        finally:
            setattr(codecs, name, saved)
        rows = np.nonzero(np.any(good != bad, axis=1))[0]
        for r in rows[:want - len(found)]:
            found.append(X[r])
        if len(found) >= want:
            return found
    raise RuntimeError(f"no {mutant} row found for {codec}")


def main():
    rng = np.random.default_rng(0xC0FFEE)
    lines = [
        "# Crafted encoder input rows (fp32 bit patterns, 128 per row), written by",
        "# tests/golden/make_crafted_rows.py, which calls only oracle/.  Inputs only:",
        "# the tests derive every expected value themselves.",
        f"# signs {''.join(f'{b:02x}' for b in SIGNS)}",
        "# kind codec channel detail : row",
    ]
    for codec, ks in (("rot4", [0, 2, 5, 6, 8, 9, 12, 14]), ("rot3", [0, 1, 2, 4, 5, 6])):
        for k in ks:
            x, j = find_tie(codec, k, rng)
            lines.append(f"tie {codec} {j} thr{k} : {_hex_row(x)}")
    for codec in ("q8_0", "q4_0"):
        for neg in (False, True):
            x, j = find_recip(codec, rng, neg)
            lines.append(f"recip {codec} {j} {'neg' if neg else 'pos'} : {_hex_row(x)}")
    for codec, muts in (("rot4", ["wht_reversed", "norm_np_sum", "block_np_sum"]),
                        ("rot3", ["wht_reversed", "block_np_sum"])):
        for m in muts:
            for x in find_order(codec, m, rng):
                lines.append(f"order {codec} -1 {m} : {_hex_row(x)}")
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {OUT} ({len(lines) - 5} rows)")


if __name__ == "__main__":
    main()
