"""Pins of oracle/probe.py (attention-probe cell scoring and eviction choice;
Randozart/VITRIOL page, "How It Works -- Resident mode").  CPU only."""

import math

import numpy as np
import pytest

from oracle import attention, probe

D = 128
SCALE = 1.0 / math.sqrt(D)


def _rows(seed, n):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D)).astype(np.float32)
    x[:, rng.choice(D, 2, replace=False)] *= 10.0
    return x


def test_probe_mass_bruteforce_tiny():
    # fp16-exact keys in an f16 plane: the dequantized keys are the keys
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, D))
    k = rng.standard_normal((5, D)).astype(np.float16).astype(np.float32)
    got = probe.probe_mass(q, k, "f16", SCALE)
    expect = [0.0] * 5
    for g in range(3):
        logits = [SCALE * sum(float(q[g, c]) * float(k[j, c]) for c in range(D)) for j in range(5)]
        e = [math.exp(x - max(logits)) for x in logits]
        for j in range(5):
            expect[j] += e[j] / sum(e)
    assert np.allclose(got, expect, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("codec", ["f16", "q8_0", "q4_0", "rot4", "rot3"])
def test_probe_mass_sums_to_the_query_heads(codec):
    signs = np.full(16, 0x5A, dtype=np.uint8) if codec in ("rot4", "rot3") else None
    m = probe.probe_mass(_rows(2, 4) * 0.5, _rows(3, 300), codec, SCALE, signs)
    assert m.shape == (300,) and np.all(m > 0)
    assert m.sum() == pytest.approx(4.0, rel=1e-12)


def test_probe_mass_special_cases():
    k = np.tile(_rows(4, 1), (7, 1))
    assert np.allclose(probe.probe_mass(_rows(5, 2), k, "q8_0", SCALE), 2.0 / 7.0)  # identical keys
    assert np.allclose(probe.probe_mass(np.zeros((3, D)), _rows(6, 9), "q4_0", SCALE), 3.0 / 9.0)  # q = 0
    q = _rows(7, 2).astype(np.float64)
    k = _rows(8, 20) * 0.01
    k[13] = (q[0] + q[1]).astype(np.float32) * 4.0  # a key aligned with both queries
    m = probe.probe_mass(q, k, "f16", SCALE)
    assert m[13] > 2.0 - 1e-6


def test_probe_mass_is_the_decode_weighting():
    # sum over heads of decode outputs = mass . V (same softmax weights)
    q, k, v = _rows(9, 4) * 0.3, _rows(10, 150), _rows(11, 150)
    m = probe.probe_mass(q, k, "q8_0", SCALE)
    out = attention.decode_reference(q, k, v, "q8_0", "f16", SCALE)
    vd = v.astype(np.float16).astype(np.float64)
    assert np.allclose(out.sum(axis=0), m @ vd, rtol=1e-10, atol=1e-10)


def test_cell_mass_sums_over_kv_heads():
    q = _rows(13, 6) * 0.2            # 6 query heads on 3 KV heads (G = 2)
    k = np.stack([_rows(14 + h, 40) for h in range(3)])
    m = probe.cell_mass(q, k, "q4_0", SCALE)
    assert m.sum() == pytest.approx(6.0, rel=1e-12)
    per_head = [probe.probe_mass(q[2 * h:2 * h + 2], k[h], "q4_0", SCALE) for h in range(3)]
    assert np.allclose(m, per_head[0] + per_head[1] + per_head[2], rtol=0, atol=0)


def test_decay_update_closed_form():
    prev0 = np.array([0.5, 2.0, 0.0])
    mass = np.array([0.25, 0.0, 1.0])
    d = 0.75
    s = prev0
    for _ in range(6):
        s = probe.decay_update(s, mass, d)
    expect = d ** 6 * prev0 + mass * (1 - d ** 6) / (1 - d)
    assert np.allclose(s, expect, rtol=1e-14)


def test_select_evictions_properties():
    rng = np.random.default_rng(12)
    for trial in range(200):
        L = int(rng.integers(0, 60))
        scores = rng.integers(0, 6, max(L, 1)).astype(np.float64)  # many ties
        ns, nr, ne = (int(x) for x in rng.integers(0, 12, 3))
        got = probe.select_evictions(scores, L, ns, nr, ne)
        lo, hi = min(ns, L), max(min(ns, L), L - nr)
        middle = list(range(lo, hi))
        assert got == sorted(got) and len(set(got)) == len(got)
        assert len(got) == min(ne, len(middle))
        assert all(lo <= j < hi for j in got)  # sinks and recent cells are never chosen
        rest = [j for j in middle if j not in got]
        for j in got:
            for r in rest:  # every chosen cell precedes every kept one in (score, cell) order
                assert (scores[j], j) < (scores[r], r)


def test_select_evictions_ties_and_edges():
    s = np.zeros(20)
    assert probe.select_evictions(s, 20, 4, 4, 5) == [4, 5, 6, 7, 8]     # equal scores: lowest cells first
    assert probe.select_evictions(s, 20, 12, 9, 5) == []                 # sinks and recent cover everything
    assert probe.select_evictions(s, 20, 0, 0, 0) == []
    assert probe.select_evictions(s, 20, 2, 3, 100) == list(range(2, 17))
    s2 = np.array([5.0, 1.0, 3.0, 1.0, 0.5, 9.0])
    assert probe.select_evictions(s2, 6, 1, 1, 3) == [1, 3, 4]
