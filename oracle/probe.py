"""Attention-probe cell scoring for sparse KV eviction, and the choice of the
cells to evict.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the Randozart/VITRIOL page -- "What sets VITRIOL apart" table
(sparse eviction driven by an attention probe that ranks the cache cells;
the first and the latest cells are kept), "Configuration" table
(score=probe, score_every=16) and "How It Works -- Resident mode" (a probe
graph of a q.K softmax with exponential decay runs every 16 steps; the
lowest-scored middle cells are evicted first; sinks and recent cells are
protected; draft tokens are excluded from probe scoring).

Readings (the page prints no formula):

* A scoring event takes the current token's query rows (the n_q_heads query
  heads of one sequence; no draft tokens) and, per query head, the softmax of
  scale * q . k over its KV head's cells 0 .. L-1, exactly as in decode
  attention.  A cell is a token position (it holds every KV head), so its
  mass is the sum of its probabilities over all n_q_heads query heads (the
  masses of one sequence sum to n_q_heads).
* Exponential decay: score <- decay * score + mass, applied per scoring event
  (scores of cells at or past L are not touched).  The event cadence (every
  16 steps) is the caller's.
* Eviction: among the middle cells n_sink <= j < L - n_recent, the n_evict
  lowest scores go first; equal scores go in increasing cell order, so the
  chosen set is unique.  It is returned in increasing cell order.
"""

import numpy as np

from . import codecs


def probe_mass(q_rows, k_rows, k_codec, scale, k_signs=None):
    """Mass per cell [L] (fp64): sum over the G query rows q_rows [G, 128] of
    softmax_j(scale * q . k_j) over the oracle's own dequantization of the
    fp32 key rows k_rows [L, 128]."""
    kd = codecs.dequant(k_codec, codecs.quantize(k_codec, k_rows, k_signs), k_signs)
    s = scale * (np.asarray(q_rows, dtype=np.float64) @ kd.T)  # [G, L]
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


def cell_mass(q_rows, k_rows, k_codec, scale, k_signs=None):
    """Mass per cell [L] of one sequence: q_rows [Hq, 128] (query head h uses
    KV head h // G), k_rows [Hkv, L, 128]; the sum over the KV heads of
    probe_mass of their G query rows."""
    hkv = len(k_rows)
    g = len(q_rows) // hkv
    return sum(probe_mass(q_rows[h * g:(h + 1) * g], k_rows[h], k_codec, scale, k_signs) for h in range(hkv))


def decay_update(prev, mass, decay):
    """One scoring event: decay * prev + mass."""
    return decay * np.asarray(prev, dtype=np.float64) + mass


def select_evictions(scores, seq_len, n_sink, n_recent, n_evict):
    """The cells to evict, in increasing order: the n_evict lowest (score,
    cell) pairs among cells n_sink .. seq_len - n_recent - 1."""
    lo = min(n_sink, seq_len)
    hi = max(lo, seq_len - n_recent)
    middle = list(range(lo, hi))
    chosen = sorted(middle, key=lambda j: (scores[j], j))[:max(0, n_evict)]
    return sorted(chosen)
