"""Decode attention in fp64, straight from its definition.

One query token per sequence attends to every cached row 0..L-1 of its KV
head (flash attention is the only attention path for typed KV on the
buun-llama-cpp page, "Requirements" paragraph under "Recommended usage"; the
result it computes is plain softmax attention).  Readings: scale 1/sqrt(128)
unless given, no mask beyond the length, no positional terms (K arrives
post-RoPE), grouped-query mapping kv_head = q_head // G.
"""

import numpy as np

from . import codecs


def attend(q, k, v, scale):
    """o = softmax(scale * q k^T) v for q [G,D], k [L,D], v [L,D]; fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scale * (q @ k.T)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ v


def attend_bruteforce(q, k, v, scale):
    """The same definition with explicit Python loops (for tiny inputs only)."""
    import math

    G, Dq = len(q), len(q[0])
    L = len(k)
    out = np.zeros((G, len(v[0])))
    for g in range(G):
        s = [scale * sum(float(q[g][c]) * float(k[i][c]) for c in range(Dq)) for i in range(L)]
        mx = max(s)
        e = [math.exp(si - mx) for si in s]
        tot = sum(e)
        for i in range(L):
            for c in range(len(v[0])):
                out[g, c] += e[i] / tot * float(v[i][c])
    return out


def partial(q, k, v, scale):
    """Unnormalised split partial over some rows: (sum_i e^{s_i - m} v_i, m, l).

    An empty row set gives (0, -inf, 0)."""
    q = np.asarray(q, dtype=np.float64)
    G = q.shape[0]
    if len(k) == 0:
        return np.zeros((G, np.shape(v)[1] if np.ndim(v) == 2 else q.shape[1])), np.full(G, -np.inf), np.zeros(G)
    s = scale * (q @ np.asarray(k, dtype=np.float64).T)
    m = s.max(axis=-1)
    e = np.exp(s - m[:, None])
    return e @ np.asarray(v, dtype=np.float64), m, e.sum(axis=-1)


def merge(parts):
    """Merge split partials: M = max m_s, L = sum l_s e^{m_s-M},
    O = sum o_s e^{m_s-M} / L.  Empty partials (l = 0) are skipped."""
    ms = np.stack([p[1] for p in parts])
    M = np.max(ms, axis=0)
    O = 0.0
    L = 0.0
    for o, m, l in parts:
        w = np.where(l > 0, np.exp(np.where(l > 0, m - M, 0.0)), 0.0)
        O = O + o * w[:, None]
        L = L + l * w
    return O / L[:, None]


def decode_reference(q_rows, k_rows, v_rows, k_codec, v_codec, scale,
                     k_signs=None, v_signs=None):
    """Full reference for one (sequence, KV head): quantize every K/V row with
    the oracle encoders, dequantize to the model domain in fp64, then attend.

    q_rows [G,128] fp32; k_rows, v_rows [L,128] fp32.  Returns fp64 [G,128].
    """
    kq = codecs.quantize(k_codec, k_rows, k_signs)
    vq = codecs.quantize(v_codec, v_rows, v_signs)
    kd = codecs.dequant(k_codec, kq, k_signs)
    vd = codecs.dequant(v_codec, vq, v_signs)
    return attend(q_rows, kd, vd, scale)


def decode_multi_reference(q_rows, k_rows, v_rows, k_codec, v_codec, scale,
                           k_signs=None, v_signs=None):
    """T new query tokens of one (sequence, KV head) at once, causal among
    themselves, as when a drafted run of tokens is verified in one pass
    (Randozart/VITRIOL page: "How It Works -- Resident mode" has the MTP head
    draft ahead with parallel verification; "Configuration" runs up to 3
    drafted tokens).  Reading: token t (0-based among the T) attends the
    cached rows and the new rows up to and including its own, i.e. rows
    0 .. L - T + t of k_rows / v_rows, which end with the T new rows.

    q_rows [T,G,128] fp32; k_rows, v_rows [L,128] fp32 (L >= T).  Returns
    fp64 [T,G,128].
    """
    T, L = len(q_rows), len(k_rows)
    if not 1 <= T <= L:
        raise ValueError("need 1 <= T <= L")
    kq = codecs.quantize(k_codec, k_rows, k_signs)
    vq = codecs.quantize(v_codec, v_rows, v_signs)
    kd = codecs.dequant(k_codec, kq, k_signs)
    vd = codecs.dequant(v_codec, vq, v_signs)
    return np.stack([attend(q_rows[t], kd[:L - T + 1 + t], vd[:L - T + 1 + t], scale) for t in range(T)])
