"""Seeded synthetic inputs for the quantized-KV decode path.

This module is the only code that both the oracle side (tests, bench's CPU
baseline) and the HIP side (tests, bench, smoke) use.  It draws random
numbers and shapes them into the workloads' distributions; it holds none of
the codec or attention arithmetic.

Every array is addressable without generating the rest: each (config, kind,
layer, seq, head, chunk) has its own PCG64 stream seeded through
``numpy.random.SeedSequence(BASE_SEED, spawn_key=...)``, with chunks of 4096
positions, so any slice of any (sequence, head) can be regenerated anywhere.

Workloads (one per entry of ``CONFIGS``):
  1 tiny     1 layer, 1 seq, Hq 4 / Hkv 1, L 512, K f16 / V q8_0; K, V, Q ~ N(0,1)
             with 2 seeded outlier channels per (tensor, head) scaled x20.
  2 batched  8 seqs x 1 new token, Hq 32 / Hkv 8, L 8192, q8_0 / q8_0; N(0,1) times
             a per-(tensor, head, channel) log-normal scale exp(1.0 * N(0,1)).
  3 lowbit   4 seqs, Hq 40 / Hkv 8, L 32768, q4_0 / q4_0; N(0,1) where each entry
             is replaced with probability 0.01 by a Student-t(3) draw.
  4 rotated  1 seq, Hq 16 / Hkv 2, L 131072, rot4 / rot4; N(0,1) with 2 outlier
             channels x20 per (tensor, head); one random sign mask per side.
  5 ladder   16 layers, 2 seqs, capacity 200704, Hq 32 / Hkv 8; per (layer, side)
             a codec from a seeded balanced permutation of 8 x {f16, q8_0, rot4,
             q4_0}; data as workload 2; rows 0..198655 pre-filled, each step
             re-appends a 2048-row ubatch (rows 198656..200703) then decodes one
             token per sequence over all 200704 rows.
The pages measure on a public text corpus through real models; none of that is
here, and these synthetic K/V/Q of the same shapes and head structure (GQA,
outlier channels, heavy tails) stand in for it.
"""

import numpy as np

BASE_SEED = 0x5EED2026
CHUNK = 4096
HEAD_DIM = 128

KIND_K, KIND_V, KIND_Q, KIND_SIGNS, KIND_CODECMAP, KIND_OUTLIER, KIND_SCALES, KIND_MASK = range(8)
SIDE_KIND = {"k": KIND_K, "v": KIND_V}

CONFIGS = {
    "tiny": dict(name="tiny", layers=1, seqs=1, hq=4, hkv=1, ctx=512, capacity=512,
            k_codec="f16", v_codec="q8_0", dist="outlier", fused_append=False),
    "batched": dict(name="batched", layers=1, seqs=8, hq=32, hkv=8, ctx=8192, capacity=8192,
            k_codec="q8_0", v_codec="q8_0", dist="lognormal", fused_append=True),
    "lowbit": dict(name="lowbit", layers=1, seqs=4, hq=40, hkv=8, ctx=32768, capacity=32768,
            k_codec="q4_0", v_codec="q4_0", dist="heavy", fused_append=False),
    "rotated": dict(name="rotated", layers=1, seqs=1, hq=16, hkv=2, ctx=131072, capacity=131072,
            k_codec="rot4", v_codec="rot4", dist="outlier", fused_append=False),
    "ladder": dict(name="ladder", layers=16, seqs=2, hq=32, hkv=8, ctx=200704, capacity=200704,
            k_codec=None, v_codec=None, dist="lognormal", fused_append=False,
            prefill=198656, ubatch=2048),
}

# each workload's number in the seed derivation (fixes every generated value)
SEED_ID = {"tiny": 1, "batched": 2, "lowbit": 3, "rotated": 4, "ladder": 5}

LADDER_CODECS = ("f16", "q8_0", "rot4", "q4_0")


def rng(cfg, kind, layer, seq, head, chunk):
    """The PCG64 generator of one (config, kind, layer, seq, head, chunk)."""
    ss = np.random.SeedSequence(BASE_SEED, spawn_key=(SEED_ID[cfg], kind, layer, seq, head, chunk))
    return np.random.Generator(np.random.PCG64(ss))


def outlier_channels(cfg, kind, layer, head, count=2):
    """The seeded outlier channels of one (tensor kind, layer, head)."""
    g = rng(cfg, KIND_OUTLIER, layer, kind, head, 0)
    return np.sort(g.choice(HEAD_DIM, size=count, replace=False))


def channel_scales(cfg, kind, layer, head, sigma=1.0):
    """Per-channel log-normal scales exp(sigma * N(0,1)) of one (kind, layer, head)."""
    g = rng(cfg, KIND_SCALES, layer, kind, head, 0)
    return np.exp(sigma * g.standard_normal(HEAD_DIM)).astype(np.float32)


def _shape(cfg, kind, layer, head, x):
    dist = CONFIGS[cfg]["dist"]
    if dist == "outlier":
        ch = outlier_channels(cfg, kind, layer, head)
        x[..., ch] *= np.float32(20.0)
    elif dist == "lognormal":
        x *= channel_scales(cfg, kind, layer, head)
    return x


def _chunk(cfg, kind, layer, seq, head, chunk):
    g = rng(cfg, kind, layer, seq, head, chunk)
    x = g.standard_normal((CHUNK, HEAD_DIM)).astype(np.float32)
    if CONFIGS[cfg]["dist"] == "heavy":
        hit = g.random((CHUNK, HEAD_DIM)) < 0.01
        x[hit] = g.standard_t(3.0, size=int(hit.sum())).astype(np.float32)
    return _shape(cfg, kind, layer, head, x)


def kv_rows(cfg, side, layer, seq, head, start, count):
    """fp32 [count, 128] rows start..start+count-1 of one (side, layer, seq, KV head)."""
    kind = SIDE_KIND[side]
    out = np.empty((count, HEAD_DIM), dtype=np.float32)
    pos = start
    end = start + count
    while pos < end:
        c = pos // CHUNK
        lo = pos - c * CHUNK
        n = min(CHUNK - lo, end - pos)
        out[pos - start:pos - start + n] = _chunk(cfg, kind, layer, seq, head, c)[lo:lo + n]
        pos += n
    return out


def q_rows(cfg, layer, seq, n_q_heads):
    """fp32 [Hq, 128] query rows of one (layer, seq) (the decoded token)."""
    out = np.empty((n_q_heads, HEAD_DIM), dtype=np.float32)
    for h in range(n_q_heads):
        x = rng(cfg, KIND_Q, layer, seq, h, 0).standard_normal((1, HEAD_DIM)).astype(np.float32)
        out[h] = _shape(cfg, KIND_Q, layer, h, x)[0]
    return out


def sign_mask(cfg, layer, side):
    """16 random bytes: the rot4 sign mask of one (layer, side)."""
    g = rng(cfg, KIND_SIGNS, layer, SIDE_KIND[side], 0, 0)
    return g.integers(0, 256, size=16, dtype=np.uint8)


def codec_map(cfg):
    """[(k_codec, v_codec)] per layer.  Workload 5 draws a balanced permutation
    (8 of each codec over the 32 (layer, side) slots)."""
    c = CONFIGS[cfg]
    if c["k_codec"] is not None:
        return [(c["k_codec"], c["v_codec"])] * c["layers"]
    slots = np.repeat(np.arange(len(LADDER_CODECS)), 2 * c["layers"] // len(LADDER_CODECS))
    perm = rng(cfg, KIND_CODECMAP, 0, 0, 0, 0).permutation(slots)
    return [(LADDER_CODECS[perm[2 * i]], LADDER_CODECS[perm[2 * i + 1]]) for i in range(c["layers"])]


def poison_pattern(nbytes, seed=0):
    """Bytes used to fill buffers that must not be read (0xFF and NaN-like runs)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(BASE_SEED, spawn_key=(99, seed))))
    b = g.integers(0, 256, size=nbytes, dtype=np.uint8)
    b[::2] = 0xFF
    return b
