"""Pins of the oracle's WHT, Lloyd-Max solve, attention and byte model (CPU only)."""

import math
import os

import numpy as np
import pytest

from oracle import attention, bytes_model, codecs, fp, lloyd_max, wht

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden(name):
    rows = []
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------- WHT
def test_sylvester_orthogonality():
    H = wht.sylvester(128)
    assert np.array_equal(H @ H.T, 128 * np.eye(128, dtype=np.int64))
    assert np.array_equal(H, H.T)


def test_wht_of_unit_vectors_is_sylvester_rows():
    H = wht.sylvester(128)
    E = np.eye(128, dtype=np.float32)
    assert np.array_equal(wht.wht(E, np.float32), H.astype(np.float32))


def test_wht_matches_matrix_and_involution_on_integers(rng):
    x = rng.integers(-50, 50, (9, 128)).astype(np.float32)
    H = wht.sylvester(128)
    assert np.array_equal(wht.wht(x, np.float32), (x.astype(np.int64) @ H.T).astype(np.float32))
    assert np.array_equal(wht.wht(wht.wht(x, np.float32), np.float32), 128 * x)


def test_wht_parseval_fp32(rng):
    x = rng.standard_normal((100, 128)).astype(np.float32)
    w = wht.wht(x, np.float32).astype(np.float64)
    assert np.allclose((w * w).sum(1), 128 * (x.astype(np.float64) ** 2).sum(1), rtol=1e-5)


def test_rotation_preserves_dot_products(rng):
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    s = wht.sign_vector(rng.integers(0, 256, 16, dtype=np.uint8)).astype(np.float64)
    qt = wht.wht(s * q, np.float64) / math.sqrt(128)
    kt = wht.wht(s * k, np.float64) / math.sqrt(128)
    assert abs(qt @ kt - q @ k) < 1e-12


def test_sign_mask_bit_order():
    m = np.zeros(16, np.uint8)
    m[0] = 0b00000101  # channels 0 and 2
    m[15] = 0b10000000  # channel 127
    s = wht.sign_vector(m)
    assert s[0] == -1 and s[1] == 1 and s[2] == -1 and s[127] == -1 and s.sum() == 128 - 6


# --------------------------------------------------------------- Lloyd-Max
@pytest.mark.parametrize("n_levels", [16, 8])
def test_lloyd_max_matches_max_1960_table(n_levels):
    lv, thr, _ = lloyd_max.solve_positive_half(n_levels)
    for kind, k, sval in _golden(f"max1960_gaussian_{n_levels}level.txt"):
        k, val = int(k), float(sval)
        # the table is rounded to its last printed digit (3 or 4 decimals)
        tol = 0.5 * 10.0 ** -len(sval.split(".")[1]) + 1e-4
        if kind == "level":
            assert abs(lv[k] - val) <= tol, (k, lv[k], val)
        elif kind == "thresh":
            assert abs(thr[k] - val) <= tol, (k, thr[k], val)
        else:
            full = np.concatenate([-lv[::-1], lv])
            ths = np.concatenate([-thr[::-1], [0.0], thr])
            assert abs(lloyd_max.mse_fp64(full, ths) - val) <= 1e-5


@pytest.mark.parametrize("n_levels", [16, 8])
def test_lloyd_max_optimality_by_independent_integration(n_levels):
    """Centroid and midpoint conditions, checked with scipy's adaptive
    quadrature (independent of the closed forms the solver uses)."""
    from scipy import integrate
    from scipy.stats import norm

    lv, thr, _ = lloyd_max.solve_positive_half(n_levels)
    edges = [0.0] + list(thr) + [np.inf]
    for i, y in enumerate(lv):
        a, b = edges[i], edges[i + 1]
        m0 = integrate.quad(norm.pdf, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        m1 = integrate.quad(lambda x: x * norm.pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(m1 / m0 - y) < 1e-9
    for i, t in enumerate(thr):
        assert abs(t - 0.5 * (lv[i] + lv[i + 1])) < 1e-15
    full = np.concatenate([-lv[::-1], lv])
    ths = np.concatenate([-thr[::-1], [0.0], thr])
    mse_q = 0.0
    e = [-np.inf] + list(ths) + [np.inf]
    for k, y in enumerate(full):
        mse_q += integrate.quad(lambda x: (x - y) ** 2 * norm.pdf(x), e[k], e[k + 1],
                                epsabs=1e-14, epsrel=1e-12)[0]
    assert abs(mse_q - lloyd_max.mse_fp64(full, ths)) < 1e-10
    # SNR of the Gaussian Lloyd-Max quantizer: 20.22 dB at 16 levels, 14.62 dB at 8
    assert abs(10 * math.log10(1 / mse_q) - {16: 20.22, 8: 14.62}[n_levels]) < 0.01


def test_lloyd_max_is_a_local_minimum():
    lv, thr, _ = lloyd_max.solve_positive_half()
    full = np.concatenate([-lv[::-1], lv])
    ths = np.concatenate([-thr[::-1], [0.0], thr])
    base = lloyd_max.mse_fp64(full, ths)
    for k in range(16):
        for dlt in (1e-3, -1e-3):
            f2 = full.copy()
            f2[k] += dlt
            assert lloyd_max.mse_fp64(f2, ths) > base


def test_stored_codebook_fp16_and_midpoints():
    lv16, thr, bits = lloyd_max.codebook()
    full = lloyd_max.full_levels_fp64()
    # stored levels are the RNE fp16 roundings of the fp64 levels
    assert np.array_equal(bits, np.array(full).astype(np.float16).view(np.uint16))
    assert np.all(np.abs(lv16 - full) <= np.abs(full) * 2.0 ** -11)
    assert np.array_equal(lv16[::-1], -lv16)  # odd symmetry survives rounding
    assert thr[7] == 0.0
    assert np.array_equal(thr.astype(np.float64), (lv16[:-1].astype(np.float64) + lv16[1:]) / 2)


# -------------------------------------------------------------- attention
def test_attention_single_row_returns_value(rng):
    q = rng.standard_normal((4, 128))
    v = rng.standard_normal((1, 128))
    o = attention.attend(q, rng.standard_normal((1, 128)), v, 1 / math.sqrt(128))
    assert np.allclose(o, np.repeat(v, 4, 0), atol=1e-15)


def test_attention_uniform_cases_give_mean(rng):
    v = rng.standard_normal((37, 128))
    k = np.repeat(rng.standard_normal((1, 128)), 37, 0)
    o = attention.attend(rng.standard_normal((3, 128)), k, v, 0.1)
    assert np.allclose(o, v.mean(0), atol=1e-13)
    o = attention.attend(np.zeros((2, 128)), rng.standard_normal((37, 128)), v, 0.1)
    assert np.allclose(o, v.mean(0), atol=1e-13)


def test_attention_dominating_key(rng):
    q = rng.standard_normal((1, 128))
    k = rng.standard_normal((50, 128))
    k[17] = 50 * q[0]
    v = rng.standard_normal((50, 128))
    o = attention.attend(q, k, v, 1 / math.sqrt(128))
    assert np.allclose(o[0], v[17], atol=1e-9)


@pytest.mark.parametrize("G,L", [(1, 5), (4, 17), (8, 64)])
def test_attention_bruteforce_and_permutation(rng, G, L):
    q = rng.standard_normal((G, 8)) * 2
    k = rng.standard_normal((L, 8))
    v = rng.standard_normal((L, 8))
    o = attention.attend(q, k, v, 0.7)
    ob = attention.attend_bruteforce(q.tolist(), k.tolist(), v.tolist(), 0.7)
    assert np.allclose(o, ob, atol=1e-13)
    perm = rng.permutation(L)
    assert np.allclose(attention.attend(q, k[perm], v[perm], 0.7), o, atol=1e-13)


def test_split_merge_identity_any_partition(rng):
    q = rng.standard_normal((4, 128)) * 3
    k = rng.standard_normal((300, 128))
    v = rng.standard_normal((300, 128))
    ref = attention.attend(q, k, v, 1 / math.sqrt(128))
    for _ in range(5):
        cuts = np.sort(rng.integers(0, 301, rng.integers(1, 9)))
        bounds = [0] + cuts.tolist() + [300]
        parts = [attention.partial(q, k[a:b], v[a:b], 1 / math.sqrt(128)) for a, b in zip(bounds[:-1], bounds[1:])]
        assert np.allclose(attention.merge(parts), ref, atol=1e-12)


def test_f16_codec_attention_equals_fp64_attention_on_rounded_inputs(rng):
    q = rng.standard_normal((4, 128)).astype(np.float32)
    k = (rng.standard_normal((200, 128)) * 3).astype(np.float32)
    v = rng.standard_normal((200, 128)).astype(np.float32)
    o = attention.decode_reference(q, k, v, "f16", "f16", 1 / math.sqrt(128))
    k16 = k.astype(np.float16).astype(np.float64)
    v16 = v.astype(np.float16).astype(np.float64)
    assert np.allclose(o, attention.attend(q, k16, v16, 1 / math.sqrt(128)), atol=1e-12)
    o32 = attention.attend(q, k, v, 1 / math.sqrt(128))
    assert np.max(np.abs(o - o32)) < 5e-3 * np.sqrt(np.mean(o32 ** 2)) + 1e-3


def test_gqa_identical_queries_identical_outputs(rng):
    q = np.repeat(rng.standard_normal((1, 128)), 4, 0).astype(np.float32)
    k = rng.standard_normal((64, 128)).astype(np.float32)
    v = rng.standard_normal((64, 128)).astype(np.float32)
    o = attention.decode_reference(q, k, v, "q8_0", "q4_0", 0.088)
    assert np.array_equal(o[0], o[3])


def test_quantized_attention_tracks_fp32_attention(rng):
    q = rng.standard_normal((4, 128)).astype(np.float32)
    k = rng.standard_normal((512, 128)).astype(np.float32)
    v = rng.standard_normal((512, 128)).astype(np.float32)
    ref = attention.attend(q, k, v, 1 / math.sqrt(128))
    rms = np.sqrt(np.mean(ref ** 2))
    errs = {}
    s = rng.integers(0, 256, 16, dtype=np.uint8)
    for c in codecs.CODECS:
        o = attention.decode_reference(q, k, v, c, c, 1 / math.sqrt(128), s, s)
        errs[c] = np.max(np.abs(o - ref)) / rms
    assert errs["f16"] < errs["q8_0"] < errs["q4_0"]
    assert errs["rot4"] < 1.0


def test_rotation_helps_rows_with_outlier_channels(rng):
    """The rotated 4-bit codec spreads two x20 channels over all 128, so its
    reconstruction error is well below q4_0's at similar bits/value."""
    x = rng.standard_normal((2000, 128)).astype(np.float32)
    x[:, [9, 100]] *= 20
    s = rng.integers(0, 256, 16, dtype=np.uint8)
    rel = {}
    for c in ("q4_0", "rot4"):
        xh = codecs.dequant(c, codecs.quantize(c, x, s), s)
        rel[c] = ((xh - x) ** 2).sum() / (x.astype(np.float64) ** 2).sum()
    assert rel["rot4"] < 0.5 * rel["q4_0"]


# ------------------------------------------------------------- byte model
def test_byte_model_matches_page_figures():
    g = {row[0]: float(row[1]) for row in _golden("page_byte_figures.txt")}
    B = bytes_model.BPV
    for c in ("f16", "q8_0", "q4_0", "turbo8", "turbo4"):
        assert B[c] == g["bpv_" + c]
    assert round(100 * (1 - B["tq3_0"] / B["q4_0"])) == g["tq3_smaller_than_q4_pct"]
    # VBR: 32 equal tensors (16 layers x K,V), one then two degraded to turbo8
    agg1 = bytes_model.aggregate_bpv(["turbo8"] + ["f16"] * 31)
    agg2 = bytes_model.aggregate_bpv(["turbo8"] * 2 + ["f16"] * 30)
    assert round(agg1, 2) == g["vbr_step1_bpv"] and round(agg2, 2) == g["vbr_step2_bpv"]
    assert bytes_model.vbr_steps(16) == g["vbr_steps_16_layers"]
    assert bytes_model.vbr_steps(60) == g["vbr_steps_60_layers"]
    # per-token KV with K f16: scale a model whose f16 K half costs 16 KiB/token
    half_f16 = 16 * 1024
    kib_kf16_vq8 = (half_f16 + half_f16 * B["q8_0"] / B["f16"]) / 1024
    assert kib_kf16_vq8 == g["kf16_vq8_kib_per_token"]
    assert 2 * half_f16 / 1024 == g["kf16_vf16_kib_per_token"]
    assert round(3 * 262144 * kib_kf16_vq8 / 2 ** 20, 1) == g["three_262144_slots_gib"]
    assert 49152 * kib_kf16_vq8 / 1024 == g["pool_drop_49152_mib"]
    assert g["slot_pool_tokens"] == 2 * g["slot_tokens"] and g["slot_tokens"] % 256 == 0
    # the same accounting through the row-byte function used for the cache planes
    assert bytes_model.row_bytes("f16") == 256 and bytes_model.row_bytes("q8_0") == 136
    assert bytes_model.row_bytes("q4_0") == 72 and bytes_model.row_bytes("rot4") == 74


def test_decode_read_bytes_of_workloads():
    assert bytes_model.decode_kv_read_bytes("f16", "q8_0", 1, 1, 512) == 200704
    assert bytes_model.decode_kv_read_bytes("q8_0", "q8_0", 8, 8, 8192) == 142606336
    assert bytes_model.decode_kv_read_bytes("q4_0", "q4_0", 4, 8, 32768) == 150994944
    assert bytes_model.decode_kv_read_bytes("rot4", "rot4", 1, 2, 131072) == 38797312


# --- several new tokens per sequence (drafted tokens verified together) ---

def test_multi_token_single_token_is_decode(rng):
    q = rng.standard_normal((4, 128)).astype(np.float32)
    k = rng.standard_normal((40, 128)).astype(np.float32)
    v = rng.standard_normal((40, 128)).astype(np.float32)
    got = attention.decode_multi_reference(q[None], k, v, "q8_0", "q4_0", 1 / np.sqrt(128))
    assert np.array_equal(got[0], attention.decode_reference(q, k, v, "q8_0", "q4_0", 1 / np.sqrt(128)))


def test_multi_token_causality_and_last_token(rng):
    """Token t must not see rows past its own position: changing those rows
    leaves it unchanged, and the last token sees every row."""
    T, L = 3, 50
    q = rng.standard_normal((T, 2, 128)).astype(np.float32)
    k = rng.standard_normal((L, 128)).astype(np.float32)
    v = rng.standard_normal((L, 128)).astype(np.float32)
    a = attention.decode_multi_reference(q, k, v, "f16", "f16", 0.1)
    k2, v2 = k.copy(), v.copy()
    k2[L - 1] += 5.0  # the last new row: only token T-1 sees it
    v2[L - 1] -= 7.0
    b = attention.decode_multi_reference(q, k2, v2, "f16", "f16", 0.1)
    assert np.array_equal(a[:T - 1], b[:T - 1])
    assert not np.allclose(a[T - 1], b[T - 1])
    assert np.array_equal(a[T - 1], attention.decode_reference(q[T - 1], k, v, "f16", "f16", 0.1))


def test_multi_token_bruteforce(rng):
    """Tiny case against explicit loops over the causal row sets (f16 codec:
    the oracle's dequantized rows are the fp16-rounded inputs)."""
    T, L, G = 2, 5, 2
    q = rng.standard_normal((T, G, 128)).astype(np.float32)
    k = rng.standard_normal((L, 128)).astype(np.float32)
    v = rng.standard_normal((L, 128)).astype(np.float32)
    got = attention.decode_multi_reference(q, k, v, "f16", "f16", 0.2)
    kr = k.astype(np.float16).astype(np.float64)
    vr = v.astype(np.float16).astype(np.float64)
    for t in range(T):
        n = L - T + 1 + t
        want = attention.attend_bruteforce(q[t].tolist(), kr[:n].tolist(), vr[:n].tolist(), 0.2)
        assert np.allclose(got[t], want, rtol=1e-12, atol=1e-12)
