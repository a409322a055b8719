"""Pins of oracle/vbr.py: the degrade step (re-encoding stored rows) and the
classic ladder's band-by-band order (buun-llama-cpp page, "VBR -- Variable
Bit-Rate KV Cache").  CPU only."""

import numpy as np
import pytest

from oracle import bytes_model, codecs, vbr
from oracle.fp import f16_bits


def _rows(seed, n=40):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32)
    x *= np.exp(rng.standard_normal(128)).astype(np.float32)  # per-channel scales
    x[rng.random((n, 128)) < 0.01] *= 30.0                    # outliers
    x[3, :32] = 0.0                                           # a zero block
    return x


# ------------------------------------------------------------ degrade step
@pytest.mark.parametrize("codec", ["f16", "q8_0", "q4_0"])
def test_transcode_to_own_codec_is_identity(codec):
    # Stored rows decode to values that the encoder maps back to the same
    # fields: f16 is lossless on fp16 values; q8_0 finds amax = 127 |d|; q4_0
    # finds its signed maximum at code 0, i.e. -8 d, so d' = d.
    q = codecs.quantize(codec, _rows(1))
    t = vbr.transcode(codec, codec, q)
    for key in q:
        assert np.array_equal(t[key], q[key]), key


@pytest.mark.parametrize("dst", ["q8_0", "q4_0", "rot4", "rot3"])
def test_transcode_from_f16_equals_encoding_the_values(dst):
    # rows that are already fp16 values come out of an f16 plane unchanged
    x = _rows(2).astype(np.float16).astype(np.float32)
    signs = (np.arange(16) * 37 % 256).astype(np.uint8) if dst in ("rot4", "rot3") else None
    t = vbr.transcode("f16", dst, codecs.quantize("f16", x), dst_signs=signs)
    ref = codecs.quantize(dst, x, signs)
    for key in ref:
        assert np.array_equal(t[key], ref[key]), key


def test_transcode_q8_to_q4_worked_block():
    # One q8_0 block worked by hand: scale 0.5, codes 100, -64, 7, 3, -3, 0...
    # values 50, -32, 3.5, 1.5, -1.5, 0 ...; signed max m = 50 -> d = -6.25
    # (fp16 0xC640), 1/d = -0.16 in fp32; x/d -> -8, 5.12, -0.56, -0.24, 0.24
    # -> RHAZ + 8 = 0, 13, 7, 8, 8.  The other three blocks are zero.
    codes = np.zeros((1, 128), dtype=np.int8)
    codes[0, :5] = [100, -64, 7, 3, -3]
    scales = np.zeros((1, 4), dtype=np.uint16)
    scales[0, 0] = 0x3800  # 0.5
    t = vbr.transcode("q8_0", "q4_0", {"codes": codes, "scales": scales})
    exp_codes = np.full((1, 128), 8, dtype=np.uint8)
    exp_codes[0, :5] = [0, 13, 7, 8, 8]
    assert np.array_equal(t["codes"], exp_codes)
    assert t["scales"].tolist() == [[0xC640, 0, 0, 0]]


def test_transcode_q8_to_rot4_norm_is_the_row_norm():
    # rot4 stores fp16(||x||) of the decoded row; ||x||^2 = sum_b d_b^2 sum_j c_j^2
    q = codecs.quantize("q8_0", _rows(3))
    signs = np.full(16, 0xA5, dtype=np.uint8)
    t = vbr.transcode("q8_0", "rot4", q, dst_signs=signs)
    d = q["scales"].view(np.float16).astype(np.float64)
    c2 = (q["codes"].astype(np.float64) ** 2).reshape(-1, 4, 32).sum(axis=-1)
    expect = f16_bits(np.sqrt((c2 * d * d).sum(axis=-1)).astype(np.float32))
    diff = np.abs(t["norms"].astype(np.int64) - expect.astype(np.int64))
    assert diff.max() <= 1  # fp32 summation order vs fp64: at most one fp16 ulp


def test_transcode_rejects_inexact_source_and_added_bits():
    q4 = codecs.quantize("q4_0", _rows(4))
    with pytest.raises(AssertionError):
        vbr.transcode("q4_0", "q8_0", q4)
    signs = np.zeros(16, dtype=np.uint8)
    r4 = codecs.quantize("rot4", _rows(4), signs)
    with pytest.raises(AssertionError):
        vbr.transcode("rot4", "q4_0", r4, src_signs=signs)


# ------------------------------------------------------------ classic order
def test_classic_schedule_full_ladder_closed_form():
    n = 32  # 16 attention layers x (K, V)
    order = list(np.random.default_rng(5).permutation(n))
    steps = vbr.classic_schedule(["f16"] * n, order)
    # every tensor reaches q8_0 (in price order) before any goes on to q4_0
    assert steps == [(i, "q8_0") for i in order] + [(i, "q4_0") for i in order]
    # 2 rungs per tensor: the page's count rule (tensors x rungs) for this ladder
    assert len(steps) == bytes_model.vbr_steps(16, n_rungs=2) == 64
    state = ["f16"] * n
    for k, (i, c) in enumerate(steps, start=1):
        state[i] = c
        expect = 16.0 - 7.5 * k / n if k <= n else 8.5 - 4.0 * (k - n) / n
        assert vbr.aggregate_bpv(state) == pytest.approx(expect, abs=1e-12)


def test_classic_schedule_stays_banded_with_pinned_sides():
    rng = np.random.default_rng(6)
    for trial in range(20):
        n = int(rng.integers(2, 40))
        movable = list(rng.random(n) < 0.7)
        order = list(rng.permutation(n))
        state = ["f16"] * n
        steps = vbr.classic_schedule(state, order, movable)
        assert len(steps) == 2 * sum(movable)
        for i, c in steps:
            assert movable[i]
            state[i] = c
            m = [state[j] for j in range(n) if movable[j]]
            assert not ("q4_0" in m and "f16" in m), "a tensor reached q4_0 while another was still f16"
        assert all(state[j] == ("q4_0" if movable[j] else "f16") for j in range(n))


def test_classic_schedule_resumes_a_partly_degraded_cache():
    # tensors 0 and 2 already at q8_0: the remaining f16 tensors move first
    state = ["q8_0", "f16", "q8_0", "f16"]
    steps = vbr.classic_schedule(state, [3, 2, 1, 0])
    assert steps == [(3, "q8_0"), (1, "q8_0"), (3, "q4_0"), (2, "q4_0"), (1, "q4_0"), (0, "q4_0")]


@pytest.mark.parametrize("floor,n_steps", [(16.0, 0), (12.25, 16), (8.5, 32), (8.4, 32), (4.5, 64), (1.25, 64)])
def test_classic_schedule_stops_at_the_floor(floor, n_steps):
    # after k <= 32 steps the aggregate is 16 - 7.5 k / 32, after 32 + j it is
    # 8.5 - 4 j / 32: the last step still >= the floor ends the schedule
    steps = vbr.classic_schedule(["f16"] * 32, list(range(32)), floor_bpv=floor)
    assert len(steps) == n_steps
