"""GPU parity of vit_kv_transcode (a VBR degrade step) against
oracle.vbr.transcode: codes, fp16 scales and norms bit-exact on the rows
re-encoded, destination rows past n_rows untouched.

The source plane is filled by vit_kv_append_quant; the oracle's input is its
own quantization of the same fp32 rows (append parity makes the two equal),
never the plane's contents.
"""

import numpy as np
import pytest

import synth
from gpu_helpers import append_rows, fill_plane_synth, make_plane, say, torch_cuda, unit_view
from oracle import codecs, vbr

D = 128
PAIRS = [("f16", "q8_0"), ("f16", "q4_0"), ("f16", "rot4"), ("q8_0", "q4_0"), ("q8_0", "rot4"),
         ("f16", "rot3"), ("q8_0", "rot3"), ("q4_0", "rot3")]


def _rows(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    x *= np.exp(rng.standard_normal(shape[-2:])).astype(np.float32)  # per-(head, channel) scales
    x[rng.random(shape) < 0.01] *= 40.0
    x[..., 5, :, :32] = 0.0   # a zero block in row 5 of every (seq, head)
    x[..., 9, :, 64:96] = 3.0  # a constant block (ties of the block max)
    return x


def _check_rows(dst_view, fresh_view, expect, s, h, n):
    for key in expect:
        got = dst_view[key][s, h]
        exp = expect[key]
        if key == "codes" and got.dtype != exp.dtype:
            got = got.astype(exp.dtype)
        bad = np.argwhere(got[:n] != exp[:n])
        assert bad.size == 0, f"{key} mismatch at (seq {s}, head {h}) rows {bad[:5, 0]}"
        # rows past n_rows keep what the destination held before
        assert np.array_equal(dst_view[key][s, h, n:], fresh_view[key][s, h, n:]), f"{key} rows past n_rows changed"


@pytest.mark.gpu
@pytest.mark.parametrize("side", ["k", "v"])
@pytest.mark.parametrize("src_c,dst_c", PAIRS)
def test_transcode_matches_oracle(src_c, dst_c, side):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    say(f"[transcode] {src_c} -> {dst_c} side {side}")
    rng = np.random.default_rng(900 + 10 * PAIRS.index((src_c, dst_c)) + (side == "v"))
    S, H, cap = 3, 2, 512
    n_rows = [300, 37, 512]  # ragged: a partial tile, a partial 8-row group, every row
    dsigns = rng.integers(0, 256, 16, dtype=np.uint8) if dst_c in ("rot4", "rot3") else None
    src = make_plane(src_c, side, S, H, cap)
    x = _rows(rng, (S, cap, H, D))
    append_rows(src, x, [0] * S)
    dst = make_plane(dst_c, side, S, H, cap, dsigns)  # poisoned: every bit set
    fresh = dst.host_view()
    vit.vit_kv_transcode(src, dst, n_rows)
    torch.cuda.synchronize()
    view = dst.host_view()
    for s in range(S):
        for h in range(H):
            q_src = codecs.quantize(src_c, x[s, :, h])
            expect = vbr.transcode(src_c, dst_c, q_src, dst_signs=dsigns)
            _check_rows(view, fresh, expect, s, h, n_rows[s])


@pytest.mark.gpu
def test_transcode_zero_rows_and_a_second_step():
    """n_rows 0 leaves the destination as it was; q8_0 written by one step is
    the source of the next (f16 -> q8_0 -> q4_0, the classic ladder)."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(77)
    S, H, cap = 2, 3, 256
    x = _rows(rng, (S, cap, H, D))
    a = make_plane("f16", "v", S, H, cap)
    append_rows(a, x, [0] * S)
    b = make_plane("q8_0", "v", S, H, cap)
    c = make_plane("q4_0", "v", S, H, cap)
    fresh_c = c.host_view()
    vit.vit_kv_transcode(a, b, [256, 0])
    vit.vit_kv_transcode(b, c, [256, 0])
    torch.cuda.synchronize()
    vb, vc_ = b.host_view(), c.host_view()
    for h in range(H):
        q8 = vbr.transcode("f16", "q8_0", codecs.quantize("f16", x[0, :, h]))
        q4 = vbr.transcode("q8_0", "q4_0", q8)
        _check_rows(vb, b.host_view(), q8, 0, h, 256)
        _check_rows(vc_, fresh_c, q4, 0, h, 256)
        _check_rows(vc_, fresh_c, q4, 1, h, 0)  # sequence 1: nothing re-encoded


@pytest.mark.gpu
def test_transcode_ladder_tensor_full_size():
    """One (layer, side) tensor of the 200,704-row ladder slots (2 sequences x
    8 KV heads), f16 -> q8_0 on the K side as bench.py --transcode times it;
    sampled (sequence, KV head) units checked on every row."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    c = synth.CONFIGS["ladder"]
    S, H, cap = c["seqs"], c["hkv"], c["capacity"]
    units = [(1, 6)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(55)
    say(f"[transcode ladder] f16 -> q8_0, {S} x {H} x {cap} rows, units {units}")
    src = make_plane("f16", "k", S, H, cap, poison=False)
    fill_plane_synth(src, "ladder", 0, "k", 0, cap, units, torch, gen)
    torch.cuda.empty_cache()
    dst = make_plane("q8_0", "k", S, H, cap, poison=False)
    vit.vit_kv_transcode(src, dst, [cap] * S)
    torch.cuda.synchronize()
    for (s, h) in units:
        view = unit_view(dst, s, h)
        rows = synth.kv_rows("ladder", "k", 0, s, h, 0, cap)
        expect = vbr.transcode("f16", "q8_0", codecs.quantize("f16", rows))
        assert np.array_equal(view["codes"].astype(np.int8), expect["codes"])
        assert np.array_equal(view["scales"], expect["scales"])
    del src, dst
    torch.cuda.empty_cache()
