"""GPU parity of vit_kv_append_quant: codes, fp16 scales and norms must equal
the oracle's bit for bit, for every codec and both plane sides, on seeded
rows plus crafted edge rows, at ragged and misaligned positions; rows outside
the appended range must stay untouched (planes are poisoned first)."""

import numpy as np
import pytest

from gpu_helpers import append_rows, compare_plane_rows, make_plane, say, torch_cuda
from test_oracle_crafted import ROWS as CRAFTED, SIGNS as CRAFTED_SIGNS

CODECS = ["f16", "q8_0", "q4_0", "rot4", "rot3"]
D = 128


def _edge_rows():
    """Rows that exercise ties, zero blocks, subnormal scales and clamps."""
    rows = []
    z = np.zeros(D, np.float32)
    rows.append(z.copy())                                  # zero row
    for k in (0, 3, 10):                                   # exact q8 ties at d = 2^-k
        u = np.float32(2.0 ** -k)
        r = z.copy()
        r[:7] = np.array([127, 2.5, -2.5, 1.5, -0.5, 0.5, 126.5], np.float32) * u
        r[32:40] = np.array([-8, 2.5, -2.5, 0.5, -0.5, 7.5, 3.5, -3.5], np.float32) * u  # q4 ties, d = u
        r[64] = 1.0
        r[65] = -1.0                                          # q4 opposite-sign tie
        r[96:] = np.linspace(-3, 3, 32, dtype=np.float32)
        rows.append(r)
    r = z.copy()
    r[:32] = np.float32(127e-6) * np.linspace(-1, 1, 32, dtype=np.float32)  # fp16 subnormal scales
    r[32:64] = np.float32(1e-30)                              # fp32 tiny values, norm path
    rows.append(r)
    r = np.full(D, 0.49999997, np.float32)                    # RHAZ trap
    r[0] = 127.0
    rows.append(r)
    r = z.copy()
    r[5] = -3.0                                               # single element
    rows.append(r)
    r = np.zeros(D, np.float32)
    r[:] = np.float32(1.0e-25)                                # tiny rows (squares underflow)
    r[::3] = np.float32(-3.0e-25)
    rows.append(r)
    # rows on which the reciprocal rule, a tie rule or the operation order
    # decides a stored field (tests/golden/crafted_rows.txt)
    rows += [c["x"] for c in CRAFTED]
    return np.stack(rows).astype(np.float32)


@pytest.mark.gpu
@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("side", ["k", "v"])
def test_append_bit_exact(codec, side):
    torch = torch_cuda()
    say(f"[append] codec={codec} side={side}")
    S, H, cap = 3, 2, 512
    rng = np.random.default_rng(1000 + 10 * CODECS.index(codec) + (side == "v"))
    signs = rng.integers(0, 256, 16, dtype=np.uint8) if codec in ("rot4", "rot3") else None
    plane = make_plane(codec, side, S, H, cap, signs)
    edge = _edge_rows()
    written = {}
    # three appends: misaligned ragged start, a run across tiles, a single row
    for pos0, T in (([3, 100, 250], 37), ([40, 170, 290], 70), ([511, 0, 137], 1)):
        x = (rng.standard_normal((S, T, H, D)) * rng.lognormal(0, 1.5, (S, T, H, 1))).astype(np.float32)
        x[:, :, :, rng.integers(0, D, 2)] *= 20.0
        ne = min(T, len(edge))
        x[0, :ne, 0] = edge[:ne]
        append_rows(plane, x, pos0)
        for s in range(S):
            for h in range(H):
                for t in range(T):
                    written[(s, h, pos0[s] + t)] = x[s, t, h]
    torch.cuda.synchronize()
    view = plane.host_view()
    for s in range(S):
        for h in range(H):
            idx = np.array(sorted(p for (ss, hh, p) in written if ss == s and hh == h))
            rows = np.stack([written[(s, h, p)] for p in idx])
            compare_plane_rows(plane, view, s, h, idx, rows)
            # untouched rows keep the poison
            mask = np.ones(cap, bool)
            mask[idx] = False
            untouched = view["codes"][s, h, mask]
            if codec == "f16":
                assert np.all(untouched == 0xFFFF)
            elif codec == "q8_0":
                assert np.all(untouched.astype(np.int8) == -1)
            else:
                assert np.all(untouched == (7 if codec == "rot3" else 15))  # every code bit set
            if "scales" in view:
                assert np.all(view["scales"][s, h, mask] == 0xFFFF)


@pytest.mark.gpu
@pytest.mark.parametrize("codec", ["q4_0", "rot4", "q8_0", "rot3"])
def test_append_many_random_rows(codec):
    """20k seeded rows per codec (heavy tails, outliers, tiny rows) through
    the K and V layouts; exercises the correctly rounded sqrt of rot4."""
    torch_cuda()
    say(f"[append-many] codec={codec}")
    S, H, cap = 2, 4, 2560
    rng = np.random.default_rng(77 + CODECS.index(codec))
    signs = rng.integers(0, 256, 16, dtype=np.uint8) if codec in ("rot4", "rot3") else None
    x = rng.standard_normal((S, cap, H, D)).astype(np.float32)
    hit = rng.random(x.shape) < 0.01
    x[hit] = rng.standard_t(3, int(hit.sum())).astype(np.float32)
    x *= rng.lognormal(0, 2.5, (S, cap, H, 1)).astype(np.float32)
    # stay inside the fp16 range of the stored norm / scales
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    x = np.where(n > 3.0e4, x * (3.0e4 / n), x).astype(np.float32)
    for side in ("k", "v"):
        plane = make_plane(codec, side, S, H, cap, signs)
        append_rows(plane, x, [0, 0])
        view = plane.host_view()
        for s in range(S):
            for h in range(H):
                compare_plane_rows(plane, view, s, h, np.arange(cap), x[s, :, h])


@pytest.mark.gpu
def test_kernel_events_bracket_the_append_kernel():
    """vit_arm_kernel_events before vit_kv_append_quant: the append dispatch
    records both events, the stored planes equal an unarmed append's, and the
    arming is one-shot."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    say("[append-events]")
    rng = np.random.default_rng(19)
    S, H, cap = 2, 2, 512
    x = rng.standard_normal((S, 300, H, D)).astype(np.float32)
    plain = make_plane("q4_0", "v", S, H, cap)
    timed = make_plane("q4_0", "v", S, H, cap)
    append_rows(plain, x, [5, 100])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    vit.vit_arm_kernel_events(e0, e1)
    append_rows(timed, x, [5, 100])
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert 0.0 < ms < 100.0, ms
    a, b = plain.host_view(), timed.host_view()
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    # consumed: a second append does not touch the events again
    append_rows(timed, x, [5, 100])
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == ms


@pytest.mark.gpu
@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("side", ["k", "v"])
def test_append_crafted_rows(codec, side):
    """The crafted rows (tests/golden/crafted_rows.txt) with the sign mask
    they were found for: whitened values exactly on rot4 / rot3 thresholds,
    q8_0 / q4_0 elements where x * (1/d) and x / d round differently, and
    rows where the WHT stage order or the summation order moves a field.
    Bit-exact against the oracle; the tie channels also against their
    hand-stated index (the level farther from zero)."""
    torch_cuda()
    say(f"[append-crafted] codec={codec} side={side}")
    S, H, cap = 2, 2, 256
    rng = np.random.default_rng(4242)
    x = rng.standard_normal((S, len(CRAFTED), H, D)).astype(np.float32)
    for i, c in enumerate(CRAFTED):
        x[0, i, 0] = c["x"]
        x[1, i, 1] = c["x"]
    signs = CRAFTED_SIGNS if codec in ("rot4", "rot3") else None
    plane = make_plane(codec, side, S, H, cap, signs)
    pos0 = [3, 200 - len(CRAFTED)]
    append_rows(plane, x, pos0)
    view = plane.host_view()
    for s in range(S):
        for h in range(H):
            idx = np.arange(pos0[s], pos0[s] + len(CRAFTED))
            compare_plane_rows(plane, view, s, h, idx, x[s, :, h])
    if codec in ("rot4", "rot3"):
        from oracle import lloyd_max

        lv, _, _ = lloyd_max.codebook(16 if codec == "rot4" else 8)
        for i, c in enumerate(CRAFTED):
            if c["kind"] == "tie" and c["codec"] == codec:
                k = int(c["detail"][3:])
                want = k + 1 if lv[k] + lv[k + 1] > 0 else k
                for s, h in ((0, 0), (1, 1)):
                    assert int(view["codes"][s, h, pos0[s] + i, c["ch"]]) == want, (codec, k)
