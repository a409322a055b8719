"""GPU parity of vit_kv_append_quant_multi (one launch appending to several
planes): every plane must hold exactly what vit_kv_append_quant writes into
a plane of the same codec and side from the same rows (compared array by
array, bit for bit, poisoned rows included), and the oracle's codes, scales
and norms for the appended rows.  Covers all ten (codec, side) pairs in one
call, ragged and misaligned positions, a single row, the 32-plane limit,
a call with no rows, and kernel events armed on the call."""

import numpy as np
import pytest

from gpu_helpers import compare_plane_rows, make_plane, say, torch_cuda

CODECS = ["f16", "q8_0", "q4_0", "rot4", "rot3"]
D = 128


def _rows(rng, shape):
    x = (rng.standard_normal(shape) * rng.lognormal(0, 1.5, shape[:-1] + (1,))).astype(np.float32)
    x[..., rng.integers(0, D, 2)] *= 20.0
    return x


def _pairs(rng, S, H, cap, kinds):
    """For each (codec, side): the multi-append's plane and a twin for the
    single-plane call, both poisoned."""
    out = []
    for codec, side in kinds:
        signs = rng.integers(0, 256, 16, dtype=np.uint8) if codec in ("rot4", "rot3") else None
        out.append((make_plane(codec, side, S, H, cap, signs), make_plane(codec, side, S, H, cap, signs)))
    return out


def _same_arrays(a, b, what):
    for x, y in zip(a.tensors(), b.tensors()):
        assert x.numel() == y.numel()
        assert bool((x.view(-1) == y.view(-1)).all()), f"{what}: multi-plane append differs from vit_kv_append_quant"


@pytest.mark.gpu
def test_append_multi_all_codecs_equals_single():
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    S, H, cap = 3, 2, 512
    rng = np.random.default_rng(4242)
    kinds = [(c, s) for c in CODECS for s in ("k", "v")]
    pairs = _pairs(rng, S, H, cap, kinds)
    written = [dict() for _ in kinds]
    # a misaligned ragged run, a run across several 32-row tiles, one row
    for pos0, T in (([3, 100, 250], 37), ([40, 170, 290], 70), ([511, 0, 137], 1)):
        say(f"[append-multi] 10 planes (every codec and side) pos0={pos0} T={T}")
        xs = [_rows(rng, (S, T, H, D)) for _ in kinds]
        srcs = [torch.from_numpy(x).cuda() for x in xs]
        vit.vit_kv_append_quant_multi([m for m, _ in pairs], srcs, pos0)
        for (_, single), src in zip(pairs, srcs):
            vit.vit_kv_append_quant(single, src, pos0)
        for i, x in enumerate(xs):
            for s in range(S):
                for h in range(H):
                    for t in range(T):
                        written[i][(s, h, pos0[s] + t)] = x[s, t, h]
    torch.cuda.synchronize()
    for i, ((multi, single), (codec, side)) in enumerate(zip(pairs, kinds)):
        _same_arrays(multi, single, f"{codec}/{side}")
        view = multi.host_view()
        for s in range(S):
            for h in range(H):
                idx = np.array(sorted(p for (ss, hh, p) in written[i] if ss == s and hh == h))
                compare_plane_rows(multi, view, s, h, idx, np.stack([written[i][(s, h, p)] for p in idx]))


@pytest.mark.gpu
def test_append_multi_32_planes_ladder_shape():
    """The step's call: 16 layers x (K, V) with mixed codecs, 2 sequences, 8
    KV heads, a 300-row ubatch at unaligned rows."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    S, H, cap, T = 2, 8, 1024, 300
    rng = np.random.default_rng(77)
    kinds = [(CODECS[int(rng.integers(0, 4))], side) for _ in range(16) for side in ("k", "v")]
    pairs = _pairs(rng, S, H, cap, kinds)
    pos0 = [517, 3]
    say(f"[append-multi] 32 planes S={S} H={H} T={T} pos0={pos0}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    srcs = [torch.randn((S, T, H, D), generator=gen, device="cuda") * 3.0 for _ in kinds]
    assert len(pairs) == vit.MAX_APPEND_PLANES
    vit.vit_kv_append_quant_multi([m for m, _ in pairs], srcs, pos0)
    for (_, single), src in zip(pairs, srcs):
        vit.vit_kv_append_quant(single, src, pos0)
    torch.cuda.synchronize()
    for i, ((multi, single), (codec, side)) in enumerate(zip(pairs, kinds)):
        _same_arrays(multi, single, f"plane {i} {codec}/{side}")
    # and the oracle on one (sequence, head) of a few planes
    for i in (0, 7, 31):
        multi = pairs[i][0]
        view = multi.host_view()
        x = srcs[i].cpu().numpy()
        for s in range(S):
            compare_plane_rows(multi, view, s, 5, pos0[s] + np.arange(T), x[s, :, 5])


@pytest.mark.gpu
def test_append_multi_no_rows_writes_nothing():
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(3)
    pairs = _pairs(rng, 2, 2, 256, [("q4_0", "k"), ("rot4", "v")])
    srcs = [torch.zeros((2, 0, 2, D), device="cuda") for _ in pairs]
    say("[append-multi] n_tokens 0")
    vit.vit_kv_append_quant_multi([m for m, _ in pairs], srcs, [0, 0])
    torch.cuda.synchronize()
    for multi, single in pairs:  # both still poisoned
        _same_arrays(multi, single, "no rows")


@pytest.mark.gpu
def test_append_multi_kernel_events():
    """Armed kernel events bracket the multi-plane append's one kernel, the
    arming is consumed by the call, and the planes equal an unarmed call's."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    say("[append-multi] kernel events")
    rng = np.random.default_rng(23)
    pairs = _pairs(rng, 2, 2, 512, [("q8_0", "k"), ("rot4", "v"), ("f16", "v")])
    srcs = [torch.from_numpy(_rows(rng, (2, 200, 2, D))).cuda() for _ in pairs]
    vit.vit_kv_append_quant_multi([s for _, s in pairs], srcs, [7, 300])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    vit.vit_arm_kernel_events(e0, e1)
    vit.vit_kv_append_quant_multi([m for m, _ in pairs], srcs, [7, 300])
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert 0.0 < ms < 100.0, ms
    for multi, single in pairs:
        _same_arrays(multi, single, "armed call")
    vit.vit_kv_append_quant_multi([m for m, _ in pairs], srcs, [7, 300])
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == ms
