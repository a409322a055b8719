"""GPU parity of vit_attn_decode + vit_attn_splitk_reduce against the oracle.

Bar: max |o_gpu - o_ref| <= 2e-3 x RMS(o_ref) per decode call, with o_ref the
oracle's fp64 attention over its own quantization of the same fp32 rows.
Covers all 16 (K codec, V codec) pairs, G in {1, 4, 5, 8, 16}, ragged lengths
(1 row, partial tiles), empty splits, fused append, determinism, poisoned
planes, and the single-layer workloads at full size on every (sequence, KV
head) unit (the ladder's 16 layers are in test_gpu_ladder.py).
"""

import math

import numpy as np
import pytest

import synth
from gpu_helpers import append_rows, check_close, make_plane, ref_unit, say, torch_cuda

CODECS = ["f16", "q8_0", "q4_0", "rot4", "rot3"]
D = 128


def _rand_rows(rng, shape, outliers=True):
    x = rng.standard_normal(shape).astype(np.float32)
    if outliers:
        ch = rng.choice(D, 2, replace=False)
        x[..., ch] *= 20.0
    return x


def _run_small(kc, vc, G, lens, n_splits, seed, S=2, H=2, cap=512, vmul=1.0, kmul=1.0):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(seed)
    ks = rng.integers(0, 256, 16, dtype=np.uint8) if kc in ("rot4", "rot3") else None
    vs = rng.integers(0, 256, 16, dtype=np.uint8) if vc in ("rot4", "rot3") else None
    K = make_plane(kc, "k", S, H, cap, ks)
    V = make_plane(vc, "v", S, H, cap, vs)
    Lmax = max(lens)
    kx = _rand_rows(rng, (S, Lmax, H, D)) * np.float32(kmul)
    vx = _rand_rows(rng, (S, Lmax, H, D)) * np.float32(vmul)
    append_rows(K, kx, [0] * S)
    append_rows(V, vx, [0] * S)
    Hq = H * G
    q = _rand_rows(rng, (S, Hq, D))
    qd = torch.from_numpy(q).cuda()
    out = vit.decode(K, V, qd, Hq, lens, n_splits=n_splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = np.zeros_like(got, dtype=np.float64)
    scale = 1.0 / math.sqrt(D)
    for s in range(S):
        for h in range(H):
            L = lens[s]
            ref[s, h * G:(h + 1) * G] = ref_unit(q[s, h * G:(h + 1) * G], kx[s, :L, h], vx[s, :L, h],
                                                 kc, vc, scale, ks, vs)
    return got, ref


@pytest.mark.gpu
@pytest.mark.parametrize("kc", CODECS)
@pytest.mark.parametrize("vc", CODECS)
def test_all_codec_pairs(kc, vc):
    say(f"[decode-pairs] K={kc} V={vc}")
    for G, lens, ns in ((4, [37, 300], 1), (8, [1, 257], 3)):
        got, ref = _run_small(kc, vc, G, lens, ns, seed=100 * CODECS.index(kc) + 10 * CODECS.index(vc) + G)
        check_close(got, ref, f"K={kc} V={vc} G={G} lens={lens} splits={ns}")


@pytest.mark.gpu
@pytest.mark.parametrize("G", [1, 2, 5, 12, 16])
def test_gqa_widths(G):
    say(f"[decode-gqa] G={G}")
    for kc, vc in (("q8_0", "q4_0"), ("rot4", "f16")):
        got, ref = _run_small(kc, vc, G, [96, 33], 2, seed=500 + G)
        check_close(got, ref, f"G={G} K={kc} V={vc}")


@pytest.mark.gpu
@pytest.mark.parametrize("vc", ["q8_0", "q4_0", "rot4", "rot3"])
@pytest.mark.parametrize("vmul", [1e-5, 1e-3, 1e2])
def test_v_magnitude_range(vc, vmul):
    """V rows far from unit scale: the P.V operand (probability times V block
    factor) must stay accurate whatever the magnitude of V (tiny block
    scales would otherwise put it into fp16 subnormals)."""
    say(f"[decode-vmag] V={vc} x{vmul:g}")
    for G, kc, ns in ((4, "q8_0", 2), (8, "f16", 3)):
        got, ref = _run_small(kc, vc, G, [300, 77], ns, seed=900 + G, vmul=vmul)
        check_close(got, ref, f"V={vc} x{vmul:g} K={kc} G={G}")


@pytest.mark.gpu
def test_split_counts_and_empty_splits():
    say("[decode-splits]")
    outs = []
    for ns in (1, 2, 3, 7, 16, 64):
        got, ref = _run_small("q4_0", "rot4", 4, [100, 33], ns, seed=77)
        check_close(got, ref, f"splits={ns}")
        outs.append(got)
    # split counts change only fp32 rounding
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-4 * np.sqrt(np.mean(outs[0] ** 2))


@pytest.mark.gpu
def test_deterministic_bitwise():
    """Two identical calls give bitwise identical outputs (small shape)."""
    say("[decode-determinism]")
    a, _ = _run_small("q8_0", "q8_0", 4, [480, 512], 5, seed=9)
    b, _ = _run_small("q8_0", "q8_0", 4, [480, 512], 5, seed=9)
    assert np.array_equal(a, b)


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", ["batched", "lowbit", "rotated"])
def test_deterministic_bitwise_full_size(cfg):
    """At full size, in the launch configuration bench.py times (default
    split count: 64, 128 and 32 tiles per split for these workloads, the
    fused append for batched), repeated calls on the same planes give
    bitwise identical outputs: each wave's tiles and the merge order are
    fixed."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    c = synth.CONFIGS[cfg]
    S, Hq, H, cap, L = c["seqs"], c["hq"], c["hkv"], c["capacity"], c["ctx"]
    kc, vc = synth.codec_map(cfg)[0]
    ks = synth.sign_mask(cfg, 0, "k") if kc in ("rot4", "rot3") else None
    vs = synth.sign_mask(cfg, 0, "v") if vc in ("rot4", "rot3") else None
    ns = vit.vit_attn_default_splits(S, H, Hq, L)
    say(f"[decode-determinism] {cfg} K={kc} V={vc} splits={ns} ({(L // 32 + ns - 1) // ns} tiles per split)")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321)
    K = make_plane(kc, "k", S, H, cap, ks)
    V = make_plane(vc, "v", S, H, cap, vs)
    _fill_units(K, 0, L, {}, torch, gen)
    _fill_units(V, 0, L, {}, torch, gen)
    q = torch.randn((S, Hq, D), generator=gen, device="cuda")
    knew = torch.randn((S, H, D), generator=gen, device="cuda") if c["fused_append"] else None
    vnew = torch.randn((S, H, D), generator=gen, device="cuda") if c["fused_append"] else None
    outs = []
    for _ in range(3):
        o = vit.decode(K, V, q, Hq, [L] * S, k_new=knew, v_new=vnew, n_splits=ns)
        torch.cuda.synchronize()
        outs.append(o.cpu().numpy())
    assert np.isfinite(outs[0]).all()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.gpu
def test_kernel_events_bracket_the_decode_kernel():
    """vit_arm_kernel_events: the decode dispatch records both events, the
    output is unchanged, and the arming is one-shot."""
    say("[decode-events]")
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(12)
    S, H, G, cap, L = 2, 2, 4, 512, 400
    K = make_plane("q8_0", "k", S, H, cap)
    V = make_plane("q4_0", "v", S, H, cap)
    append_rows(K, _rand_rows(rng, (S, L, H, D)), [0] * S)
    append_rows(V, _rand_rows(rng, (S, L, H, D)), [0] * S)
    q = torch.from_numpy(_rand_rows(rng, (S, H * G, D))).cuda()
    plain = vit.decode(K, V, q, H * G, [L] * S, n_splits=1).cpu().numpy()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    vit.vit_arm_kernel_events(e0, e1)
    timed = vit.decode(K, V, q, H * G, [L] * S, n_splits=1)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert 0.0 < ms < 100.0, ms
    assert np.array_equal(timed.cpu().numpy(), plain)
    # consumed: a second decode does not touch the events again
    e0.synchronize()
    again = vit.decode(K, V, q, H * G, [L] * S, n_splits=1)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == ms
    assert np.array_equal(again.cpu().numpy(), plain)


@pytest.mark.gpu
@pytest.mark.parametrize("kc,vc", [("q8_0", "q8_0"), ("rot4", "q4_0"), ("f16", "rot4"), ("rot3", "rot3")])
def test_fused_append_matches_separate_append(kc, vc):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    say(f"[decode-fused] K={kc} V={vc}")
    rng = np.random.default_rng(31)
    S, H, G, cap = 3, 2, 4, 512
    ks = rng.integers(0, 256, 16, dtype=np.uint8)
    lens = [200, 1, 512]
    kx = _rand_rows(rng, (S, cap, H, D))
    vx = _rand_rows(rng, (S, cap, H, D))
    q = torch.from_numpy(_rand_rows(rng, (S, H * G, D))).cuda()
    planes = []
    for fused in (False, True):
        K = make_plane(kc, "k", S, H, cap, ks if kc in ("rot4", "rot3") else None)
        V = make_plane(vc, "v", S, H, cap, ks if vc in ("rot4", "rot3") else None)
        # rows 0 .. max(len)-2 of every sequence; the new row then lands at len-1
        T = max(lens) - 1
        append_rows(K, kx[:, :T], [0] * S)
        append_rows(V, vx[:, :T], [0] * S)
        knew = np.stack([kx[s, lens[s] - 1] for s in range(S)])[:, None]
        vnew = np.stack([vx[s, lens[s] - 1] for s in range(S)])[:, None]
        if fused:
            out = vit.decode(K, V, q, H * G, lens, k_new=torch.from_numpy(knew[:, 0]).cuda(),
                             v_new=torch.from_numpy(vnew[:, 0]).cuda(), n_splits=4)
        else:
            append_rows(K, knew, [l - 1 for l in lens])
            append_rows(V, vnew, [l - 1 for l in lens])
            out = vit.decode(K, V, q, H * G, lens, n_splits=4)
        torch.cuda.synchronize()
        planes.append((K.host_view(), V.host_view(), out.cpu().numpy()))
    (k0, v0, o0), (k1, v1, o1) = planes
    for s in range(S):
        L = lens[s]
        for a, b in ((k0, k1), (v0, v1)):
            for key in a:
                assert np.array_equal(a[key][s, :, :L], b[key][s, :, :L]), key
    assert np.array_equal(o0, o1)


# ---------------------------------------------------------------- workloads


def _fill_units(plane, start, count, rows, torch, gen):
    """Rows start .. start+count-1 of every (seq, head) stream of a plane: the
    given rows (full streams, indexed by unit) where known, seeded device
    normals elsewhere; one vit_kv_append_quant call."""
    from quantized_kv_cache_append_amd import vit_kv_append_quant

    S, H = plane.n_seqs, plane.n_kv_heads
    src = torch.randn((S, count, H, D), generator=gen, device="cuda", dtype=torch.float32)
    for (s, h), r in rows.items():
        src[s, :, h] = torch.from_numpy(np.ascontiguousarray(r[start:start + count])).cuda()
    vit_kv_append_quant(plane, src, [start] * S)


def _run_workload(cfg, units, layers=(0,)):
    """One decode call of a workload at full size, in the launch
    configuration bench.py times (the library's default split count, fused
    append where the workload has one); the oracle checks every listed
    (sequence, KV head) unit, all its query heads."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    c = synth.CONFIGS[cfg]
    S, Hq, H, cap = c["seqs"], c["hq"], c["hkv"], c["capacity"]
    G = Hq // H
    cmap = synth.codec_map(cfg)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.SEED_ID[cfg])
    scale = 1.0 / math.sqrt(D)
    for layer in layers:
        kc, vc = cmap[layer]
        ks = synth.sign_mask(cfg, layer, "k") if kc in ("rot4", "rot3") else None
        vs = synth.sign_mask(cfg, layer, "v") if vc in ("rot4", "rot3") else None
        say(f"[workload {c['name']}] layer {layer} K={kc} V={vc}: {len(units)} of {S * H} (seq, KV head) units")
        K = make_plane(kc, "k", S, H, cap, ks)
        V = make_plane(vc, "v", S, H, cap, vs)
        L = c["ctx"]
        lens = [L] * S
        krows = {u: synth.kv_rows(cfg, "k", layer, u[0], u[1], 0, L) for u in units}
        vrows = {u: synth.kv_rows(cfg, "v", layer, u[0], u[1], 0, L) for u in units}
        q = np.stack([synth.q_rows(cfg, layer, s, Hq) for s in range(S)])
        qd = torch.from_numpy(q).cuda()
        ns = vit.vit_attn_default_splits(S, H, Hq, L)
        if c["fused_append"]:
            _fill_units(K, 0, L - 1, krows, torch, gen)
            _fill_units(V, 0, L - 1, vrows, torch, gen)
            knew = torch.randn((S, H, D), generator=gen, device="cuda")
            vnew = torch.randn((S, H, D), generator=gen, device="cuda")
            for (s, h) in units:
                knew[s, h] = torch.from_numpy(krows[(s, h)][L - 1]).cuda()
                vnew[s, h] = torch.from_numpy(vrows[(s, h)][L - 1]).cuda()
            out = vit.decode(K, V, qd, Hq, lens, k_new=knew, v_new=vnew, n_splits=ns)
        else:
            _fill_units(K, 0, L, krows, torch, gen)
            _fill_units(V, 0, L, vrows, torch, gen)
            out = vit.decode(K, V, qd, Hq, lens, n_splits=ns)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        gots, refs = [], []
        for (s, h) in units:
            r = ref_unit(q[s, h * G:(h + 1) * G], krows[(s, h)], vrows[(s, h)], kc, vc, scale, ks, vs)
            gots.append(got[s, h * G:(h + 1) * G])
            refs.append(r)
        check_close(np.stack(gots), np.stack(refs), f"{c['name']} layer {layer} ({kc},{vc}) splits={ns}")
        del K, V
        torch.cuda.empty_cache()


def _every_unit(cfg):
    c = synth.CONFIGS[cfg]
    return [(s, h) for s in range(c["seqs"]) for h in range(c["hkv"])]


@pytest.mark.gpu
def test_workload_tiny():
    _run_workload("tiny", _every_unit("tiny"))


@pytest.mark.gpu
@pytest.mark.timeout(600)
def test_workload_batched():
    _run_workload("batched", _every_unit("batched"))


@pytest.mark.gpu
@pytest.mark.timeout(600)
def test_workload_lowbit():
    _run_workload("lowbit", _every_unit("lowbit"))


@pytest.mark.gpu
@pytest.mark.timeout(600)
def test_workload_rotated():
    _run_workload("rotated", _every_unit("rotated"))
