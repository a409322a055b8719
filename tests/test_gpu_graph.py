"""A decode step (fused append + vit_attn_decode + vit_attn_splitk_reduce)
captured into a HIP graph and replayed, as a serving loop (or bench.py --graph)
would do.

Each replay runs after unrelated eager work and a synchronization, and its
output is checked against the eager call (same kernels and inputs; every
wave's tiles and summation order are fixed, so the bar is bit equality) and
against the oracle (the usual 2e-3 x RMS).  The second test captures a whole
multi-layer step of the step driver (one multi-plane append, then a merged
decode per layer) and checks its replays the same way.
"""

import math

import numpy as np
import pytest

from gpu_helpers import append_rows, check_close, make_plane, ref_unit, say, torch_cuda

D = 128


@pytest.mark.gpu
@pytest.mark.parametrize("kc,vc,G", [("q8_0", "q8_0", 4), ("q4_0", "rot4", 8), ("rot4", "f16", 5)])
def test_captured_step_replays_match_eager(kc, vc, G):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    say(f"[graph] K={kc} V={vc} G={G}")
    rng = np.random.default_rng(2024 + G)
    S, H, cap, n_splits = 2, 2, 512, 3
    lens = [300, 97]
    ks = rng.integers(0, 256, 16, dtype=np.uint8) if kc in ("rot4", "rot3") else None
    vs = rng.integers(0, 256, 16, dtype=np.uint8) if vc in ("rot4", "rot3") else None
    K = make_plane(kc, "k", S, H, cap, ks)
    V = make_plane(vc, "v", S, H, cap, vs)
    kx = rng.standard_normal((S, max(lens), H, D)).astype(np.float32)
    vx = rng.standard_normal((S, max(lens), H, D)).astype(np.float32)
    # rows 0 .. 298 appended here; row L-1 of each sequence comes again with
    # the decode call (fused append, same values)
    append_rows(K, kx[:, :max(lens) - 1], [0] * S)
    append_rows(V, vx[:, :max(lens) - 1], [0] * S)
    q = rng.standard_normal((S, H * G, D)).astype(np.float32)
    k_new = np.stack([kx[s, lens[s] - 1] for s in range(S)])  # [S][H][D]
    v_new = np.stack([vx[s, lens[s] - 1] for s in range(S)])
    qd = torch.from_numpy(q).cuda()
    knd = torch.from_numpy(np.ascontiguousarray(k_new)).cuda()
    vnd = torch.from_numpy(np.ascontiguousarray(v_new)).cuda()
    ws = torch.empty(vit.vit_attn_workspace_bytes(S, H * G, D, n_splits), dtype=torch.uint8, device="cuda")

    eager = vit.decode(K, V, qd, H * G, lens, k_new=knd, v_new=vnd, n_splits=n_splits, workspace=ws)
    torch.cuda.synchronize()
    ref_e = eager.cpu().numpy()

    ref = np.zeros_like(ref_e, dtype=np.float64)
    for s in range(S):
        L = lens[s]
        for h in range(H):
            ref[s, h * G:(h + 1) * G] = ref_unit(q[s, h * G:(h + 1) * G], kx[s, :L, h], vx[s, :L, h], kc, vc,
                                                 1.0 / math.sqrt(D), ks, vs)
    check_close(ref_e, ref, f"eager K={kc} V={vc} G={G}")

    stream = torch.cuda.Stream()
    out = torch.empty_like(eager)
    with torch.cuda.stream(stream):
        d = vit.prepare_decode(K, V, qd, H * G, lens, out, k_new=knd, v_new=vnd, n_splits=n_splits,
                               workspace=ws, stream=stream)
        red = vit.prepare_reduce(ws, S, H * G, n_splits, V, out, stream=stream)
        d()
        red()  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        d()
        red()
    torch.cuda.synchronize()

    rms = float(np.sqrt(np.mean(ref_e.astype(np.float64) ** 2)))
    other = torch.empty_like(eager)
    for rep in range(4):
        out.fill_(float("nan"))
        # unrelated eager work between replays
        vit.decode(K, V, qd, H * G, [l - 1 for l in lens], n_splits=2, out=other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        err = float(np.max(np.abs(got.astype(np.float64) - ref_e)))
        say(f"  replay {rep}: max|graph - eager| / rms = {err / rms:.2e}")
        assert np.all(np.isfinite(got)), f"replay {rep}: non-finite output"
        assert np.array_equal(got, ref_e), f"replay {rep}: graph output differs from eager by {err:.3e}"
        check_close(got, ref, f"replay {rep} K={kc} V={vc} G={G}")


@pytest.mark.gpu
def test_captured_multilayer_step_replays_match_eager():
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit
    from quantized_kv_cache_append_amd.step import DecodeStep

    n_layers, S, H, G, cap, pre, T = 6, 2, 2, 4, 512, 200, 33
    Hq, L = H * G, pre + T
    codecs = [("f16", "q4_0"), ("q8_0", "rot4"), ("rot4", "q8_0"), ("q4_0", "f16"), ("rot3", "rot3"), ("q8_0", "q8_0")]
    rng = np.random.default_rng(99)
    layers, host, q_dev, new_rows, out = [], [], [], [], []
    for kc, vc in codecs:
        ks = rng.integers(0, 256, 16, dtype=np.uint8) if kc in ("rot4", "rot3") else None
        vs = rng.integers(0, 256, 16, dtype=np.uint8) if vc in ("rot4", "rot3") else None
        K, V = make_plane(kc, "k", S, H, cap, ks), make_plane(vc, "v", S, H, cap, vs)
        kx = rng.standard_normal((S, L, H, D)).astype(np.float32)
        vx = rng.standard_normal((S, L, H, D)).astype(np.float32)
        append_rows(K, kx[:, :pre], [0] * S)
        append_rows(V, vx[:, :pre], [0] * S)
        q = rng.standard_normal((S, Hq, D)).astype(np.float32)
        layers.append((K, V))
        host.append((kc, vc, ks, vs, kx, vx, q))
        q_dev.append(torch.from_numpy(q).cuda())
        new_rows.append((torch.from_numpy(np.ascontiguousarray(kx[:, pre:])).cuda(),
                         torch.from_numpy(np.ascontiguousarray(vx[:, pre:])).cuda()))
        out.append(torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda"))
    n_splits = 4
    ws = torch.empty(vit.vit_attn_workspace_bytes(S, Hq, D, n_splits), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    counters = vit.merge_counters(layers[0][0])
    torch.cuda.synchronize()
    step = DecodeStep(layers, q_dev, new_rows, out, [L] * S, pre, Hq, n_splits, ws, stream, None, counters=counters)
    assert step.merged and step.append_mode == "batched"
    say(f"[graph] multi-layer step: {n_layers} layers, one multi-plane append, merged decodes")
    with torch.cuda.stream(stream):
        step()  # eager, also the warm-up on the capture stream
    torch.cuda.synchronize()
    eager = [o.cpu().numpy() for o in out]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    other = torch.empty((S, Hq, D), dtype=torch.float32, device="cuda")
    for rep in range(4):
        for o in out:
            o.fill_(float("nan"))
        K0, V0 = layers[0]
        vit.decode(K0, V0, q_dev[0], Hq, [pre] * S, n_splits=2, out=other)  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(counters.abs().sum()) == 0, f"replay {rep}: arrival counters not back at zero"
        for li, o in enumerate(out):
            got = o.cpu().numpy()
            assert np.array_equal(got, eager[li]), f"replay {rep}, layer {li}: graph output differs from eager"
    for li, (kc, vc, ks, vs, kx, vx, q) in enumerate(host):
        ref = np.zeros_like(eager[li], dtype=np.float64)
        for s in range(S):
            for h in range(H):
                ref[s, h * G:(h + 1) * G] = ref_unit(q[s, h * G:(h + 1) * G], kx[s, :, h], vx[s, :, h], kc, vc,
                                                     1.0 / math.sqrt(D), ks, vs)
        check_close(eager[li], ref, f"multi-layer step layer {li} ({kc},{vc})")
