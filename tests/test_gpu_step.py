"""GPU checks of the step driver (quantized_kv_cache_append_amd.step.DecodeStep)
at a small shape with more layers than one multi-plane append call takes:
20 layers, so 40 planes go out as two vit_kv_append_quant_multi calls (32 +
8), or as 20 two-plane calls.  For all three schedules, with the split
merge in the decode launch and as a separate reduce launch, the step's
outputs equal a serial replay with per-plane appends bit for bit, every
plane holds the oracle's encoding of its ubatch rows, and every layer's
output is within 2e-3 x RMS of the oracle's attention over all its rows."""

import math

import numpy as np
import pytest

from gpu_helpers import check_close, compare_plane_rows, make_plane, ref_unit, say, torch_cuda

D = 128
CODECS = ["f16", "q8_0", "q4_0", "rot4", "rot3"]


@pytest.mark.gpu
@pytest.mark.parametrize("merged", [True, False])
@pytest.mark.parametrize("mode", ["batched", "per_layer", "overlapped"])
def test_step_more_layers_than_one_append_call(mode, merged):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit
    from quantized_kv_cache_append_amd.step import DecodeStep

    n_layers, S, H, G, cap, pre, T = 20, 2, 2, 4, 512, 300, 45
    Hq, L = H * G, pre + T
    rng = np.random.default_rng(2024 + ["batched", "per_layer", "overlapped"].index(mode))
    layers, host, q_dev, new_rows, out = [], [], [], [], []
    for li in range(n_layers):
        kc, vc = CODECS[li % 5], CODECS[(3 * li + 1) % 5]
        ks = rng.integers(0, 256, 16, dtype=np.uint8) if kc in ("rot4", "rot3") else None
        vs = rng.integers(0, 256, 16, dtype=np.uint8) if vc in ("rot4", "rot3") else None
        K, V = make_plane(kc, "k", S, H, cap, ks), make_plane(vc, "v", S, H, cap, vs)
        kx = rng.standard_normal((S, L, H, D)).astype(np.float32)
        vx = rng.standard_normal((S, L, H, D)).astype(np.float32)
        vit.vit_kv_append_quant(K, torch.from_numpy(np.ascontiguousarray(kx[:, :pre])).cuda(), [0] * S)
        vit.vit_kv_append_quant(V, torch.from_numpy(np.ascontiguousarray(vx[:, :pre])).cuda(), [0] * S)
        q = rng.standard_normal((S, Hq, D)).astype(np.float32)
        layers.append((K, V))
        host.append((kc, vc, ks, vs, kx, vx, q))
        q_dev.append(torch.from_numpy(q).cuda())
        new_rows.append((torch.from_numpy(np.ascontiguousarray(kx[:, pre:])).cuda(),
                         torch.from_numpy(np.ascontiguousarray(vx[:, pre:])).cuda()))
        out.append(torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    n_splits = 4
    ws = torch.empty(vit.vit_attn_workspace_bytes(S, Hq, D, n_splits), dtype=torch.uint8, device="cuda")
    stream, astream = torch.cuda.Stream(), torch.cuda.Stream()
    counters = vit.merge_counters(layers[0][0]) if merged else None
    step = DecodeStep(layers, q_dev, new_rows, out, [L] * S, pre, Hq, n_splits, ws, stream, astream,
                      counters=counters, append_mode=mode)
    assert step.merged == merged  # without counters: decode + reduce launches
    if mode == "batched":
        assert len(step.append_all) == 2
    if mode == "per_layer":
        assert len(step.layer_appends) == n_layers
    say(f"[step] {mode}, merged={merged}: {n_layers} layers, {2 * n_layers} planes, ubatch {T} rows at {pre}")
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    got = [o.cpu().numpy() for o in out]
    for o in out:
        o.fill_(float("nan"))
    step.run_serial()
    serial = [o.cpu().numpy() for o in out]
    if merged:
        assert int(counters.abs().sum()) == 0
    for li, ((K, V), (kc, vc, ks, vs, kx, vx, q)) in enumerate(zip(layers, host)):
        assert np.array_equal(got[li], serial[li]), f"layer {li}: step != serial replay"
        for P, x in ((K, kx), (V, vx)):
            view = P.host_view()
            for s in range(S):
                for h in range(H):
                    compare_plane_rows(P, view, s, h, np.arange(L), x[s, :, h])
        ref = np.zeros_like(got[li], dtype=np.float64)
        for s in range(S):
            for h in range(H):
                ref[s, h * G:(h + 1) * G] = ref_unit(q[s, h * G:(h + 1) * G], kx[s, :, h], vx[s, :, h], kc, vc,
                                                     1.0 / math.sqrt(D), ks, vs)
        check_close(got[li], ref, f"step layer {li} ({kc},{vc})")
