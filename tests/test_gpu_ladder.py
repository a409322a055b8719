"""GPU parity of the ladder workload's whole step against the oracle.

The ladder: 16 layers, each (layer, side) with its own codec from a seeded
balanced map (8 each of f16, q8_0, q4_0, rot4; 10 distinct (K, V) pairs),
2 sequences x 8 KV heads x 200,704-row slots, Hq 32.  One step through the
step driver (quantized_kv_cache_append_amd.step.DecodeStep) on planes that
were poisoned and then pre-filled with rows 0 .. 198,655: the 2048-row
ubatch (rows 198,656 .. 200,703) is appended to all 32 planes by one
vit_kv_append_quant_multi launch, then the 16 decodes run; each layer's
decode and split merge is one vit_attn_decode_merged launch.

The rows a decode would read before the append finished are still poison
(NaN fp16 scales, all-ones codes), so a wrong order shows up as a wrong
output.  Each layer has its own sampled (sequence, KV head) unit --
16 distinct units -- whose rows and queries come from ``synth``; the other
units get seeded device normals.  Per layer: the stored ubatch rows of the
unit are bit-exact against the oracle's encoders, and the decode output of
its 4 query heads is within 2e-3 x RMS of the oracle's fp64 attention over
all 200,704 rows, and every output equals a serial replay with per-plane
appends (vit_kv_append_quant, then all decodes) bit for bit.  Same split
count and launch configuration as bench.py.

The step driver's other schedule, per-plane appends on a second stream
overlapped with the decodes (decode l waiting only for layer l's appends),
is then checked the same way on a ubatch scaled by 8 in place: a decode
that ran before its layer's appends would read the unscaled rows, whose
logits differ by O(1), so the overlapped step must equal its serial replay
bit for bit.
"""

import math

import numpy as np
import pytest

import synth
from gpu_helpers import check_close, make_plane, ref_unit, say, torch_cuda, unit_view
from oracle import codecs

D = 128
CFG = "ladder"


def _unit(layer):
    return (layer // 8) % 2, (3 * layer + 1) % 8


@pytest.fixture(scope="module")
def ladder_step():
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit
    from quantized_kv_cache_append_amd.step import DecodeStep

    c = synth.CONFIGS[CFG]
    S, Hq, H, cap, L, pre, ub = c["seqs"], c["hq"], c["hkv"], c["capacity"], c["ctx"], c["prefill"], c["ubatch"]
    cmap = synth.codec_map(CFG)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.SEED_ID[CFG] + 1000)
    layers, q_dev, q_host, new_rows, out, rows = [], [], [], [], [], {}
    for li, (kc, vc) in enumerate(cmap):
        s, h = _unit(li)
        say(f"[ladder step] filling layer {li} ({kc},{vc}), sampled unit ({s},{h})")
        ks = synth.sign_mask(CFG, li, "k") if kc in ("rot4", "rot3") else None
        vs = synth.sign_mask(CFG, li, "v") if vc in ("rot4", "rot3") else None
        K = make_plane(kc, "k", S, H, cap, ks)
        V = make_plane(vc, "v", S, H, cap, vs)
        nr = []
        for side, P in (("k", K), ("v", V)):
            r = synth.kv_rows(CFG, side, li, s, h, 0, L)
            rows[(li, side)] = r
            for p0 in range(0, pre, 16384):
                n = min(16384, pre - p0)
                src = torch.randn((S, n, H, D), generator=gen, device="cuda")
                src[s, :, h] = torch.from_numpy(r[p0:p0 + n]).cuda()
                vit.vit_kv_append_quant(P, src, [p0] * S)
            x = torch.randn((S, ub, H, D), generator=gen, device="cuda")
            x[s, :, h] = torch.from_numpy(r[pre:pre + ub]).cuda()
            nr.append(x)
        qh = torch.randn((S, Hq, D), generator=gen, device="cuda")
        qh[s] = torch.from_numpy(synth.q_rows(CFG, li, s, Hq)).cuda()
        layers.append((K, V))
        new_rows.append(tuple(nr))
        q_dev.append(qh)
        q_host.append(qh.cpu().numpy())
        out.append(torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda"))
        torch.cuda.synchronize()
    n_splits = vit.vit_attn_default_splits(S, H, Hq, L)
    ws = torch.empty(vit.vit_attn_workspace_bytes(S, Hq, D, n_splits), dtype=torch.uint8, device="cuda")
    stream, astream = torch.cuda.Stream(), torch.cuda.Stream()
    counters = vit.merge_counters(layers[0][0])
    step = DecodeStep(layers, q_dev, new_rows, out, [L] * S, pre, Hq, n_splits, ws, stream, astream,
                      counters=counters)
    assert step.merged, "the ladder's decodes run as one merged launch each, as bench.py runs them"
    assert step.append_mode == "batched"
    say(f"[ladder step] one step (one multi-plane append), {n_splits} splits, decode and merge in one launch")
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    outs = [o.cpu().numpy() for o in out]
    # per-plane appends, then every decode, each call finished before the
    # next: the decode's summation order is fixed, so the outputs must match
    # bitwise
    say("[ladder step] serial replay with per-plane appends")
    for o in out:
        o.fill_(float("nan"))
    step.run_serial()
    serial = [o.cpu().numpy() for o in out]
    # the sampled unit's stored ubatch rows (logical codes, scales, norms)
    stored = []
    for li, (K, V) in enumerate(layers):
        s, h = _unit(li)
        sv = {}
        for side, P in (("k", K), ("v", V)):
            view = unit_view(P, s, h)
            sv[side] = {key: a[pre:pre + ub] for key, a in view.items()}
        stored.append(sv)
    assert int(counters.abs().sum()) == 0, "arrival counters not back at zero"
    # the overlapped schedule, on the ubatch scaled by 8
    for kv in new_rows:
        for x in kv:
            x.mul_(8.0)
    torch.cuda.synchronize()
    ostep = DecodeStep(layers, q_dev, new_rows, out, [L] * S, pre, Hq, n_splits, ws, stream, astream,
                       counters=counters, append_mode="overlapped")
    say("[ladder step] one overlapped step (appends on a second stream), ubatch x 8")
    for o in out:
        o.fill_(float("nan"))
    with torch.cuda.stream(stream):
        ostep()
    torch.cuda.synchronize()
    o_outs = [o.cpu().numpy() for o in out]
    for o in out:
        o.fill_(float("nan"))
    ostep.run_serial()
    o_serial = [o.cpu().numpy() for o in out]
    assert int(counters.abs().sum()) == 0, "arrival counters not back at zero"
    res = dict(outs=outs, serial=serial, o_outs=o_outs, o_serial=o_serial, q=q_host, rows=rows, stored=stored,
               cmap=cmap, n_splits=n_splits, G=Hq // H, pre=pre, ub=ub, L=L)
    del layers, step, ostep, new_rows, out, ws
    torch.cuda.empty_cache()
    return res


def test_ladder_map_covers_every_pair():
    """CPU: the 16 layers carry all 10 distinct (K, V) codec pairs of the
    seeded map, and the sampled units are 16 distinct (sequence, KV head)."""
    cmap = synth.codec_map(CFG)
    assert len(cmap) == 16 and len(set(cmap)) == 10
    assert len({_unit(li) for li in range(16)}) == 16


@pytest.mark.gpu
@pytest.mark.timeout(900)
@pytest.mark.parametrize("layer", range(16))
def test_ladder_step_layer(ladder_step, layer):
    r = ladder_step
    kc, vc = r["cmap"][layer]
    s, h = _unit(layer)
    G, pre, ub, L = r["G"], r["pre"], r["ub"], r["L"]
    say(f"[ladder step] layer {layer} ({kc},{vc}) unit ({s},{h}), splits {r['n_splits']}")
    ks = synth.sign_mask(CFG, layer, "k") if kc in ("rot4", "rot3") else None
    vs = synth.sign_mask(CFG, layer, "v") if vc in ("rot4", "rot3") else None
    kr, vr = r["rows"][(layer, "k")], r["rows"][(layer, "v")]
    # the ubatch rows as stored by the multi-plane append
    for side, codec, x, sg in (("k", kc, kr, ks), ("v", vc, vr, vs)):
        want = codecs.quantize(codec, x[pre:pre + ub], sg)
        got = r["stored"][layer][side]
        for key, w in want.items():
            g = got[key].astype(np.int8) if (codec == "q8_0" and key == "codes") else got[key]
            assert np.array_equal(g.reshape(w.shape), w), f"layer {layer} {side} {codec} ubatch {key} differ"
    ref = ref_unit(r["q"][layer][s, h * G:(h + 1) * G], kr, vr, kc, vc, 1.0 / math.sqrt(D), ks, vs)
    check_close(r["outs"][layer][s, h * G:(h + 1) * G], ref, f"ladder layer {layer} ({kc},{vc}) unit ({s},{h}) L={L}")
    # every output of the step is finite (no unit read poison), and the
    # step equals its serial replay bit for bit
    assert np.isfinite(r["outs"][layer]).all()
    assert np.array_equal(r["outs"][layer], r["serial"][layer]), f"layer {layer}: step != serial replay"
    # the overlapped schedule: equal to its serial replay, and not the
    # first step's output (its ubatch was scaled)
    assert np.isfinite(r["o_outs"][layer]).all()
    assert np.array_equal(r["o_outs"][layer], r["o_serial"][layer]), f"layer {layer}: overlapped != serial"
    assert not np.array_equal(r["o_outs"][layer], r["outs"][layer])
