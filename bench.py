#!/usr/bin/env python3
"""Decode-attention throughput of the quantized KV path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ladder]

A step is one pass of the whole hot path over one batch.  The default
workload is the ladder, the largest configuration: 16 layers whose K and V
tensors each carry a codec from a seeded map over {f16, q8_0, q4_0, rot4},
2 sequences, 32 query heads on 8 KV heads, head_dim 128, 200,704-row slots;
a step appends a 2048-row ubatch to every (layer, side) plane in one
vit_kv_append_quant_multi launch and then decodes one token per sequence
through all 16 layers (decode + split-K merge per layer).
``--append-schedule per_layer`` appends each layer's K and V with one
two-plane launch just before that layer's decode (the order a model's
forward pass allows); ``overlapped`` issues per-plane appends on a second
stream, decode l waiting for layer l's two appends only.  With the default
schedule the line also carries ``per_layer_appends_ms_per_step`` (and its
tokens/s), the same steps timed in the per-layer order.  The single-layer workloads (tiny, batched, lowbit,
rotated) are available with --workload: a step there is the fused append of
the new token's K/V rows, the decode and the merge.  ``--q-len N`` (2 .. 4,
single-layer workloads) makes each step verify N new tokens per sequence at
once, causal among themselves (vit_attn_decode_mq, all N rows appended by
the decode call); ``value`` then counts the N tokens of every sequence.

Inputs are synthetic (seeded device normals shaped like the workload) and
resident in HBM before timing starts.  Because the batched cache (143 MB)
fits in the 256 MB last-level cache, each timed step reads a different one of
R device replicas (R * footprint >= 1 GiB), round-robin.

The timed steps are eager C calls with pre-marshalled arguments.  Pass 1
gives the step time: ``--repeats`` blocks of exactly K steps, each between
device synchronisations; ``ms_per_step`` is the median block, with the
fastest and slowest blocks beside it.  In pass 2 every decode dispatch records a pair of
HIP events at its own start and end (vit_arm_kernel_events ->
hipExtLaunchKernel), so the duration covers the kernel alone, as rocprofv3's
kernel trace does; recording them costs the host about 16 us per launch,
which is why pass 1 runs without them.  ``--graph`` adds a pass that captures
each replica's step once into a HIP graph and replays one graph per step
(reported as ``graph_ms_per_step``).

Prints ONE JSON line.  ``value`` is decode tokens/s (sequences / step time).
``roofline`` describes the dominant kernel (decode): algorithmic KV bytes per
launch / its mean duration, against the 8 TB/s HBM peak, and against the
read bandwidth measured in the same run with the library's read-only
streaming kernel (vit_stream_read, 1 GiB).  ``traffic``
is the HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE (scaled by
a copy-kernel calibration), read from profiles/ only when it was measured on
the current kernel sources.  ``cpu_baseline`` times the numpy oracle on the
host for the same step on every core this process may use, with the 1-core
time and the CPU model (a baseline, not a target); it runs before the GPU
is touched.
"""

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOADS = ("tiny", "batched", "lowbit", "rotated", "ladder")
D = 128


# each measured kernel's own sources (the kernel, its device helpers, its argument block)
KERNEL_SOURCES = {
    "decode": ("decode_impl.h", "decode_k*.hip", "vit_device.h", "vit_launch.h"),
    "transcode": ("append.hip", "decode_impl.h", "vit_device.h", "vit_launch.h"),
    "probe_logits": ("probe.hip", "decode_impl.h", "vit_device.h", "vit_launch.h"),
    "append": ("append.hip", "decode_impl.h", "vit_device.h", "vit_launch.h"),
}
TRANSCODE_PAIRS = ("f16:q8_0", "f16:q4_0", "f16:rot4", "f16:rot3", "q8_0:q4_0", "q8_0:rot4", "q8_0:rot3", "q4_0:rot3")
CODEC_NAMES = ("f16", "q8_0", "q4_0", "rot4", "rot3")
ROTATED = ("rot4", "rot3")


def kernel_source_hash(kind="decode"):
    """sha256 prefix over one measured kernel's sources."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_kv_cache_append_amd", "csrc")
    for p in sorted(q for pat in KERNEL_SOURCES[kind] for q in glob.glob(os.path.join(csrc, pat))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _row_bytes(codec):
    return {"f16": 256, "q8_0": 136, "q4_0": 72, "rot4": 74, "rot3": 56}[codec]


def _device_rows(torch, gen, shape, dist, scales=None):
    x = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
    if dist == "lognormal" and scales is not None:
        x *= scales
    elif dist == "outlier":
        x[..., :2] *= 20.0
    elif dist == "heavy":
        # Student-t(3) = z / sqrt(chi2_3 / 3), drawn on the device
        hit = torch.rand(shape, generator=gen, device="cuda") < 0.01
        z = torch.randn((3,) + tuple(shape), generator=gen, device="cuda")
        t = torch.randn(shape, generator=gen, device="cuda") / torch.sqrt((z * z).sum(0) / 3.0)
        x = torch.where(hit, t, x)
    return x


class Layer:
    """K and V planes of one layer plus cold-cache replicas."""

    def __init__(self, vit, cfg, kc, vc, replicas, signs_k, signs_v):
        S, H, cap = cfg["seqs"], cfg["hkv"], cfg["capacity"]
        self.K = [vit.KVPlane(kc, "k", S, H, cap, signs_k)]
        self.V = [vit.KVPlane(vc, "v", S, H, cap, signs_v)]
        self.replicas = replicas
        self.kc, self.vc = kc, vc

    def make_replicas(self, vit):
        for _ in range(self.replicas - 1):
            k = vit.KVPlane.like(self.K[0])
            v = vit.KVPlane.like(self.V[0])
            k.copy_from(self.K[0])
            v.copy_from(self.V[0])
            self.K.append(k)
            self.V.append(v)


def run_gpu(args):
    import numpy as np
    import torch

    import quantized_kv_cache_append_amd as vit
    import synth

    wl = args.workload
    cfg = synth.CONFIGS[wl]
    S, Hq, H, cap, L = cfg["seqs"], cfg["hq"], cfg["hkv"], cfg["capacity"], cfg["ctx"]
    QL = args.q_len
    if QL > 1 and ("ubatch" in cfg or (Hq // H) * QL > 16 or QL > 4):
        raise SystemExit(f"--q-len {QL} needs a single-layer workload with (n_q_heads / n_kv_heads) x q_len <= 16")
    cmap = synth.codec_map(wl)
    if args.codecs:
        if cfg["layers"] != 1:
            raise SystemExit("--codecs needs a single-layer workload")
        cmap = [tuple(args.codecs.split(":"))]
    n_layers = cfg["layers"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0x5EED2026 + synth.SEED_ID[wl])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    kv_bytes = sum(S * H * L * (_row_bytes(kc) + _row_bytes(vc)) for kc, vc in cmap)
    footprint = sum(S * H * cap * (_row_bytes(kc) + _row_bytes(vc)) for kc, vc in cmap)
    # at most 256 replicas: the tiny workload (200 KB) is launch-bound whatever the cache state
    replicas = args.replicas if args.replicas else min(256, max(1, math.ceil((1 << 30) / footprint)))
    if n_layers > 1:
        replicas = 1  # the ladder's 13.8 GB footprint already dwarfs every cache

    print(f"# workload {cfg['name']}: S={S} Hq={Hq} Hkv={H} L={L} layers={n_layers} "
          f"codecs={cmap if n_layers == 1 else 'ladder'} replicas={replicas}", file=sys.stderr, flush=True)

    layers = []
    chan_scale = {}
    for li, (kc, vc) in enumerate(cmap):
        ks = synth.sign_mask(wl, li, "k") if kc in ROTATED else None
        vs = synth.sign_mask(wl, li, "v") if vc in ROTATED else None
        lay = Layer(vit, cfg, kc, vc, replicas, ks, vs)
        for side, plane in (("k", lay.K[0]), ("v", lay.V[0])):
            sc = None
            if cfg["dist"] == "lognormal":
                sc = torch.exp(torch.randn((1, 1, H, D), generator=gen, device="cuda"))
                chan_scale[(li, side)] = sc
            pre = cfg.get("prefill", L - QL if cfg["fused_append"] else L)
            # fill the prefix in chunks to bound the fp32 staging buffer
            chunk = 16384
            for p0 in range(0, pre, chunk):
                n = min(chunk, pre - p0)
                src = _device_rows(torch, gen, (S, n, H, D), cfg["dist"], sc)
                vit.vit_kv_append_quant(plane, src, [p0] * S)
            del src
        lay.make_replicas(vit)
        layers.append(lay)
        if n_layers > 1:
            torch.cuda.synchronize()
            print(f"# filled layer {li} ({kc}/{vc})", file=sys.stderr, flush=True)
    torch.cuda.synchronize()

    # per-step inputs
    qshape = (S, Hq, D) if QL == 1 else (S, QL, Hq, D)
    q = [_device_rows(torch, gen, qshape, cfg["dist"]) for _ in range(n_layers)]
    if "ubatch" in cfg:
        T, p_new = cfg["ubatch"], cfg["prefill"]
    else:
        T, p_new = QL, L - QL
    new_rows = [[_device_rows(torch, gen, (S, T, H, D), cfg["dist"], chan_scale.get((li, s)))
                 for s in ("k", "v")] for li in range(n_layers)]
    n_splits = args.splits if args.splits else vit.vit_attn_default_splits(S, H, Hq, L)
    ws = torch.empty(vit.vit_attn_workspace_bytes(S, Hq * QL, D, n_splits), dtype=torch.uint8, device="cuda")
    out = [torch.empty(qshape, dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    lens = [L] * S
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()  # the bench's own stream (default priority): it can be captured
    # The ladder's ubatch appends, scheduled by the step driver
    # (quantized_kv_cache_append_amd.step): by default one launch appends to
    # all planes before the decodes; --append-schedule per_layer appends each
    # layer's pair just before its decode; overlapped puts per-plane appends
    # on a second stream (default priority too), decode l waiting only for
    # layer l's appends and each step's appends for the previous step's
    # decodes (they rewrite the rows those read).
    fused = "ubatch" not in cfg
    append_mode = args.append_schedule
    astream = None if fused else torch.cuda.Stream()
    # decode and split merge in one launch (vit_attn_decode_merged) where the
    # shape allows it; the arrival counters are zeroed once and every call
    # leaves them zero
    merged = (n_splits > 1 and not args.no_merge and vit.merge_fits(Hq, H, QL, n_splits))
    counters = torch.zeros((S, H), dtype=torch.int32, device="cuda") if merged else None

    # every call of a step, marshalled once per replica (the host then only
    # issues the C calls, so the GPU queue never runs dry).  One (or q_len)
    # new token(s) per sequence: their K/V rows go through the decode call's
    # fused append.
    calls = []
    for r in range(replicas):
        if not fused:
            from quantized_kv_cache_append_amd.step import DecodeStep

            calls.append(DecodeStep([(lay.K[r], lay.V[r]) for lay in layers], q, new_rows, out, lens, p_new, Hq,
                                    n_splits, ws, stream, astream, counters=counters, append_mode=append_mode))
            continue
        dec = []
        for li, lay in enumerate(layers):
            kn, vn = new_rows[li]
            # [S][H][128] rows for one token, [S][q_len][H][128] for several
            k_in = kn[:, 0].contiguous() if QL == 1 else kn
            v_in = vn[:, 0].contiguous() if QL == 1 else vn
            if merged:
                shp = (S, QL, Hq, D)  # new rows kn, vn: [S][q_len][Hkv][128]
                d = vit.prepare_merged(lay.K[r], lay.V[r], q[li].reshape(shp), Hq, QL, lens, out[li].reshape(shp),
                                       ws, counters, k_new=kn, v_new=vn, n_splits=n_splits, stream=stream)
                dec.append((d, None))
                continue
            d = vit.prepare_decode(lay.K[r], lay.V[r], q[li], Hq, lens, out[li], n_splits=n_splits,
                                   k_new=k_in, v_new=v_in, workspace=ws if n_splits > 1 else None,
                                   stream=stream, q_len=QL if QL > 1 else None)
            red = (vit.prepare_reduce(ws, S, Hq * QL, n_splits, lay.V[r], out[li], stream=stream)
                   if n_splits > 1 else None)
            dec.append((d, red))
        calls.append(dec)

    def step(i, ev=None):
        c = calls[i % replicas]
        if not fused:
            c(ev)
            return
        for li, (d, red) in enumerate(c):
            if ev is not None:
                # the decode dispatch itself records this pair at its start and end
                arm(ev[0][li], ev[1][li])
            d()
            if red is not None:
                red()

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    evs = [([torch.cuda.Event(enable_timing=True) for _ in range(n_layers)],
            [torch.cuda.Event(enable_timing=True) for _ in range(n_layers)]) for _ in range(args.steps)]
    for pair in evs:  # create the HIP events (torch does so on first record)
        for e in pair[0] + pair[1]:
            e.record(stream)
    arm = vit.vit_arm_kernel_events
    # Pass 1, the step throughput: the timed steps as eager C calls, in
    # `repeats` blocks of exactly K steps, each bracketed by a device
    # synchronisation; the median block gives ms_per_step.
    block_ms = []
    for rep in range(args.repeats):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                step(args.warmup + rep * args.steps + i)
        torch.cuda.synchronize()
        block_ms.append(1e3 * (time.perf_counter() - t0) / args.steps)
    eager_ms_per_step = float(np.median(block_ms))
    assert all(np.isfinite(o.cpu().numpy()).all() for o in out), "non-finite decode output"
    # Pass 2, the decode kernel's duration: the same steps again, each decode
    # dispatch recording its own start/stop events.  (Recording them costs the
    # host about 16 us per launch, so pass 1 runs without them.)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    dec_ms = [evs[i][0][li].elapsed_time(evs[i][1][li]) for i in range(args.steps) for li in range(n_layers)]

    # Optional pass 2: each replica's step (the same C calls) captured once
    # into a HIP graph and replayed, one graph launch per step.  (On this
    # stack a graph launch costs about as much host and dispatch time as the
    # eager calls, so the eager pass stays the default.)
    graph_ms_per_step = None
    mode, ms_per_step = "eager (pre-marshalled C calls)", eager_ms_per_step
    if args.graph:
        graphs = []
        with torch.cuda.stream(stream):
            for r in range(replicas):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step(r)
                graphs.append(g)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                graphs[i % replicas].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                graphs[(args.warmup + i) % replicas].replay()
        torch.cuda.synchronize()
        graph_ms_per_step = 1e3 * (time.perf_counter() - t0) / args.steps
        assert all(np.isfinite(o.cpu().numpy()).all() for o in out), "non-finite decode output (graph replay)"
        del graphs
    per_layer_ms = None
    if not fused and append_mode == "batched":
        # the same step in the order a model's forward pass allows: each
        # layer's K and V appended by one two-plane launch just before its
        # decode (reported beside ms_per_step, which times the workload's
        # all-appends-first order)
        from quantized_kv_cache_append_amd.step import DecodeStep

        pl = DecodeStep([(lay.K[0], lay.V[0]) for lay in layers], q, new_rows, out, lens, p_new, Hq, n_splits, ws,
                        stream, astream, counters=counters, append_mode="per_layer")
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                pl()
        pl_blocks = []
        for rep in range(args.repeats):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            with torch.cuda.stream(stream):
                for _ in range(args.steps):
                    pl()
            torch.cuda.synchronize()
            pl_blocks.append(1e3 * (time.perf_counter() - t0) / args.steps)
        per_layer_ms = float(np.median(pl_blocks))
        del pl
    if not fused:
        # The step must compute what the per-plane calls issued serially do.
        # The timed steps append the same rows every time, which would hide a
        # decode that ran before its layer's appends; so the ubatch rows are
        # scaled by 8 first (their logits then dominate the softmax, and a
        # stale read would move the output by O(1)), then one step and the
        # per-plane appends followed by the decodes, each call finished
        # before the next, must agree bit for bit (the decode's summation
        # order is fixed).
        for kv in new_rows:
            for x in kv:
                x.mul_(8.0)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            step(0)
        torch.cuda.synchronize()
        stepped = [o.clone() for o in out]
        with torch.cuda.stream(stream):
            calls[0].run_serial()
        for li, (a, b) in enumerate(zip(stepped, out)):
            assert torch.equal(a, b), f"layer {li}: {append_mode} step differs from the serial per-plane calls"
        print(f"# step check: {append_mode} step == serial per-plane calls, bit for bit, all layers", file=sys.stderr,
              flush=True)
    dec_mean_ms = float(np.mean(dec_ms))
    per_launch_bytes = kv_bytes / n_layers
    # algorithmic bytes of all timed decode launches / their summed duration
    achieved = kv_bytes * args.steps / (float(np.sum(dec_ms)) * 1e-3) / 1e9
    return dict(cfg=cfg, wl=wl, cmap=cmap, S=S, Hq=Hq, H=H, L=L, n_layers=n_layers, T=T, QL=QL, mode=mode,
                merge="in-kernel (vit_attn_decode_merged)" if merged else ("reduce kernel" if n_splits > 1 else "none"),
                appends=None if fused else {
                    "batched": "one vit_kv_append_quant_multi launch before the decodes",
                    "per_layer": "one two-plane vit_kv_append_quant_multi launch before each layer's decode",
                    "overlapped": "per-plane vit_kv_append_quant on a second stream, overlapped with the decodes",
                }[append_mode],
                replicas=replicas, n_splits=n_splits, ms_per_step=ms_per_step, graph_ms_per_step=graph_ms_per_step,
                per_layer_ms_per_step=per_layer_ms,
                block_ms=block_ms,
                dec_mean_ms=dec_mean_ms,
                dec_min_ms=float(np.min(dec_ms)), kv_bytes=kv_bytes, per_launch_bytes=per_launch_bytes,
                achieved_gbs=achieved)


def run_transcode(args):
    """One VBR degrade step of one (layer, side) tensor of the ladder
    workload's slots: every row of 2 sequences x 8 KV heads x 200,704 rows
    re-encoded from the source codec into a destination plane.  The source
    is filled once (seeded device rows, log-normal channel scales); each timed
    step re-encodes it into the same destination."""
    import numpy as np
    import torch

    import quantized_kv_cache_append_amd as vit
    import synth

    src_c, dst_c = args.transcode.split(":")
    cfg = synth.CONFIGS["ladder"]
    S, H, cap = cfg["seqs"], cfg["hkv"], cfg["capacity"]
    side = args.side
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0x5EED2026 + 77)
    torch.cuda.set_device(torch.device("cuda:0"))
    signs = synth.sign_mask("ladder", 0, side) if dst_c in ROTATED else None
    src = vit.KVPlane(src_c, side, S, H, cap)
    dst = vit.KVPlane(dst_c, side, S, H, cap, signs)
    sc = torch.exp(torch.randn((1, 1, H, D), generator=gen, device="cuda"))
    for p0 in range(0, cap, 16384):
        n = min(16384, cap - p0)
        vit.vit_kv_append_quant(src, _device_rows(torch, gen, (S, n, H, D), "lognormal", sc), [p0] * S)
    torch.cuda.synchronize()
    print(f"# transcode {src_c} -> {dst_c}, side {side}: S={S} Hkv={H} rows={cap}", file=sys.stderr, flush=True)
    stream = torch.cuda.Stream()
    call = vit.prepare_transcode(src, dst, [cap] * S, stream=stream)
    arm = vit.vit_arm_kernel_events
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            call()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            call()
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t0) / args.steps
    with torch.cuda.stream(stream):
        for a, b in evs:
            arm(a, b)
            call()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    rows = S * H * cap
    per_launch = rows * (_row_bytes(src_c) + _row_bytes(dst_c))
    return dict(src_c=src_c, dst_c=dst_c, side=side, S=S, H=H, cap=cap, rows=rows, ms_per_step=ms_per_step,
                mean_ms=float(np.mean(ms)), min_ms=float(np.min(ms)), per_launch_bytes=per_launch,
                achieved_gbs=per_launch / (float(np.mean(ms)) * 1e-3) / 1e9)


def cpu_baseline_transcode(r, budget_s=15.0):
    """oracle.vbr.transcode on the host for rows of one (sequence, KV head)
    stream (its source codes prepared untimed), scaled to the step."""
    import numpy as np

    from oracle import codecs, vbr
    import synth

    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    n = 16384
    rows = synth.kv_rows("ladder", r["side"], 0, 0, 0, 0, n)
    q_src = codecs.quantize(r["src_c"], rows)
    signs = synth.sign_mask("ladder", 0, r["side"]) if r["dst_c"] in ROTATED else None
    done = 0
    t0 = time.perf_counter()
    while True:
        vbr.transcode(r["src_c"], r["dst_c"], q_src, dst_signs=signs)
        done += n
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    return {"value": done / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": (f"{done} rows ({r['src_c']} -> {r['dst_c']}) of one (sequence, KV head) stream in "
                       f"{n}-row calls, {el:.1f} s on 1 thread; step = {r['rows']} rows")}


def run_probe(args):
    """One attention-probe scoring event over a workload's K plane (layer 0):
    per-cell softmax mass of every query head with decay 0.9, then the
    eviction choice (4 sink and 256 recent cells protected, L/16 evicted).
    Cold-cache replicas as for decode."""
    import numpy as np
    import torch

    import quantized_kv_cache_append_amd as vit
    import synth

    wl = args.workload
    cfg = synth.CONFIGS[wl]
    S, Hq, H, cap, L = cfg["seqs"], cfg["hq"], cfg["hkv"], cfg["capacity"], cfg["ctx"]
    kc = args.codecs.split(":")[0] if args.codecs else synth.codec_map(wl)[0][0]
    ks = synth.sign_mask(wl, 0, "k") if kc in ROTATED else None
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0x5EED2026 + 99 + synth.SEED_ID[wl])
    torch.cuda.set_device(torch.device("cuda:0"))
    k_bytes = S * H * L * _row_bytes(kc)
    replicas = args.replicas if args.replicas else min(256, max(1, math.ceil((1 << 30) / (S * H * cap * _row_bytes(kc)))))
    planes = [vit.KVPlane(kc, "k", S, H, cap, ks)]
    sc = torch.exp(torch.randn((1, 1, H, D), generator=gen, device="cuda")) if cfg["dist"] == "lognormal" else None
    for p0 in range(0, L, 16384):
        n = min(16384, L - p0)
        vit.vit_kv_append_quant(planes[0], _device_rows(torch, gen, (S, n, H, D), cfg["dist"], sc), [p0] * S)
    for _ in range(replicas - 1):
        k = vit.KVPlane.like(planes[0])
        k.copy_from(planes[0])
        planes.append(k)
    q = _device_rows(torch, gen, (S, Hq, D), cfg["dist"])
    scores = torch.zeros((S, cap), dtype=torch.float32, device="cuda")
    ws = torch.empty(vit.vit_attn_probe_workspace_bytes(S, Hq, cap), dtype=torch.uint8, device="cuda")
    n_evict = L // 16
    rows_out = torch.empty((S, n_evict), dtype=torch.int64, device="cuda")
    n_out = torch.empty((S,), dtype=torch.int32, device="cuda")
    sel_ws = torch.empty(vit.vit_probe_select_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    print(f"# probe {cfg['name']}: K={kc} S={S} Hq={Hq} Hkv={H} L={L} replicas={replicas}", file=sys.stderr, flush=True)
    stream = torch.cuda.Stream()
    calls = [(vit.prepare_probe(kp, q, Hq, [L] * S, scores, ws, decay=0.9, stream=stream),
              vit.prepare_select(scores, [L] * S, 4, 256, n_evict, rows_out, n_out, sel_ws, stream=stream))
             for kp in planes]
    arm = vit.vit_arm_kernel_events

    def step(i, ev=None):
        pr, sel = calls[i % replicas]
        if ev is not None:
            arm(ev[0], ev[1])
        pr()
        sel()

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            step(args.warmup + i)
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t0) / args.steps
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    assert np.isfinite(scores.cpu().numpy()).all(), "non-finite probe scores"
    per_launch = k_bytes + S * Hq * L * 4  # K read + logits written
    return dict(cfg=cfg, wl=wl, kc=kc, S=S, Hq=Hq, H=H, L=L, replicas=replicas, ms_per_step=ms_per_step,
                mean_ms=float(np.mean(ms)), min_ms=float(np.min(ms)), per_launch_bytes=per_launch,
                achieved_gbs=per_launch / (float(np.mean(ms)) * 1e-3) / 1e9, n_evict=n_evict)


def cpu_baseline_probe(r, budget_s=15.0):
    """oracle.probe (cell_mass, decay_update, select_evictions) as it stands,
    over one sequence's first 8192 cells, scaled to the step."""
    import numpy as np

    from oracle import probe
    import synth

    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    wl, H, Hq, L, kc = r["wl"], r["H"], r["Hq"], r["L"], r["kc"]
    n = min(L, 8192)
    ks = synth.sign_mask(wl, 0, "k") if kc in ROTATED else None
    keys = np.stack([synth.kv_rows(wl, "k", 0, 0, h, 0, n) for h in range(H)])
    q = synth.q_rows(wl, 0, 0, Hq)
    done = 0
    t0 = time.perf_counter()
    while True:
        mass = probe.cell_mass(q, keys, kc, 1.0 / math.sqrt(D), ks)
        sc = probe.decay_update(np.zeros(n), mass, 0.9)
        probe.select_evictions(sc, n, 4, 256, n // 16)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    per_seq = el / done * (L / n)
    return {"value": 1.0 / (per_seq * r["S"]), "unit": "scoring events/s", "cores": 1, "kind": "oracle",
            "sample": (f"{done} passes over sequence 0 ({H} KV heads x {n} cells), {el:.1f} s on 1 thread, scaled "
                       f"to {r['S']} sequences x {L} cells; pass = oracle cell mass of {Hq} query heads (its key "
                       "quantization included) + decay + eviction choice")}


def main_probe(args):
    r = run_probe(args)
    line = {
        "metric": "attention-probe scoring events per second + effective K-read GB/s (% of HBM peak), 1 GPU",
        "value": round(1e3 / r["ms_per_step"], 1),
        "unit": "scoring events/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{r['kc']} K codes, fp16 MFMA operands (hi+lo query), fp32 logits and masses",
        "data": "synthetic (seeded device normals shaped like the workload; no model weights or dataset)",
        "config": {"workload": f"probe_{r['cfg']['name']}", "n_seqs": r["S"], "n_q_heads": r["Hq"],
                   "n_kv_heads": r["H"], "head_dim": D, "context": r["L"], "k_codec": r["kc"], "decay": 0.9,
                   "n_sink": 4, "n_recent": 256, "n_evict": r["n_evict"], "cold_cache_replicas": r["replicas"],
                   "launch": "eager (pre-marshalled C calls)"},
        "roofline": {
            "bound": "hbm",
            "kernel": "probe_logits_kernel",
            "achieved": round(r["achieved_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["achieved_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": load_traffic("probe_logits", r["cfg"]["name"]),
            "algorithmic_bytes_per_launch": r["per_launch_bytes"],
            "mean_launch_ms": round(r["mean_ms"], 5),
            "min_launch_ms": round(r["min_ms"], 5),
        },
        "kernel_source_hash": kernel_source_hash("probe_logits"),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_probe(r, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def run_append(args):
    """One ubatch append of the ladder workload: 2048 new rows for each of
    2 sequences x 8 KV heads (fp32 in, one codec, one side), at rows
    198,656 .. 200,703 of its 200,704-row slots."""
    import numpy as np
    import torch

    import quantized_kv_cache_append_amd as vit
    import synth

    codec, side = args.append, args.side
    cfg = synth.CONFIGS["ladder"]
    S, H, cap, pre, ub = cfg["seqs"], cfg["hkv"], cfg["capacity"], cfg["prefill"], cfg["ubatch"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0x5EED2026 + 55)
    torch.cuda.set_device(torch.device("cuda:0"))
    signs = synth.sign_mask("ladder", 0, side) if codec in ROTATED else None
    plane = vit.KVPlane(codec, side, S, H, cap, signs)
    sc = torch.exp(torch.randn((1, 1, H, D), generator=gen, device="cuda"))
    # distinct source buffers, round-robin, so the 16.8 MB fp32 ubatch is not served from the cache
    n_src = 16
    srcs = [_device_rows(torch, gen, (S, ub, H, D), "lognormal", sc) for _ in range(n_src)]
    torch.cuda.synchronize()
    print(f"# append {codec} side {side}: S={S} Hkv={H} rows={ub} at {pre}", file=sys.stderr, flush=True)
    stream = torch.cuda.Stream()
    calls = [vit.prepare_append(plane, src, [pre] * S, stream=stream) for src in srcs]
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            calls[i % n_src]()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            calls[i % n_src]()
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t0) / args.steps
    for pair in evs:  # create the HIP events (torch does so on first record)
        for e in pair:
            e.record(stream)
    torch.cuda.synchronize()
    # the append dispatch itself records each pair at its kernel's start and end
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            vit.vit_arm_kernel_events(evs[i][0], evs[i][1])
            calls[i % n_src]()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    rows = S * H * ub
    per_launch = rows * (4 * D + _row_bytes(codec))  # fp32 row read + encoded row written
    return dict(codec=codec, side=side, S=S, H=H, ub=ub, rows=rows, ms_per_step=ms_per_step,
                mean_ms=float(np.mean(ms)), min_ms=float(np.min(ms)), per_launch_bytes=per_launch,
                achieved_gbs=per_launch / (float(np.mean(ms)) * 1e-3) / 1e9)


def cpu_baseline_append(r, budget_s=15.0):
    """oracle.codecs.quantize on the host for rows of one stream, scaled."""
    from oracle import codecs
    import synth

    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    n = 2048
    rows = synth.kv_rows("ladder", r["side"], 0, 0, 0, 0, n)
    signs = synth.sign_mask("ladder", 0, r["side"]) if r["codec"] in ROTATED else None
    done = 0
    t0 = time.perf_counter()
    while True:
        codecs.quantize(r["codec"], rows, signs)
        done += n
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    return {"value": done / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} rows ({r['codec']}) in {n}-row calls, {el:.1f} s on 1 thread; step = {r['rows']} rows"}


def main_append(args):
    r = run_append(args)
    tag = f"{r['codec']}_{r['side']}"
    line = {
        "metric": "KV append: rows quantized and stored per second + effective GB/s (% of HBM peak), 1 GPU",
        "value": round(r["rows"] / (r["ms_per_step"] * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"fp32 rows encoded to {r['codec']}",
        "data": "synthetic (seeded device normals with log-normal channel scales; no model weights or dataset)",
        "config": {"workload": f"append_{tag}", "n_seqs": r["S"], "n_kv_heads": r["H"], "head_dim": D,
                   "ubatch": r["ub"], "codec": r["codec"], "side": r["side"],
                   "launch": "eager (pre-marshalled C call)"},
        "roofline": {
            "bound": "hbm",
            "kernel": "append_kernel",
            "achieved": round(r["achieved_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["achieved_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": load_traffic("append", tag),
            "algorithmic_bytes_per_launch": r["per_launch_bytes"],
            "mean_launch_ms": round(r["mean_ms"], 5),
            "min_launch_ms": round(r["min_ms"], 5),
        },
        "kernel_source_hash": kernel_source_hash("append"),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_append(r, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def main_transcode(args):
    r = run_transcode(args)
    tag = f"{r['src_c']}_to_{r['dst_c']}_{r['side']}"
    line = {
        "metric": "VBR degrade step: rows re-encoded per second + effective GB/s (% of HBM peak), 1 GPU",
        "value": round(r["rows"] / (r["ms_per_step"] * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{r['src_c']} decoded exactly to fp32, encoded to {r['dst_c']}",
        "data": "synthetic (seeded device normals with log-normal channel scales; no model weights or dataset)",
        "config": {"workload": f"transcode_{tag}", "n_seqs": r["S"], "n_kv_heads": r["H"], "head_dim": D,
                   "rows_per_stream": r["cap"], "side": r["side"], "src_codec": r["src_c"], "dst_codec": r["dst_c"],
                   "launch": "eager (pre-marshalled C call)"},
        "roofline": {
            "bound": "hbm",
            "kernel": "transcode_kernel",
            "achieved": round(r["achieved_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["achieved_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": load_traffic("transcode", tag),
            "algorithmic_bytes_per_launch": r["per_launch_bytes"],
            "mean_launch_ms": round(r["mean_ms"], 5),
            "min_launch_ms": round(r["min_ms"], 5),
        },
        "kernel_source_hash": kernel_source_hash("transcode"),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_transcode(r, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def measure_stream_read(n_bytes=1 << 30, launches=10):
    """GB/s of the library's read-only streaming kernel (vit_stream_read: 16-byte
    nontemporal loads of a 1 GiB buffer over the whole GPU, nothing else), the
    read bandwidth this part reaches in practice; kernel events recorded by its
    dispatch, mean over the launches."""
    import torch

    import quantized_kv_cache_append_amd as vit

    buf = torch.ones(n_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(3):
            vit.vit_stream_read(buf, sink, stream=stream)
        for a, b in evs:
            vit.vit_arm_kernel_events(a, b)
            vit.vit_stream_read(buf, sink, stream=stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / launches
    del buf
    torch.cuda.empty_cache()
    return n_bytes / (ms * 1e-3) / 1e9


def run_copy_calibration(steps):
    """A plain device copy of known size, for scaling rocprofv3 counters."""
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": steps}))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def _cpu_items(wl, q_len):
    """The sampled (layer, sequence, KV head) units of a workload's step for
    the CPU baseline: one unit of every layer for the ladder (so every codec
    pair of its map is timed), up to 16 units of a single-layer workload."""
    import synth

    cfg = synth.CONFIGS[wl]
    S, H = cfg["seqs"], cfg["hkv"]
    if cfg["layers"] > 1:
        return [(li, (li // H) % S, (3 * li + 1) % H) for li in range(cfg["layers"])]
    units = [(0, s, h) for s in range(S) for h in range(H)]
    return units[:: max(1, len(units) // 16)][:16]


_CPU_ITEMS = None


def _cpu_prepare(wl, q_len, rows, n_new, items):
    """Untimed set-up of the sampled units: each unit's cached rows encoded by
    the oracle, its new rows and its query heads."""
    global _CPU_ITEMS
    from oracle import codecs
    import synth

    cfg = synth.CONFIGS[wl]
    Hq, H = cfg["hq"], cfg["hkv"]
    G = Hq // H
    cmap = synth.codec_map(wl)
    prep = []
    for (li, s, h) in items:
        kc, vc = cmap[li]
        ks = synth.sign_mask(wl, li, "k") if kc in ROTATED else None
        vs = synth.sign_mask(wl, li, "v") if vc in ROTATED else None
        kx = synth.kv_rows(wl, "k", li, s, h, 0, rows)
        vx = synth.kv_rows(wl, "v", li, s, h, 0, rows)
        qx = synth.q_rows(wl, li, s, Hq)[h * G:(h + 1) * G]
        prep.append((kc, vc, ks, vs, codecs.quantize(kc, kx[:rows - n_new], ks),
                     codecs.quantize(vc, vx[:rows - n_new], vs), kx[rows - n_new:], vx[rows - n_new:], qx, q_len))
    _CPU_ITEMS = prep
    return len(prep)


_CPU_BARRIER = None


_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def _one_thread():
    """Hold numpy's BLAS to one thread in this process (numpy loaded first,
    so that its library is there to be limited)."""
    import numpy  # noqa: F401

    try:
        from threadpoolctl import threadpool_limits

        return threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        return None


def _cpu_pool_init(barrier):
    """Pool worker start-up: one BLAS thread per worker process (set before
    numpy is imported here, and again through threadpoolctl)."""
    global _CPU_BARRIER
    for v in _THREAD_VARS:
        os.environ[v] = "1"
    _one_thread()
    _CPU_BARRIER = barrier


def _cpu_pool_prepare(a):
    _cpu_prepare(*a)
    _CPU_BARRIER.wait()


def _cpu_unit(i):
    """Timed work of one sampled unit: encode its new K/V rows, decode the
    cache, fp64 attention of each new query token over the rows up to its
    own.  Returns (encode seconds, decode + attention seconds)."""
    import numpy as np

    from oracle import attention, codecs

    kc, vc, ks, vs, kq, vq, kn, vn, qx, ql = _CPU_ITEMS[i]
    t0 = time.perf_counter()
    kq_new = codecs.quantize(kc, kn, ks) if len(kn) else None
    vq_new = codecs.quantize(vc, vn, vs) if len(vn) else None
    t1 = time.perf_counter()
    kq2 = kq if kq_new is None else {k: np.concatenate([kq[k], kq_new[k]]) for k in kq}
    vq2 = vq if vq_new is None else {k: np.concatenate([vq[k], vq_new[k]]) for k in vq}
    kd, vd = codecs.dequant(kc, kq2, ks), codecs.dequant(vc, vq2, vs)
    n = kd.shape[0]
    for t in range(ql):  # token t sees rows 0 .. n - ql + t (the timing does not depend on q's values)
        attention.attend(qx, kd[:n - ql + 1 + t], vd[:n - ql + 1 + t], 1.0 / math.sqrt(D))
    return t1 - t0, time.perf_counter() - t1


def cpu_baseline(wl, q_len, budget_s=15.0):
    """The numpy oracle, untuned, on the host's cores: for sampled
    (layer, sequence, KV head) units of the step, encode the new rows, decode
    the cache and attend in fp64; scaled to the whole step.

    One pass runs the units one after another on one core (the 1-core time,
    also split into encode and attention); a second pass runs them in a
    process pool over every core this process may use, for a wall-clock
    time.  Contexts longer than 8192 rows are attended over an 8192-row
    slice (the new rows included) and the attention time scaled by
    L / slice.  Runs before the process touches the GPU (spawned workers)."""
    import multiprocessing as mp

    import numpy as np
    import synth

    cfg = synth.CONFIGS[wl]
    S, H, L, n_layers = cfg["seqs"], cfg["hkv"], cfg["ctx"], cfg["layers"]
    n_new = cfg.get("ubatch", q_len)        # rows encoded per unit per step
    rows = min(L, max(8192, n_new + 4096))  # rows attended in the sample
    att_scale = L / rows
    items = _cpu_items(wl, q_len)
    units_per_layer = S * H
    cores = len(os.sched_getaffinity(0))
    # 1 core: every sampled unit once (after one untimed run of each)
    limiter = _one_thread()
    _cpu_prepare(wl, q_len, rows, n_new, items)
    for i in range(len(items)):
        _cpu_unit(i)
    tq, ta = np.zeros(len(items)), np.zeros(len(items))
    reps1 = 0
    t0 = time.perf_counter()
    while True:
        for i in range(len(items)):
            a, b = _cpu_unit(i)
            tq[i] += a
            ta[i] += b
        reps1 += 1
        if time.perf_counter() - t0 >= budget_s / 3:
            break
    tq /= reps1
    ta /= reps1
    if limiter is not None:
        limiter.restore_original_limits()
    per_layer = {}
    for (li, _, _), a, b in zip(items, tq, ta):
        per_layer.setdefault(li, []).append(a + b * att_scale)
    # each layer's units cost the mean of its sampled units
    one_core_step = sum(units_per_layer * float(np.mean(v)) for v in per_layer.values()) * (n_layers / len(per_layer))
    sample_work = float(np.sum(tq + ta))  # one pass over the sampled units, as executed
    # all cores: the same units in a process pool.  Every worker prepares
    # them (untimed) and waits at a barrier, so each worker takes exactly one
    # set-up task and none is still setting up when the timing starts.
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(cores)
    reps = max(math.ceil(2 * cores / len(items)), math.ceil((budget_s / 3) * cores / sample_work))
    with ctx.Pool(cores, initializer=_cpu_pool_init, initargs=(barrier,)) as pool:
        pool.map(_cpu_pool_prepare, [(wl, q_len, rows, n_new, items)] * cores, chunksize=1)
        pool.map(_cpu_unit, list(range(len(items))) * math.ceil(cores / len(items)), chunksize=1)  # warm
        t0 = time.perf_counter()
        pool.map(_cpu_unit, list(range(len(items))) * reps, chunksize=1)
        wall = time.perf_counter() - t0
    full_work = one_core_step
    pool_step = wall * full_work / (reps * sample_work)
    tokens = S * q_len
    pairs = sorted({synth.codec_map(wl)[li] for li, _, _ in items})
    return {"value": round(tokens / pool_step, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "one_core_value": round(tokens / one_core_step, 4),
            "step_s": round(pool_step, 3), "one_core_step_s": round(one_core_step, 3),
            "sample": (f"{len(items)} sampled (layer, sequence, KV head) units of the {wl} step"
                       f" ({len(pairs)} (K, V) codec pairs), each: encode its {n_new} new row(s) per side, decode "
                       f"{rows} cached rows, fp64 attention of its query heads; 1 core: {reps1} pass(es), "
                       f"{1e3 * sample_work:.0f} ms per pass; {cores} cores: {reps} x {len(items)} units in a "
                       f"process pool, {wall:.2f} s wall; scaled to {units_per_layer} units x {n_layers} layer(s)"
                       + (f" and attention over {L} rows (x{att_scale:.2f})" if att_scale > 1 else "")
                       + " per step")}


def profile_tag(workload, q_len, codecs=None):
    """Name of a workload's bench line and profiles: the workload, its codec
    pair when overridden, and the verify width."""
    tag = workload if not codecs else f"{workload}_{codecs.replace(':', '_')}"
    return tag if q_len == 1 else f"{tag}_verify{q_len}"


def load_traffic(kind, tag, n_splits=None):
    """HBM bytes per launch of the measured kernel from the committed rocprofv3
    counter runs, only if they were taken on its current sources (and, for
    decode, at this split count)."""
    p = os.path.join(ROOT, "profiles", f"{kind}_{tag}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(kind) or t.get("n_splits") != n_splits:
        return None
    return t.get("hbm_bytes_per_launch")


def _read_csv(path):
    import csv

    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _counter_kib(d, counter, name_part):
    """Mean of a rocprofv3 --pmc counter over the dispatches whose kernel name
    contains name_part (one row per dispatch and counter)."""
    rows = [r for r in _read_csv(os.path.join(d, "run_counter_collection.csv"))
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]]
    if not rows:
        raise SystemExit(f"no {counter} rows for '{name_part}' in {d}")
    v = [float(r["Counter_Value"]) for r in rows]
    return sum(v) / len(v), len(v)


SQ_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_LDS",
               "SQ_WAIT_INST_ANY", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def summarize_sq(workload, prof, command, subdir):
    """profiles/decode_<workload>_sq_counters.md: per-dispatch means of the
    issue counters of decode_kernel from one rocprofv3 --pmc run, and the
    counters' ratios to SQ_WAVE_CYCLES (how the waves' time splits)."""
    d = os.path.join(prof, subdir, "sq")
    vals = {c: _counter_kib(d, c, "decode_kernel")[0] for c in SQ_COUNTERS}
    n = _counter_kib(d, "SQ_WAVE_CYCLES", "decode_kernel")[1]
    md = [f"# decode_kernel, workload {workload}: issue counters (rocprofv3 --pmc)", "",
          f"Kernel sources: {kernel_source_hash('decode')} (sha256 prefix over the decode kernel's csrc/ files, "
          "as bench.py computes it).", "", "Command (from the repository root, with TMPDIR=/tmp):", "", "```", command, "```", "",
          f"Means over {n} decode_kernel dispatches (warmup included):", "", "| counter | per dispatch | / SQ_WAVE_CYCLES |",
          "|---|---:|---:|"]
    for c in SQ_COUNTERS:
        ratio = f"{vals[c] / vals['SQ_WAVE_CYCLES']:.3f}" if c.startswith("SQ_") and c != "SQ_WAVE_CYCLES" else ""
        md.append(f"| `{c}` | {vals[c]:.4g} | {ratio} |")
    md += ["", "The ratios compare each counter with the cycles the kernel's waves were resident "
           "(SQ_WAVE_CYCLES); they are read across workloads, not as absolute utilisations.  On this stack "
           "SQ_ACTIVE_INST_VMEM reads 0 and SQ_VALU_MFMA_BUSY_CYCLES reads exact powers of two for every "
           "workload, so neither is used; the MFMA work is 1-3 GFLOP per launch, far below the matrix peak."]
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_sq_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


def summarize_profiles(kind, workload, prof, commands, subdir=None):
    """Turn one workload's rocprofv3 runs into the committed summaries:
    profiles/<kind>_<workload>_kernel_stats.md (kernel-trace statistics beside
    the bench line of the same run) and profiles/<kind>_<workload>_traffic.json
    (HBM bytes per launch of <kind>_kernel from FETCH_SIZE and WRITE_SIZE,
    each scaled by what the counter reads for a plain 1 GiB device copy)."""
    kernel = f"{kind}_kernel"
    subdir = subdir or workload
    stats = _read_csv(os.path.join(prof, subdir, "trace", "run_kernel_stats.csv"))
    def bench_line(name):
        with open(os.path.join(prof, subdir, name)) as f:
            return json.loads([l for l in f.read().splitlines() if l.startswith("{")][-1])

    line = bench_line("bench.json")          # plain run (no profiler attached)
    traced = bench_line("bench_traced.json")  # the run under --kernel-trace
    copy_fetch, _ = _counter_kib(os.path.join(prof, "copy_fetch"), "FETCH_SIZE", "copy")
    copy_write, _ = _counter_kib(os.path.join(prof, "copy_write"), "WRITE_SIZE", "copy")
    f_fetch = (1 << 30) / (copy_fetch * 1024)
    f_write = (1 << 30) / (copy_write * 1024)
    fetch, n_f = _counter_kib(os.path.join(prof, subdir, "fetch"), "FETCH_SIZE", kernel)
    write, n_w = _counter_kib(os.path.join(prof, subdir, "write"), "WRITE_SIZE", kernel)
    hbm = fetch * 1024 * f_fetch + write * 1024 * f_write
    alg = line["roofline"]["algorithmic_bytes_per_launch"]
    dec = [r for r in stats if kernel in r["Name"]]
    calls = sum(int(r["Calls"]) for r in dec)
    avg_us = sum(float(r["TotalDurationNs"]) for r in dec) / calls / 1e3
    traffic = {
        "workload": workload, "kernel": kernel,
        "fetch_kib_per_dispatch": round(fetch, 1), "write_kib_per_dispatch": round(write, 1),
        "dispatches": [n_f, n_w],
        "copy_calibration": {"fetch_kib_per_gib": round(copy_fetch, 1), "write_kib_per_gib": round(copy_write, 1),
                             "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)},
        "hbm_bytes_per_launch": int(round(hbm)),
        "algorithmic_bytes_per_launch": alg,
        "hbm_over_algorithmic": round(hbm / alg, 4),
        "kernel_source_hash": line["kernel_source_hash"],
        "n_splits": line["config"].get("n_splits"),
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{kind}_{workload}_traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    md = [f"# {kernel}, workload {workload}: rocprofv3 kernel statistics", "",
          f"Kernel sources: {line['kernel_source_hash']} (sha256 prefix over the {kind} kernel's csrc/ files, as bench.py computes it).", "",
          "Commands (from the repository root, with TMPDIR=/tmp):", "", "```"] + commands + ["```", "",
          "| kernel | calls | average us | min us | max us | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:8]:
        name = r["Name"] if len(r["Name"]) <= 90 else r["Name"][:87] + "..."
        md.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    rl = line["roofline"]
    trl = traced["roofline"]
    splits = line["config"].get("n_splits")
    md += ["", f"rocprofv3: {kernel} average over all {calls} calls of the traced run (warmup included): "
           f"{avg_us:.2f} us.", "",
           f"bench.py, same command without a profiler attached: mean over its timed {kind} launches "
           f"{1e3 * rl['mean_launch_ms']:.2f} us (min {1e3 * rl['min_launch_ms']:.2f} us), from HIP events recorded "
           f"by the {kind} dispatch itself; value {line['value']} {line['unit']}, {line['ms_per_step']} ms/step, "
           f"roofline achieved {rl['achieved']} GB/s = {rl['frac']} of {rl['peak']} GB/s "
           f"({rl['algorithmic_bytes_per_launch']} algorithmic bytes per launch)"
           + (f", n_splits {splits}." if splits is not None else "."), "",
           f"(Inside the traced run the tracer perturbs those events: bench.py read "
           f"{1e3 * trl['mean_launch_ms']:.2f} us there.)", "",
           f"HBM traffic per {kind} launch (separate --pmc runs, one counter each):", "",
           f"- FETCH_SIZE {fetch:.1f} KiB x {f_fetch:.3f} (1 GiB copy reads {copy_fetch:.0f} KiB) "
           f"+ WRITE_SIZE {write:.1f} KiB x {f_write:.3f} (1 GiB copy writes {copy_write:.0f} KiB)",
           f"- = {hbm / 1e6:.2f} MB per launch vs {alg / 1e6:.2f} MB algorithmic ({hbm / alg:.3f}x)", ""]
    with open(os.path.join(ROOT, "profiles", f"{kind}_{workload}_kernel_stats.md"), "w") as f:
        f.write("\n".join(md))
    print("\n".join(md))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="ladder", choices=WORKLOADS)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed blocks of --steps steps each; ms_per_step is the median block")
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0, help="split count (default: the library heuristic)")
    ap.add_argument("--q-len", type=int, default=1,
                    help="new tokens per sequence verified per step (vit_attn_decode_mq when > 1)")
    ap.add_argument("--codecs", default=None, metavar="K:V",
                    help="override a single-layer workload's codec pair, e.g. rot3:rot3 ("
                    + ", ".join(CODEC_NAMES) + ")")
    ap.add_argument("--transcode", default=None, choices=TRANSCODE_PAIRS,
                    help="time a VBR degrade step (vit_kv_transcode) of one ladder-slot tensor instead")
    ap.add_argument("--side", default="k", choices=("k", "v"), help="plane side for --transcode / --append")
    ap.add_argument("--append", default=None, choices=CODEC_NAMES,
                    help="time one ladder ubatch append (vit_kv_append_quant) of this codec instead")
    ap.add_argument("--probe", action="store_true",
                    help="time an attention-probe scoring event (+ eviction choice) on --workload's K plane instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--append-schedule", default="batched", choices=("batched", "per_layer", "overlapped"),
                    help="ladder: one multi-plane append launch before the decodes (batched), one two-plane "
                    "launch before each layer's decode (per_layer), or per-plane appends on a second stream "
                    "overlapped with the decodes (overlapped)")
    ap.add_argument("--no-merge", action="store_true",
                    help="decode + separate reduce launch even where vit_attn_decode_merged applies")
    ap.add_argument("--graph", action="store_true",
                    help="also time the steps as HIP graph replays (one captured graph per replica)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy", type=int, default=0, help="only run N plain 1 GiB copies")
    ap.add_argument("--summarize-sq", metavar="PROF_DIR", default=None,
                    help="write the decode issue-counter summary for --workload from PROF_DIR/<tag>/sq (no GPU)")
    ap.add_argument("--summarize", metavar="PROF_DIR", default=None,
                    help="write profiles/ summaries for --workload from rocprofv3 output under PROF_DIR (no GPU)")
    args = ap.parse_args()
    if args.summarize_sq:
        w = profile_tag(args.workload, args.q_len, args.codecs)
        b = (f"python3 bench.py --workload {args.workload}" + (f" --q-len {args.q_len}" if args.q_len > 1 else "")
             + (f" --codecs {args.codecs}" if args.codecs else ""))
        summarize_sq(w, args.summarize_sq, f"rocprofv3 --pmc {' '.join(SQ_COUNTERS)} --output-format csv "
                     f"-d PROF/{w}/sq -o run -- {b} --steps 20 --warmup 3 --no-cpu-baseline", w)
        return
    if args.summarize:
        if args.transcode:
            kind = "transcode"
            sc, dc = args.transcode.split(":")
            w = f"{sc}_to_{dc}_{args.side}"
            b = f"python3 bench.py --transcode {args.transcode} --side {args.side}"
        elif args.append:
            kind = "append"
            w = f"{args.append}_{args.side}"
            b = f"python3 bench.py --append {args.append} --side {args.side}"
        elif args.probe:
            kind = "probe_logits"
            w = args.workload
            b = f"python3 bench.py --probe --workload {args.workload}"
        else:
            kind = "decode"
            w = profile_tag(args.workload, args.q_len, args.codecs)
            b = (f"python3 bench.py --workload {args.workload}" + (f" --q-len {args.q_len}" if args.q_len > 1 else "")
                 + (f" --codecs {args.codecs}" if args.codecs else ""))
        d = f"probe_{w}" if args.probe else (f"append_{w}" if args.append else w)  # directory under PROF
        cmds = [f"{b} --no-cpu-baseline > PROF/{d}/bench.json",
                f"rocprofv3 --kernel-trace --stats --output-format csv -d PROF/{d}/trace -o run -- "
                f"{b} --no-cpu-baseline > PROF/{d}/bench_traced.json",
                f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d PROF/{d}/fetch -o run -- "
                f"{b} --steps 20 --warmup 3 --no-cpu-baseline",
                f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d PROF/{d}/write -o run -- "
                f"{b} --steps 20 --warmup 3 --no-cpu-baseline",
                "rocprofv3 --pmc FETCH_SIZE --output-format csv -d PROF/copy_fetch -o run -- python3 bench.py --calib-copy 4",
                "rocprofv3 --pmc WRITE_SIZE --output-format csv -d PROF/copy_write -o run -- python3 bench.py --calib-copy 4",
                f"{b} --summarize PROF"]
        summarize_profiles(kind, w, args.summarize, cmds, subdir=d)
        return
    if args.codecs and any(c not in CODEC_NAMES for c in args.codecs.split(":")) or \
            (args.codecs and len(args.codecs.split(":")) != 2):
        raise SystemExit(f"--codecs takes K:V with codecs from {CODEC_NAMES}")
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path would shard by (sequence, KV head) with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    if args.calib_copy:
        run_copy_calibration(args.calib_copy)
        return
    if args.transcode:
        main_transcode(args)
        return
    if args.probe:
        main_probe(args)
        return
    if args.append:
        main_append(args)
        return
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on the host's cores, before this process touches the GPU
        cpu = cpu_baseline(args.workload, args.q_len, args.cpu_seconds)
        print(f"# cpu baseline: {cpu['value']} tokens/s on {cpu['cores']} cores ({cpu['cpu_model']})",
              file=sys.stderr, flush=True)
    r = run_gpu(args)
    stream_peak = measure_stream_read()
    print(f"# measured stream-read peak: {stream_peak:.1f} GB/s", file=sys.stderr, flush=True)
    cfg = r["cfg"]
    tok_s = r["S"] * r["QL"] / (r["ms_per_step"] * 1e-3)
    traffic = load_traffic("decode", profile_tag(args.workload, r["QL"], args.codecs), r["n_splits"])
    pairs = sorted(set(r["cmap"]))
    codec_txt = (f"K {r['cmap'][0][0]} / V {r['cmap'][0][1]}" if r["n_layers"] == 1 else
                 f"per-layer (K, V) codecs from {{{', '.join(sorted({c for p in pairs for c in p}))}}} "
                 f"({len(pairs)} pairs over {r['n_layers']} layers)")
    line = {
        "metric": "decode-attention tokens/s + effective KV-read GB/s (% of HBM peak), 1 GPU",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "ms_per_step_min": round(min(r["block_ms"]), 5),
        "ms_per_step_max": round(max(r["block_ms"]), 5),
        "repeats": args.repeats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{codec_txt} codes; fp16 MFMA operands (hi+lo split), fp32 accumulate",
        "data": "synthetic (seeded device normals shaped like the workload; no model weights or dataset)",
        "config": {
            "workload": profile_tag(cfg["name"], r["QL"], args.codecs),
            "n_seqs": r["S"], "n_q_heads": r["Hq"], "n_kv_heads": r["H"], "head_dim": D,
            "context": r["L"], "layers": r["n_layers"], "new_tokens_per_seq": r["T"], "query_tokens_per_seq": r["QL"],
            "codecs": ("ladder: " + ", ".join(f"{k}/{v}" for k, v in r["cmap"])) if r["n_layers"] > 1
            else f"K {r['cmap'][0][0]} / V {r['cmap'][0][1]}",
            "n_splits": r["n_splits"], "split_merge": r["merge"], "cold_cache_replicas": r["replicas"],
            "launch": r["mode"],
            **({"ubatch_appends": r["appends"]} if r["appends"] else {}),
        },
        "graph_ms_per_step": None if r["graph_ms_per_step"] is None else round(r["graph_ms_per_step"], 5),
        **({} if r["per_layer_ms_per_step"] is None else {
            "per_layer_appends_ms_per_step": round(r["per_layer_ms_per_step"], 5),
            "per_layer_appends_tokens_per_s": round(r["S"] * r["QL"] / (r["per_layer_ms_per_step"] * 1e-3), 1)}),
        "effective_kv_read_gbs": round(r["kv_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9, 1),
        "effective_kv_read_pct_of_hbm_peak": round(100 * r["kv_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_kernel",
            "achieved": round(r["achieved_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["achieved_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": r["per_launch_bytes"],
            "mean_launch_ms": round(r["dec_mean_ms"], 5),
            "min_launch_ms": round(r["dec_min_ms"], 5),
            "stream_read_peak": round(stream_peak, 1),
            "frac_of_stream_read_peak": round(r["achieved_gbs"] / stream_peak, 4),
        },
        "kernel_source_hash": kernel_source_hash(),
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
