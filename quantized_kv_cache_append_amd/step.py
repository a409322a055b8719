"""The multi-layer decode step: append a ubatch of new K/V rows to every
layer's planes, then decode and merge through every layer.

This is the step of the per-(layer, side) codec ladder: every layer's K and
V tensors have their own codec (buun-llama-cpp page, "VBR -- Variable
Bit-Rate KV Cache"), each step appends a ubatch of new rows to every
(layer, side) plane -- 2048 rows in the serverAppConfigs commit log's
"BATCH_SIZE 2048 -> 4096, UBATCH_SIZE 1024 -> 2048" commit, at rows of its
256-aligned 200,704-row slots ("CTX_SIZE 540672 -> 401408" commit) -- and
then decodes one token per sequence through every layer.

Schedules.  "batched" (the default): one vit_kv_append_quant_multi launch
per 32 planes (16 layers' K and V) stores the ubatch in all 2 x layers
planes, then the decodes run back to back on the same stream.  "per_layer":
layer l's K and V rows go in with one two-plane call just before layer l's
decode, on the same stream (the order a model's forward pass allows).  "overlapped": the per-plane appends go to a second
stream and decode l waits on an event recorded after layer l's two appends,
so the later layers' appends run while the first layers decode; each step's
appends wait on an event recorded on the decode stream when the step
starts, because they rewrite rows that the previous step's decodes read.
The batched and overlapped schedules need every layer's new rows when the
step starts, which is how this workload is defined (all appends, then all
decodes); in a model's forward pass layer l + 1's rows depend on layer l,
which leaves the per-layer schedule.  A decode fills every compute unit's
registers, so the overlapped appends run only in the decodes' tails, and
decodes then wait for them; the batched launch is faster.

Everything here is argument marshalling and stream ordering: every
operation of the step is a call into libvit.so.
"""

from . import (MAX_APPEND_PLANES, merge_fits, prepare_append, prepare_append_multi, prepare_decode, prepare_merged,
               prepare_reduce, vit_arm_kernel_events)

HEAD_DIM = 128


class DecodeStep:
    """One step over ``layers`` = [(K plane, V plane)] with the per-layer
    inputs prepared once.

    q[l]        fp32 [S, Hq, 128] query rows of layer l
    new_rows[l] (k, v) fp32 [S, T, Hkv, 128]: the ubatch stored at rows
                p_new .. p_new + T - 1 of every sequence before layer l decodes
    out[l]      fp32 [S, Hq, 128] outputs
    lens        rows attended per sequence (they count the ubatch rows)
    workspace   split partials (shared by the layers: the decodes are
                ordered on one stream), n_splits > 1
    counters    zeroed arrival counters (merge_counters): each layer's decode
                and split merge then run as one vit_attn_decode_merged launch
                when the shape allows; otherwise (or None) decode + reduce
    stream, append_stream   torch streams (default priority); append_stream
                is used by the "overlapped" schedule only
    append_mode "batched", "per_layer" or "overlapped" (see the module
                docstring)
    """

    def __init__(self, layers, q, new_rows, out, lens, p_new, n_q_heads, n_splits, workspace, stream,
                 append_stream, counters=None, append_mode="batched"):
        import torch

        if append_mode not in ("batched", "per_layer", "overlapped"):
            raise ValueError(f"append_mode {append_mode!r}")
        self.append_mode = append_mode
        self.stream, self.append_stream = stream, append_stream
        S = layers[0][0].n_seqs
        self.n_layers = len(layers)
        planes = [P for kv in layers for P in kv]
        srcs = [x for kv in new_rows for x in kv]
        # one multi-plane call per MAX_APPEND_PLANES planes (16 layers' K and V)
        self.append_all = ([prepare_append_multi(planes[i:i + MAX_APPEND_PLANES], srcs[i:i + MAX_APPEND_PLANES],
                                                 [p_new] * S, stream=stream)
                            for i in range(0, len(planes), MAX_APPEND_PLANES)]
                           if append_mode == "batched" else [])
        self.layer_appends = ([prepare_append_multi([K, V], [kn, vn], [p_new] * S, stream=stream)
                               for (K, V), (kn, vn) in zip(layers, new_rows)]
                              if append_mode == "per_layer" else [])
        self.merged = (counters is not None and n_splits > 1
                       and merge_fits(n_q_heads, layers[0][0].n_kv_heads, 1, n_splits))
        self.appends, self.decodes = [], []
        for (K, V), ql, (kn, vn), o in zip(layers, q, new_rows, out):
            self.appends.append((prepare_append(K, kn, [p_new] * S, stream=append_stream),
                                 prepare_append(V, vn, [p_new] * S, stream=append_stream)))
            if self.merged:
                d = prepare_merged(K, V, ql.reshape(S, 1, n_q_heads, -1), n_q_heads, 1, lens,
                                   o.reshape(S, 1, n_q_heads, -1), workspace, counters, n_splits=n_splits,
                                   stream=stream)
                self.decodes.append((d, None))
                continue
            d = prepare_decode(K, V, ql, n_q_heads, lens, o, n_splits=n_splits,
                               workspace=workspace if n_splits > 1 else None, stream=stream)
            r = prepare_reduce(workspace, S, n_q_heads, n_splits, V, o, stream=stream) if n_splits > 1 else None
            self.decodes.append((d, r))
        self.fork = torch.cuda.Event()
        self.app_done = [torch.cuda.Event() for _ in range(self.n_layers)]

    def __call__(self, kernel_events=None):
        """Issue one step.  ``kernel_events`` = (starts, stops), one pair per
        layer, armed so that each decode dispatch records its own pair."""
        if self.append_mode in ("batched", "per_layer"):
            for c in self.append_all:
                c()
            for li, (d, r) in enumerate(self.decodes):
                if self.layer_appends:
                    self.layer_appends[li]()
                if kernel_events is not None:
                    vit_arm_kernel_events(kernel_events[0][li], kernel_events[1][li])
                d()
                if r is not None:
                    r()
            return
        self.fork.record(self.stream)  # everything issued on the decode stream before this step
        self.append_stream.wait_event(self.fork)
        for li, (ck, cv) in enumerate(self.appends):
            ck()
            cv()
            self.app_done[li].record(self.append_stream)
        for li, (d, r) in enumerate(self.decodes):
            self.stream.wait_event(self.app_done[li])
            if kernel_events is not None:
                vit_arm_kernel_events(kernel_events[0][li], kernel_events[1][li])
            d()
            if r is not None:
                r()

    def run_serial(self):
        """The same work as one call at a time: every per-plane append, then
        every decode (the reference each schedule must agree with, bit for
        bit)."""
        import torch

        torch.cuda.synchronize()
        for ck, cv in self.appends:  # the per-plane appends, one after another
            ck()
            cv()
        torch.cuda.synchronize()
        for d, r in self.decodes:
            d()
            if r is not None:
                r()
        torch.cuda.synchronize()
