"""Quantized KV-cache append and flash-decode attention for MI355X (gfx950).

The compute lives in libvit.so (hand-written HIP kernels behind the C ABI of
include/vit.h).  This module only marshals torch tensors into those calls:
PyTorch provides device memory and the stream, nothing else.  The Python
names mirror the C entry points:

    vit_kv_plane_sizes, vit_kv_append_quant, vit_kv_append_quant_multi,
    vit_kv_transcode, vit_vbr_classic_next_step, vit_attn_workspace_bytes,
    vit_attn_default_splits, vit_attn_decode, vit_attn_decode_mq,
    vit_attn_decode_merged, vit_attn_decode_noalloc, vit_attn_splitk_reduce,
    vit_attn_probe_workspace_bytes,
    vit_attn_probe_scores, vit_probe_select_evictions,
    vit_arm_kernel_events, vit_stream_read (measurement aids)

``KVPlane`` allocates the three arrays of one (layer, side) cache tensor.
"""

import ctypes

import numpy as np

from . import _lib, layout
from ._lib import CODEC_IDS, SIDE_IDS, VitError, VitKvPlane

__all__ = [
    "KVPlane", "VitError", "layout",
    "vit_kv_plane_sizes", "vit_kv_append_quant", "vit_kv_append_quant_multi", "vit_kv_transcode",
    "vit_vbr_classic_next_step", "vit_attn_workspace_bytes",
    "vit_attn_default_splits", "vit_attn_decode", "vit_attn_decode_mq", "vit_attn_decode_merged",
    "vit_attn_decode_noalloc",
    "vit_attn_splitk_reduce",
    "vit_attn_probe_workspace_bytes", "vit_attn_probe_scores", "vit_probe_select_evictions",
    "vit_probe_select_workspace_bytes",
    "vit_arm_kernel_events", "vit_stream_read",
]

HEAD_DIM = 128
MAX_APPEND_PLANES = _lib.MAX_APPEND_PLANES  # planes per vit_kv_append_quant_multi call


def _stream_handle(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _fptr(t, name, dtype_name="float32"):
    import torch

    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if str(t.dtype) != f"torch.{dtype_name}":
        raise TypeError(f"{name} must be {dtype_name}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def vit_kv_plane_sizes(codec, n_seqs, n_kv_heads, head_dim, capacity):
    """(codes_bytes, scales_bytes, norms_bytes) of one plane."""
    lib = _lib.load()
    c, s, n = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    st = lib.vit_kv_plane_sizes(CODEC_IDS[codec] if isinstance(codec, str) else int(codec),
                                n_seqs, n_kv_heads, head_dim, capacity,
                                ctypes.byref(c), ctypes.byref(s), ctypes.byref(n))
    _lib.check("vit_kv_plane_sizes", st)
    return c.value, s.value, n.value


class KVPlane:
    """One (layer, side) KV cache tensor in device memory (torch-allocated).

    ``side`` is "k" or "v"; ``signs`` (rot4 only) is the 16-byte sign mask,
    kept on the host and passed by value at each call.
    """

    def __init__(self, codec, side, n_seqs, n_kv_heads, capacity, signs=None, device="cuda"):
        import torch

        self.codec, self.side = codec, side
        self.n_seqs, self.n_kv_heads, self.capacity = n_seqs, n_kv_heads, capacity
        cb, sb, nb = vit_kv_plane_sizes(codec, n_seqs, n_kv_heads, HEAD_DIM, capacity)
        self.codes = torch.empty(cb, dtype=torch.uint8, device=device)
        self.scales = torch.empty(sb // 2, dtype=torch.int16, device=device) if sb else None
        self.norms = torch.empty(nb // 2, dtype=torch.int16, device=device) if nb else None
        if codec in ("rot4", "rot3"):
            if signs is None:
                raise ValueError(f"{codec} planes need a 16-byte sign mask")
            self.signs = np.ascontiguousarray(signs, dtype=np.uint8).reshape(16).copy()
        else:
            self.signs = None

    @classmethod
    def like(cls, other, device="cuda"):
        return cls(other.codec, other.side, other.n_seqs, other.n_kv_heads, other.capacity,
                   other.signs, device)

    def struct(self):
        """The C descriptor (built once: the arrays never move)."""
        if getattr(self, "_struct", None) is not None:
            return self._struct
        p = VitKvPlane()
        p.codec = CODEC_IDS[self.codec]
        p.side = SIDE_IDS[self.side]
        p.n_seqs, p.n_kv_heads, p.head_dim, p.reserved = self.n_seqs, self.n_kv_heads, HEAD_DIM, 0
        p.capacity = self.capacity
        p.codes = self.codes.data_ptr()
        p.scales = self.scales.data_ptr() if self.scales is not None else None
        p.norms = self.norms.data_ptr() if self.norms is not None else None
        p.signs = self.signs.ctypes.data if self.signs is not None else None
        self._struct = p
        return p

    def tensors(self):
        return [t for t in (self.codes, self.scales, self.norms) if t is not None]

    def copy_from(self, other):
        for a, b in zip(self.tensors(), other.tensors()):
            a.copy_(b, non_blocking=True)

    def host_view(self):
        """Logical contents on the host: dict(codes, scales, norms) shaped per row."""
        S, H, cap = self.n_seqs, self.n_kv_heads, self.capacity
        out = {"codes": layout.unpack_codes(self.codec, self.side, self.codes.cpu().numpy(), S, H, cap)}
        if self.scales is not None:
            out["scales"] = layout.unpack_scales(self.side, self.scales.cpu().numpy().view(np.uint16), S, H, cap)
        if self.norms is not None:
            out["norms"] = layout.unpack_norms(self.norms.cpu().numpy().view(np.uint16), S, H, cap)
        return out


def vit_kv_append_quant(plane, src, pos0, n_tokens=None, stream=None):
    """Quantize src fp32 [S, T, Hkv, 128] into rows pos0[s] .. pos0[s]+T-1."""
    lib = _lib.load()
    if n_tokens is None:
        n_tokens = src.shape[1]
    p0 = (ctypes.c_int64 * len(pos0))(*[int(x) for x in pos0])
    p = plane.struct()
    st = lib.vit_kv_append_quant(ctypes.byref(p), _fptr(src, "src"), p0, int(n_tokens), _stream_handle(stream))
    return _lib.check("vit_kv_append_quant", st)


def _multi_args(planes, srcs, pos0, n_tokens):
    if len(planes) != len(srcs):
        raise ValueError("one source per plane")
    arr = (_lib.VitKvPlane * len(planes))(*[p.struct() for p in planes])
    ptrs = (ctypes.c_void_p * len(srcs))(*[_fptr(x, "src").value for x in srcs])
    p0 = (ctypes.c_int64 * len(pos0))(*[int(x) for x in pos0])
    n_tokens = srcs[0].shape[1] if n_tokens is None else n_tokens
    return arr, ptrs, p0, int(n_tokens)


def vit_kv_append_quant_multi(planes, srcs, pos0, n_tokens=None, stream=None):
    """vit_kv_append_quant of srcs[i] (fp32 [S, T, Hkv, 128]) into planes[i]
    for every i, in one launch (planes of equal S and Hkv)."""
    lib = _lib.load()
    arr, ptrs, p0, n = _multi_args(planes, srcs, pos0, n_tokens)
    st = lib.vit_kv_append_quant_multi(arr, len(planes), ptrs, p0, n, _stream_handle(stream))
    return _lib.check("vit_kv_append_quant_multi", st)


def vit_kv_transcode(src, dst, n_rows, stream=None):
    """Re-encode rows 0 .. n_rows[s]-1 of every KV head of plane ``src`` into
    plane ``dst`` (a VBR degrade step: f16 -> q8_0 / q4_0 / rot4,
    q8_0 -> q4_0 / rot4)."""
    lib = _lib.load()
    nr = (ctypes.c_int64 * len(n_rows))(*[int(x) for x in n_rows])
    sp, dp = src.struct(), dst.struct()
    st = lib.vit_kv_transcode(ctypes.byref(sp), ctypes.byref(dp), nr, _stream_handle(stream))
    return _lib.check("vit_kv_transcode", st)


def vit_vbr_classic_next_step(codecs, price_order, movable=None, floor_bpv=None):
    """The classic ladder's next degrade step for tensors with these codec
    names, as (tensor index, new codec name), or None when no step is left."""
    lib = _lib.load()
    n = len(codecs)
    ids = {v: k for k, v in _lib.CODEC_IDS.items()}
    c = (ctypes.c_int32 * n)(*[_lib.CODEC_IDS[x] for x in codecs])
    o = (ctypes.c_int32 * n)(*[int(x) for x in price_order])
    m = None if movable is None else (ctypes.c_uint8 * n)(*[1 if x else 0 for x in movable])
    t, nc = ctypes.c_int32(), ctypes.c_int32()
    st = lib.vit_vbr_classic_next_step(n, c, o, m, 0.0 if floor_bpv is None else float(floor_bpv),
                                       ctypes.byref(t), ctypes.byref(nc))
    _lib.check("vit_vbr_classic_next_step", st)
    return None if t.value < 0 else (t.value, ids[nc.value])


def vit_attn_workspace_bytes(n_seqs, n_q_heads, head_dim, n_splits):
    return int(_lib.load().vit_attn_workspace_bytes(n_seqs, n_q_heads, head_dim, n_splits))


def vit_attn_default_splits(n_seqs, n_kv_heads, n_q_heads, max_seq_len):
    return int(_lib.load().vit_attn_default_splits(n_seqs, n_kv_heads, n_q_heads, int(max_seq_len)))


def vit_attn_decode(k, v, q, n_q_heads, seq_len, k_new=None, v_new=None, scale=None, n_splits=1,
                    workspace=None, out=None, stream=None):
    """Decode attention; returns ``out`` (fp32 [S, Hq, 128]), which holds the
    result only when n_splits == 1 (otherwise call vit_attn_splitk_reduce)."""
    import torch

    lib = _lib.load()
    if scale is None:
        scale = 1.0 / np.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((k.n_seqs, n_q_heads, HEAD_DIM), dtype=torch.float32, device=q.device)
    sl = (ctypes.c_int64 * len(seq_len))(*[int(x) for x in seq_len])
    kp, vp = k.struct(), v.struct()
    st = lib.vit_attn_decode(ctypes.byref(kp), ctypes.byref(vp), _fptr(q, "q"), int(n_q_heads), sl,
                             _fptr(k_new, "k_new"), _fptr(v_new, "v_new"), float(scale), int(n_splits),
                             _fptr(workspace, "workspace", "uint8") if workspace is not None else None,
                             _fptr(out, "out"), _stream_handle(stream))
    _lib.check("vit_attn_decode", st)
    return out


def vit_attn_decode_mq(k, v, q, n_q_heads, q_len, seq_len, k_new=None, v_new=None, scale=None, n_splits=1,
                       workspace=None, out=None, stream=None):
    """Decode attention for ``q_len`` new tokens per sequence, causal among
    themselves; q fp32 [S, q_len, Hq, 128]; returns ``out`` (fp32
    [S, q_len, Hq, 128]), which holds the result only when n_splits == 1
    (otherwise vit_attn_splitk_reduce with n_q_heads * q_len rows)."""
    import torch

    lib = _lib.load()
    if scale is None:
        scale = 1.0 / np.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((k.n_seqs, q_len, n_q_heads, HEAD_DIM), dtype=torch.float32, device=q.device)
    sl = (ctypes.c_int64 * len(seq_len))(*[int(x) for x in seq_len])
    kp, vp = k.struct(), v.struct()
    st = lib.vit_attn_decode_mq(ctypes.byref(kp), ctypes.byref(vp), _fptr(q, "q"), int(n_q_heads), int(q_len), sl,
                                _fptr(k_new, "k_new"), _fptr(v_new, "v_new"), float(scale), int(n_splits),
                                _fptr(workspace, "workspace", "uint8") if workspace is not None else None,
                                _fptr(out, "out"), _stream_handle(stream))
    _lib.check("vit_attn_decode_mq", st)
    return out


def merge_fits(n_q_heads, n_kv_heads, q_len, n_splits):
    """Whether vit_attn_decode_merged takes this shape (else decode + reduce)."""
    rows = (n_q_heads // n_kv_heads) * q_len
    return n_splits == 1 or (n_splits <= _lib.MERGE_MAX_SPLITS and rows * n_splits <= _lib.MERGE_MAX_PARTIALS)


def merge_counters(k, device=None):
    """Zeroed arrival counters for vit_attn_decode_merged on ``k``'s shape
    (uint32 [S][Hkv], stored as int32; every call leaves them zero)."""
    import torch

    return torch.zeros((k.n_seqs, k.n_kv_heads), dtype=torch.int32, device=device or "cuda")


def vit_attn_decode_merged(k, v, q, n_q_heads, q_len, seq_len, out, workspace=None, counters=None, k_new=None,
                           v_new=None, scale=None, n_splits=1, stream=None):
    """Decode attention and its split merge in one launch: q, out fp32
    [S, q_len, Hq, 128]; ``counters`` from merge_counters (zero between calls)."""
    lib = _lib.load()
    if scale is None:
        scale = 1.0 / np.sqrt(HEAD_DIM)
    sl = (ctypes.c_int64 * len(seq_len))(*[int(x) for x in seq_len])
    kp, vp = k.struct(), v.struct()
    st = lib.vit_attn_decode_merged(ctypes.byref(kp), ctypes.byref(vp), _fptr(q, "q"), int(n_q_heads), int(q_len),
                                    sl, _fptr(k_new, "k_new"), _fptr(v_new, "v_new"), ctypes.c_float(scale),
                                    int(n_splits),
                                    _fptr(workspace, "workspace", "uint8") if workspace is not None else None,
                                    _fptr(counters, "counters", "int32") if counters is not None else None,
                                    _fptr(out, "out"), _stream_handle(stream))
    _lib.check("vit_attn_decode_merged", st)
    return out


def vit_attn_decode_noalloc(k, v, q, n_q_heads, q_len, seq_len, out, k_new=None, v_new=None, scale=None,
                            n_splits=1, stream=None):
    """Decode attention (+ split-K merge) with the split partials in the
    library's static device scratch: q, out fp32 [S, q_len, Hq, 128] (out is
    caller-allocated; the call allocates nothing)."""
    lib = _lib.load()
    if scale is None:
        scale = 1.0 / np.sqrt(HEAD_DIM)
    sl = (ctypes.c_int64 * len(seq_len))(*[int(x) for x in seq_len])
    kp, vp = k.struct(), v.struct()
    st = lib.vit_attn_decode_noalloc(ctypes.byref(kp), ctypes.byref(vp), _fptr(q, "q"), int(n_q_heads), int(q_len),
                                     sl, _fptr(k_new, "k_new"), _fptr(v_new, "v_new"), ctypes.c_float(scale),
                                     int(n_splits), _fptr(out, "out"), _stream_handle(stream))
    _lib.check("vit_attn_decode_noalloc", st)
    return out


def vit_attn_splitk_reduce(workspace, n_seqs, n_q_heads, head_dim, n_splits, v, out, stream=None):
    lib = _lib.load()
    vp = v.struct()
    st = lib.vit_attn_splitk_reduce(_fptr(workspace, "workspace", "uint8"), int(n_seqs), int(n_q_heads),
                                    int(head_dim), int(n_splits), ctypes.byref(vp), _fptr(out, "out"),
                                    _stream_handle(stream))
    return _lib.check("vit_attn_splitk_reduce", st)


def decode(k, v, q, n_q_heads, seq_len, k_new=None, v_new=None, scale=None, n_splits=None,
           workspace=None, out=None, stream=None, q_len=None):
    """vit_attn_decode (or, with ``q_len``, vit_attn_decode_mq: q
    [S, q_len, Hq, 128]) followed when n_splits > 1 by vit_attn_splitk_reduce."""
    import torch

    rows = n_q_heads * (q_len or 1)
    if n_splits is None:
        n_splits = vit_attn_default_splits(k.n_seqs, k.n_kv_heads, n_q_heads, max(seq_len))
    if n_splits > 1 and workspace is None:
        workspace = torch.empty(vit_attn_workspace_bytes(k.n_seqs, rows, HEAD_DIM, n_splits),
                                dtype=torch.uint8, device=q.device)
    if q_len is None:
        out = vit_attn_decode(k, v, q, n_q_heads, seq_len, k_new, v_new, scale, n_splits, workspace, out, stream)
    else:
        out = vit_attn_decode_mq(k, v, q, n_q_heads, q_len, seq_len, k_new, v_new, scale, n_splits, workspace,
                                 out, stream)
    if n_splits > 1:
        vit_attn_splitk_reduce(workspace, k.n_seqs, rows, HEAD_DIM, n_splits, v, out, stream)
    return out


def vit_attn_probe_workspace_bytes(n_seqs, n_q_heads, capacity):
    return int(_lib.load().vit_attn_probe_workspace_bytes(int(n_seqs), int(n_q_heads), int(capacity)))


def vit_attn_probe_scores(k, q, n_q_heads, seq_len, scores, scale=None, decay=1.0, workspace=None, stream=None):
    """One probe scoring event: scores fp32 [S, capacity] (in/out) <- decay *
    scores + per-cell softmax mass of q fp32 [S, Hq, 128] over K plane ``k``."""
    import torch

    lib = _lib.load()
    scale = 1.0 / np.sqrt(HEAD_DIM) if scale is None else scale
    if workspace is None:
        workspace = torch.empty(vit_attn_probe_workspace_bytes(k.n_seqs, n_q_heads, k.capacity),
                                dtype=torch.uint8, device=q.device)
    sl = (ctypes.c_int64 * len(seq_len))(*[int(x) for x in seq_len])
    kp = k.struct()
    st = lib.vit_attn_probe_scores(ctypes.byref(kp), _fptr(q, "q"), int(n_q_heads), sl, ctypes.c_float(scale),
                                   ctypes.c_float(decay), _fptr(workspace, "workspace", "uint8"),
                                   _fptr(scores, "scores"), _stream_handle(stream))
    _lib.check("vit_attn_probe_scores", st)
    return scores


def vit_probe_select_workspace_bytes(n_seqs):
    return int(_lib.load().vit_probe_select_workspace_bytes(int(n_seqs)))


def vit_probe_select_evictions(scores, seq_len, n_sink, n_recent, n_evict, rows_out=None, n_out=None,
                               workspace=None, stream=None):
    """The cells to evict per sequence: (rows_out int64 [S, n_evict], -1
    padded; n_out int32 [S]) from scores fp32 [S, capacity]."""
    import torch

    lib = _lib.load()
    S, cap = scores.shape
    if rows_out is None:
        rows_out = torch.empty((S, max(1, n_evict)), dtype=torch.int64, device=scores.device)
    if n_out is None:
        n_out = torch.empty((S,), dtype=torch.int32, device=scores.device)
    if workspace is None:
        workspace = torch.empty(vit_probe_select_workspace_bytes(S), dtype=torch.uint8, device=scores.device)
    sl = (ctypes.c_int64 * len(seq_len))(*[int(x) for x in seq_len])
    st = lib.vit_probe_select_evictions(_fptr(scores, "scores"), int(S), int(cap), sl, int(n_sink), int(n_recent),
                                        int(n_evict), _fptr(rows_out, "rows_out", "int64"),
                                        _fptr(n_out, "n_out", "int32"), _fptr(workspace, "workspace", "uint8"),
                                        _stream_handle(stream))
    _lib.check("vit_probe_select_evictions", st)
    return rows_out[:, :n_evict], n_out


def _event_handle(ev):
    if ev is None:
        return None
    h = int(ev.cuda_event)
    if h == 0:
        raise ValueError("event has no HIP handle yet: record it once before arming")
    return ctypes.c_void_p(h)


def vit_arm_kernel_events(start, stop):
    """Make the kernel of the next decode, transcode or probe call record
    torch.cuda.Event ``start``/``stop`` at its own dispatch start and end
    (both None disarms)."""
    st = _lib.load().vit_arm_kernel_events(_event_handle(start), _event_handle(stop))
    return _lib.check("vit_arm_kernel_events", st)


def vit_stream_read(buf, sink, stream=None):
    """Measurement aid: read every byte of the uint8 CUDA tensor ``buf`` once
    (16-byte nontemporal loads over the whole GPU, nothing else)."""
    st = _lib.load().vit_stream_read(_fptr(buf, "buf", "uint8"), ctypes.c_size_t(buf.numel()),
                                     _fptr(sink, "sink", "int32"), _stream_handle(stream))
    return _lib.check("vit_stream_read", st)


class _Prepared:
    """A C-ABI call with every argument already marshalled (for loops that
    issue the same call many times, e.g. a decode step)."""

    def __init__(self, name, fn, args, keep):
        self.name, self.fn, self.args, self._keep = name, fn, args, keep

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            _lib.check(self.name, st)


def prepare_append(plane, src, pos0, n_tokens=None, stream=None):
    lib = _lib.load()
    n_tokens = src.shape[1] if n_tokens is None else n_tokens
    p0 = (ctypes.c_int64 * len(pos0))(*[int(x) for x in pos0])
    p = plane.struct()
    args = (ctypes.byref(p), _fptr(src, "src"), p0, int(n_tokens), _stream_handle(stream))
    return _Prepared("vit_kv_append_quant", lib.vit_kv_append_quant, args, (p, p0, src, plane))


def prepare_append_multi(planes, srcs, pos0, n_tokens=None, stream=None):
    lib = _lib.load()
    arr, ptrs, p0, n = _multi_args(planes, srcs, pos0, n_tokens)
    args = (arr, len(planes), ptrs, p0, n, _stream_handle(stream))
    return _Prepared("vit_kv_append_quant_multi", lib.vit_kv_append_quant_multi, args,
                     (arr, ptrs, p0, tuple(planes), tuple(srcs)))


def prepare_transcode(src, dst, n_rows, stream=None):
    lib = _lib.load()
    nr = (ctypes.c_int64 * len(n_rows))(*[int(x) for x in n_rows])
    sp, dp = src.struct(), dst.struct()
    args = (ctypes.byref(sp), ctypes.byref(dp), nr, _stream_handle(stream))
    return _Prepared("vit_kv_transcode", lib.vit_kv_transcode, args, (sp, dp, nr, src, dst))


def prepare_probe(k, q, n_q_heads, seq_len, scores, workspace, scale=None, decay=1.0, stream=None):
    lib = _lib.load()
    scale = 1.0 / np.sqrt(HEAD_DIM) if scale is None else scale
    sl = (ctypes.c_int64 * len(seq_len))(*[int(x) for x in seq_len])
    kp = k.struct()
    args = (ctypes.byref(kp), _fptr(q, "q"), int(n_q_heads), sl, ctypes.c_float(scale), ctypes.c_float(decay),
            _fptr(workspace, "workspace", "uint8"), _fptr(scores, "scores"), _stream_handle(stream))
    return _Prepared("vit_attn_probe_scores", lib.vit_attn_probe_scores, args, (kp, sl, q, workspace, scores, k))


def prepare_select(scores, seq_len, n_sink, n_recent, n_evict, rows_out, n_out, workspace, stream=None):
    lib = _lib.load()
    S, cap = scores.shape
    sl = (ctypes.c_int64 * len(seq_len))(*[int(x) for x in seq_len])
    args = (_fptr(scores, "scores"), int(S), int(cap), sl, int(n_sink), int(n_recent), int(n_evict),
            _fptr(rows_out, "rows_out", "int64"), _fptr(n_out, "n_out", "int32"),
            _fptr(workspace, "workspace", "uint8"), _stream_handle(stream))
    return _Prepared("vit_probe_select_evictions", lib.vit_probe_select_evictions, args,
                     (sl, scores, rows_out, n_out, workspace))


def prepare_decode(k, v, q, n_q_heads, seq_len, out, k_new=None, v_new=None, scale=None, n_splits=1,
                   workspace=None, stream=None, q_len=None):
    lib = _lib.load()
    scale = 1.0 / np.sqrt(HEAD_DIM) if scale is None else scale
    sl = (ctypes.c_int64 * len(seq_len))(*[int(x) for x in seq_len])
    kp, vp = k.struct(), v.struct()
    tail = (_fptr(k_new, "k_new"), _fptr(v_new, "v_new"), ctypes.c_float(scale), int(n_splits),
            _fptr(workspace, "workspace", "uint8") if workspace is not None else None,
            _fptr(out, "out"), _stream_handle(stream))
    keep = (kp, vp, sl, q, k_new, v_new, workspace, out, k, v)
    if q_len is None:
        args = (ctypes.byref(kp), ctypes.byref(vp), _fptr(q, "q"), int(n_q_heads), sl) + tail
        return _Prepared("vit_attn_decode", lib.vit_attn_decode, args, keep)
    args = (ctypes.byref(kp), ctypes.byref(vp), _fptr(q, "q"), int(n_q_heads), int(q_len), sl) + tail
    return _Prepared("vit_attn_decode_mq", lib.vit_attn_decode_mq, args, keep)


def prepare_merged(k, v, q, n_q_heads, q_len, seq_len, out, workspace, counters, k_new=None, v_new=None,
                   scale=None, n_splits=1, stream=None):
    lib = _lib.load()
    scale = 1.0 / np.sqrt(HEAD_DIM) if scale is None else scale
    sl = (ctypes.c_int64 * len(seq_len))(*[int(x) for x in seq_len])
    kp, vp = k.struct(), v.struct()
    args = (ctypes.byref(kp), ctypes.byref(vp), _fptr(q, "q"), int(n_q_heads), int(q_len), sl,
            _fptr(k_new, "k_new"), _fptr(v_new, "v_new"), ctypes.c_float(scale), int(n_splits),
            _fptr(workspace, "workspace", "uint8") if workspace is not None else None,
            _fptr(counters, "counters", "int32") if counters is not None else None, _fptr(out, "out"),
            _stream_handle(stream))
    keep = (kp, vp, sl, q, k_new, v_new, workspace, counters, out, k, v)
    return _Prepared("vit_attn_decode_merged", lib.vit_attn_decode_merged, args, keep)


def prepare_reduce(workspace, n_seqs, n_q_heads, n_splits, v, out, stream=None):
    lib = _lib.load()
    vp = v.struct()
    args = (_fptr(workspace, "workspace", "uint8"), int(n_seqs), int(n_q_heads), HEAD_DIM, int(n_splits),
            ctypes.byref(vp), _fptr(out, "out"), _stream_handle(stream))
    return _Prepared("vit_attn_splitk_reduce", lib.vit_attn_splitk_reduce, args, (vp, workspace, out, v))
