"""ctypes declarations of the C ABI in include/vit.h (argument marshalling only).

Loading fails loudly when libvit.so has not been built: there is no fallback
path of any kind.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvit.so")

VIT_OK = 0
VIT_E_ARG = -1
VIT_E_UNSUPPORTED = -2
VIT_E_CAPACITY = -3
VIT_E_ALIGN = -4
VIT_E_HIP = -5
VIT_E_SCRATCH = -6
NOALLOC_SCRATCH_BYTES = 4 << 20  # VIT_NOALLOC_SCRATCH_BYTES
MERGE_MAX_SPLITS = 64  # VIT_MERGE_MAX_SPLITS
MERGE_MAX_PARTIALS = 128  # VIT_MERGE_MAX_PARTIALS
MAX_APPEND_PLANES = 32  # VIT_MAX_APPEND_PLANES

CODEC_IDS = {"f16": 0, "q8_0": 1, "q4_0": 2, "rot4": 3, "rot3": 4}
SIDE_IDS = {"k": 0, "v": 1}

# every symbol include/vit.h declares
EXPORTS = (
    "vit_kv_plane_sizes",
    "vit_kv_append_quant",
    "vit_kv_append_quant_multi",
    "vit_kv_transcode",
    "vit_vbr_classic_next_step",
    "vit_attn_workspace_bytes",
    "vit_attn_default_splits",
    "vit_attn_decode",
    "vit_attn_decode_mq",
    "vit_attn_decode_merged",
    "vit_attn_decode_noalloc",
    "vit_attn_splitk_reduce",
    "vit_attn_probe_workspace_bytes",
    "vit_attn_probe_scores",
    "vit_probe_select_evictions",
    "vit_probe_select_workspace_bytes",
    "vit_arm_kernel_events",
    "vit_stream_read",
    "vit_status_string",
)


class VitKvPlane(ctypes.Structure):
    _fields_ = [
        ("codec", ctypes.c_int32),
        ("side", ctypes.c_int32),
        ("n_seqs", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("norms", ctypes.c_void_p),
        ("signs", ctypes.c_void_p),
    ]


class VitError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def load():
    """Load libvit.so once; raise ImportError if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m quantized_kv_cache_append_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    i32, i64, sz, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    plane_p = P(VitKvPlane)
    lib.vit_kv_plane_sizes.argtypes = [i32, i32, i32, i32, i64, P(sz), P(sz), P(sz)]
    lib.vit_kv_plane_sizes.restype = ctypes.c_int
    lib.vit_kv_append_quant.argtypes = [plane_p, vp, P(i64), i32, vp]
    lib.vit_kv_append_quant.restype = ctypes.c_int
    lib.vit_kv_append_quant_multi.argtypes = [plane_p, i32, P(vp), P(i64), i32, vp]
    lib.vit_kv_append_quant_multi.restype = ctypes.c_int
    lib.vit_kv_transcode.argtypes = [plane_p, plane_p, P(i64), vp]
    lib.vit_kv_transcode.restype = ctypes.c_int
    lib.vit_vbr_classic_next_step.argtypes = [i32, P(i32), P(i32), P(ctypes.c_uint8), ctypes.c_double,
                                              P(i32), P(i32)]
    lib.vit_vbr_classic_next_step.restype = ctypes.c_int
    lib.vit_attn_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.vit_attn_workspace_bytes.restype = sz
    lib.vit_attn_default_splits.argtypes = [i32, i32, i32, i64]
    lib.vit_attn_default_splits.restype = i32
    lib.vit_arm_kernel_events.argtypes = [vp, vp]
    lib.vit_arm_kernel_events.restype = ctypes.c_int
    lib.vit_attn_decode.argtypes = [plane_p, plane_p, vp, i32, P(i64), vp, vp, f32, i32, vp, vp, vp]
    lib.vit_attn_decode.restype = ctypes.c_int
    lib.vit_attn_decode_mq.argtypes = [plane_p, plane_p, vp, i32, i32, P(i64), vp, vp, f32, i32, vp, vp, vp]
    lib.vit_attn_decode_mq.restype = ctypes.c_int
    lib.vit_attn_decode_merged.argtypes = [plane_p, plane_p, vp, i32, i32, P(i64), vp, vp, f32, i32, vp, vp, vp, vp]
    lib.vit_attn_decode_merged.restype = ctypes.c_int
    lib.vit_attn_decode_noalloc.argtypes = [plane_p, plane_p, vp, i32, i32, P(i64), vp, vp, f32, i32, vp, vp]
    lib.vit_attn_decode_noalloc.restype = ctypes.c_int
    lib.vit_attn_splitk_reduce.argtypes = [vp, i32, i32, i32, i32, plane_p, vp, vp]
    lib.vit_attn_splitk_reduce.restype = ctypes.c_int
    lib.vit_attn_probe_workspace_bytes.argtypes = [i32, i32, i64]
    lib.vit_attn_probe_workspace_bytes.restype = sz
    lib.vit_attn_probe_scores.argtypes = [plane_p, vp, i32, P(i64), f32, f32, vp, vp, vp]
    lib.vit_attn_probe_scores.restype = ctypes.c_int
    lib.vit_probe_select_evictions.argtypes = [vp, i32, i64, P(i64), i64, i64, i32, vp, vp, vp, vp]
    lib.vit_probe_select_evictions.restype = ctypes.c_int
    lib.vit_probe_select_workspace_bytes.argtypes = [i32]
    lib.vit_probe_select_workspace_bytes.restype = sz
    lib.vit_stream_read.argtypes = [vp, sz, vp, vp]
    lib.vit_stream_read.restype = ctypes.c_int
    lib.vit_status_string.argtypes = [ctypes.c_int]
    lib.vit_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status):
    return load().vit_status_string(int(status)).decode()


def check(fn, status):
    if status != VIT_OK:
        raise VitError(fn, status, status_string(status))
    return status
