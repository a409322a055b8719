"""C ABI checks that need no GPU: exports, sizes, and every validation path.

Validation runs on the host before anything is enqueued, so these calls use
fake (never dereferenced) device addresses and must return an error status.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from quantized_kv_cache_append_amd import _lib, layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vit.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(vit_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declarations_are_all_exported(lib):
    names = _declared_functions()
    assert len(names) >= 7, names
    assert sorted(_lib.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert _lib.status_string(s) != "unknown status"
    assert _lib.status_string(7) == "unknown status"


@pytest.mark.parametrize("codec,rb,sb,nb", [(0, 256, 0, 0), (1, 128, 8, 0), (2, 64, 8, 0), (3, 64, 8, 2), (4, 48, 8, 0)])
def test_plane_sizes(lib, codec, rb, sb, nb):
    c, s, n = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.vit_kv_plane_sizes(codec, 2, 8, 128, 200704, ctypes.byref(c), ctypes.byref(s), ctypes.byref(n)) == 0
    rows = 2 * 8 * 200704
    assert (c.value, s.value, n.value) == (rows * rb, rows * sb, rows * nb)
    # bits per value of the plane = the codec's bits per value
    assert 8 * (c.value + s.value + n.value) / (rows * 128) == {0: 16, 1: 8.5, 2: 4.5, 3: 4.625, 4: 3.5}[codec]


def test_plane_size_errors(lib):
    z = ctypes.c_size_t()
    r = ctypes.byref(z)
    assert lib.vit_kv_plane_sizes(5, 1, 1, 128, 256, r, r, r) == _lib.VIT_E_UNSUPPORTED
    assert lib.vit_kv_plane_sizes(0, 1, 1, 64, 256, r, r, r) == _lib.VIT_E_UNSUPPORTED
    assert lib.vit_kv_plane_sizes(0, 1, 1, 128, 300, r, r, r) == _lib.VIT_E_CAPACITY
    assert lib.vit_kv_plane_sizes(0, 0, 1, 128, 256, r, r, r) == _lib.VIT_E_ARG
    assert lib.vit_kv_plane_sizes(0, 65, 1, 128, 256, r, r, r) == _lib.VIT_E_UNSUPPORTED
    assert lib.vit_kv_plane_sizes(0, 1, 1, 128, 1 << 30, r, r, r) == _lib.VIT_OK
    assert lib.vit_kv_plane_sizes(0, 1, 1, 128, (1 << 30) + 256, r, r, r) == _lib.VIT_E_UNSUPPORTED


def test_workspace_and_splits(lib):
    assert lib.vit_attn_workspace_bytes(8, 32, 128, 16) == 8 * 32 * 16 * 130 * 4
    assert lib.vit_attn_workspace_bytes(8, 32, 64, 16) == 0
    assert lib.vit_attn_workspace_bytes(8, 32, 128, 0) == 0
    s = lib.vit_attn_default_splits(8, 8, 32, 8192)
    assert 1 <= s <= 8192 // 32 // 4
    assert lib.vit_attn_default_splits(1, 1, 4, 512) >= 1


FAKE = 0x100000  # 256-aligned fake device address; never dereferenced


def _plane(codec=1, side=0, S=2, H=2, cap=512, codes=FAKE, scales=FAKE, norms=FAKE, signs=None):
    p = _lib.VitKvPlane()
    p.codec, p.side, p.n_seqs, p.n_kv_heads, p.head_dim, p.reserved, p.capacity = codec, side, S, H, 128, 0, cap
    p.codes, p.scales, p.norms = codes, scales, norms
    p.signs = signs
    return p


_SIGNS = (ctypes.c_uint8 * 16)()


def _append(lib, p, src=FAKE, pos0=(0, 0), n=1):
    arr = (ctypes.c_int64 * len(pos0))(*pos0)
    return lib.vit_kv_append_quant(ctypes.byref(p), src, arr, n, None)


def test_append_validation(lib):
    assert _append(lib, _plane(), pos0=(500, 0), n=13) == _lib.VIT_E_CAPACITY
    assert _append(lib, _plane(), pos0=(-1, 0)) == _lib.VIT_E_CAPACITY
    assert _append(lib, _plane(cap=300)) == _lib.VIT_E_CAPACITY
    assert _append(lib, _plane(codec=9)) == _lib.VIT_E_UNSUPPORTED
    assert _append(lib, _plane(side=2)) == _lib.VIT_E_ARG
    assert _append(lib, _plane(codes=FAKE + 16)) == _lib.VIT_E_ALIGN
    assert _append(lib, _plane(scales=None)) == _lib.VIT_E_ARG
    assert _append(lib, _plane(codec=3, signs=None)) == _lib.VIT_E_ARG
    assert _append(lib, _plane(codec=3, norms=None, signs=ctypes.addressof(_SIGNS))) == _lib.VIT_E_ARG
    assert _append(lib, _plane(), src=FAKE + 4) == _lib.VIT_E_ALIGN
    assert _append(lib, _plane(), src=None) == _lib.VIT_E_ARG
    assert _append(lib, _plane(), n=-1) == _lib.VIT_E_ARG
    assert _append(lib, _plane(), n=0) == _lib.VIT_OK  # no-op, nothing enqueued
    p = _plane()
    p.head_dim = 64
    assert _append(lib, p) == _lib.VIT_E_UNSUPPORTED
    p = _plane()
    p.reserved = 1
    assert _append(lib, p) == _lib.VIT_E_ARG
    assert _append(lib, _plane(cap=(1 << 30) + 256)) == _lib.VIT_E_UNSUPPORTED


def _append_multi(lib, planes, srcs=None, pos0=(0, 0), n=1, n_planes=None):
    arr = (_lib.VitKvPlane * len(planes))(*planes)
    srcs = [FAKE] * len(planes) if srcs is None else srcs
    ptrs = (ctypes.c_void_p * len(srcs))(*srcs)
    p0 = (ctypes.c_int64 * len(pos0))(*pos0)
    return lib.vit_kv_append_quant_multi(arr, len(planes) if n_planes is None else n_planes, ptrs, p0, n, None)


def test_append_multi_validation(lib):
    """Every plane is checked as vit_kv_append_quant checks it, then the
    batch: equal geometry, pairwise disjoint arrays, 1..32 planes (no compute:
    every case fails or has no rows)."""
    MB = 0x100000

    def pl(i, **kw):  # plane i: q8_0 K, arrays in their own 1 MiB windows
        return _plane(codes=(2 * i + 16) * MB, scales=(2 * i + 17) * MB, norms=None, **kw)

    two = [pl(0), pl(1, side=1)]
    assert _append_multi(lib, two, n=0) == _lib.VIT_OK  # no-op, nothing enqueued
    assert _append_multi(lib, two, n=-1) == _lib.VIT_E_ARG
    assert _append_multi(lib, two, pos0=(500, 0), n=13) == _lib.VIT_E_CAPACITY
    assert _append_multi(lib, two, pos0=(-1, 0)) == _lib.VIT_E_CAPACITY
    assert _append_multi(lib, two, n_planes=0) == _lib.VIT_E_UNSUPPORTED
    assert _lib.MAX_APPEND_PLANES == 32
    many = [pl(i) for i in range(33)]
    assert _append_multi(lib, many, n=0, n_planes=33) == _lib.VIT_E_UNSUPPORTED
    assert _append_multi(lib, many[:32], n=0) == _lib.VIT_OK
    assert _append_multi(lib, [pl(0), pl(1, H=4)]) == _lib.VIT_E_ARG                   # geometry
    assert _append_multi(lib, [pl(0), pl(1, S=3)], pos0=(0, 0, 0)) == _lib.VIT_E_ARG   # geometry
    assert _append_multi(lib, [pl(0), pl(1, codec=9)]) == _lib.VIT_E_UNSUPPORTED        # a bad plane
    assert _append_multi(lib, [pl(0), pl(1, codec=3)]) == _lib.VIT_E_ARG               # rotated, no signs
    assert _append_multi(lib, two, srcs=[FAKE, None]) == _lib.VIT_E_ARG
    assert _append_multi(lib, two, srcs=[FAKE, FAKE + 4]) == _lib.VIT_E_ALIGN
    assert _append_multi(lib, two, srcs=[FAKE, None], n=0) == _lib.VIT_OK             # no rows, no sources
    # arrays of two planes that overlap: the same codes, codes inside another
    # plane's scales, scales inside another plane's codes
    assert _append_multi(lib, [pl(0), pl(0, side=1)]) == _lib.VIT_E_ARG
    assert _append_multi(lib, [pl(0), _plane(codes=17 * MB + 0x100, scales=40 * MB, norms=None)]) == _lib.VIT_E_ARG
    assert _append_multi(lib, [pl(0), _plane(codes=40 * MB, scales=16 * MB + 0x1000, norms=None)]) == _lib.VIT_E_ARG
    # adjacent arrays do not overlap (q8_0 codes of 2 x 2 x 512 rows: 256 KiB)
    assert _append_multi(lib, [pl(0), _plane(codes=16 * MB + 0x40000, scales=40 * MB, norms=None)], n=0) == _lib.VIT_OK


def _decode(lib, k, v, hq=4, seq_len=(10, 10), k_new=None, v_new=None, scale=0.088, ns=1, ws=None, q=FAKE, out=FAKE):
    arr = (ctypes.c_int64 * len(seq_len))(*seq_len)
    return lib.vit_attn_decode(ctypes.byref(k), ctypes.byref(v), q, hq, arr, k_new, v_new, scale, ns, ws, out, None)


def test_decode_validation(lib):
    K, V = _plane(side=0), _plane(side=1)
    assert _decode(lib, K, V, seq_len=(513, 1)) == _lib.VIT_E_CAPACITY
    assert _decode(lib, K, V, seq_len=(0, 1)) == _lib.VIT_E_ARG
    assert _decode(lib, K, V, hq=3) == _lib.VIT_E_ARG            # Hq % Hkv != 0
    assert _decode(lib, K, V, hq=34) == _lib.VIT_E_UNSUPPORTED   # G = 17
    assert _decode(lib, K, V, k_new=FAKE) == _lib.VIT_E_ARG       # k_new xor v_new
    assert _decode(lib, K, V, ns=0) == _lib.VIT_E_ARG
    assert _decode(lib, K, V, ns=5000) == _lib.VIT_E_ARG
    assert _decode(lib, K, V, ns=4, ws=None) == _lib.VIT_E_ARG
    assert _decode(lib, K, V, q=None) == _lib.VIT_E_ARG
    assert _decode(lib, K, V, out=FAKE + 8) == _lib.VIT_E_ALIGN
    assert _decode(lib, K, V, scale=float("nan")) == _lib.VIT_E_ARG
    assert _decode(lib, V, K) == _lib.VIT_E_ARG                  # sides swapped
    assert _decode(lib, K, _plane(side=1, H=4)) == _lib.VIT_E_ARG
    assert _decode(lib, K, _plane(side=1, cap=1024)) == _lib.VIT_E_ARG


def _decode_mq(lib, k, v, hq=4, q_len=2, seq_len=(10, 10), ns=1, ws=None):
    arr = (ctypes.c_int64 * len(seq_len))(*seq_len)
    return lib.vit_attn_decode_mq(ctypes.byref(k), ctypes.byref(v), FAKE, hq, q_len, arr, None, None, 0.088, ns, ws,
                                  FAKE, None)


def test_decode_mq_validation(lib):
    """Several new tokens per call: q_len 1..4, G * q_len <= 16 and every
    sequence at least q_len rows long (no compute: every case fails)."""
    K, V = _plane(side=0), _plane(side=1)
    assert _decode_mq(lib, K, V, q_len=0) == _lib.VIT_E_ARG
    assert _decode_mq(lib, K, V, q_len=5) == _lib.VIT_E_UNSUPPORTED
    assert _decode_mq(lib, K, V, hq=18, q_len=2) == _lib.VIT_E_UNSUPPORTED   # G 9 x 2 rows
    assert _decode_mq(lib, K, V, q_len=3, seq_len=(10, 2)) == _lib.VIT_E_ARG  # shorter than q_len
    assert _decode_mq(lib, K, V, q_len=2, seq_len=(513, 10)) == _lib.VIT_E_CAPACITY
    assert _decode_mq(lib, K, V, q_len=2, ns=3, ws=None) == _lib.VIT_E_ARG


def _decode_noalloc(lib, k, v, hq=4, q_len=1, seq_len=(10, 10), ns=1, k_new=None, v_new=None, out=FAKE):
    arr = (ctypes.c_int64 * len(seq_len))(*seq_len)
    return lib.vit_attn_decode_noalloc(ctypes.byref(k), ctypes.byref(v), FAKE, hq, q_len, arr, k_new, v_new, 0.088,
                                       ns, out, None)


def test_decode_noalloc_validation(lib):
    """The no-allocation decode checks its arguments like vit_attn_decode_mq
    and rejects split partials larger than its static scratch, on the host,
    before it looks up the scratch or enqueues anything (no GPU here)."""
    K, V = _plane(side=0, cap=1 << 20), _plane(side=1, cap=1 << 20)
    assert _decode_noalloc(lib, K, V, seq_len=(0, 1)) == _lib.VIT_E_ARG
    assert _decode_noalloc(lib, K, V, hq=3) == _lib.VIT_E_ARG
    assert _decode_noalloc(lib, K, V, q_len=5) == _lib.VIT_E_UNSUPPORTED
    assert _decode_noalloc(lib, K, V, k_new=FAKE) == _lib.VIT_E_ARG
    assert _decode_noalloc(lib, K, V, ns=0) == _lib.VIT_E_ARG
    assert _decode_noalloc(lib, K, V, out=FAKE + 4) == _lib.VIT_E_ALIGN
    assert _decode_noalloc(lib, V, K) == _lib.VIT_E_ARG
    # partials of 2 x 32 rows x n_splits x 520 B against the 4 MiB array
    limit = _lib.NOALLOC_SCRATCH_BYTES
    need = lambda ns: lib.vit_attn_workspace_bytes(2, 32, 128, ns)
    ns_max = max(n for n in range(2, 4097) if need(n) <= limit)
    assert need(ns_max) <= limit < need(ns_max + 1)
    assert _decode_noalloc(lib, K, V, hq=32, ns=ns_max + 1) == _lib.VIT_E_SCRATCH
    assert _decode_noalloc(lib, K, V, hq=32, ns=4096) == _lib.VIT_E_SCRATCH
    assert _decode_noalloc(lib, K, V, hq=16, q_len=2, ns=ns_max + 1) == _lib.VIT_E_SCRATCH  # 16 x 2 rows
    assert _lib.status_string(_lib.VIT_E_SCRATCH).startswith("split partials larger than the static scratch")


def _decode_merged(lib, k, v, hq=4, q_len=1, seq_len=(10, 10), ns=2, ws=FAKE, counters=FAKE, out=FAKE):
    arr = (ctypes.c_int64 * len(seq_len))(*seq_len)
    return lib.vit_attn_decode_merged(ctypes.byref(k), ctypes.byref(v), FAKE, hq, q_len, arr, None, None, 0.088, ns,
                                      ws, counters, out, None)


def test_decode_merged_validation(lib):
    """The one-launch decode + merge checks its arguments like
    vit_attn_decode_mq, then its own: arrival counters present and 8-B
    aligned, at most 64 splits and 128 partial rows per KV head (query rows
    per KV head x splits), all on the host (no compute: every case fails)."""
    K, V = _plane(side=0), _plane(side=1)  # 2 KV heads
    assert _decode_merged(lib, K, V, seq_len=(0, 1)) == _lib.VIT_E_ARG
    assert _decode_merged(lib, K, V, q_len=5) == _lib.VIT_E_UNSUPPORTED
    assert _decode_merged(lib, K, V, ws=None) == _lib.VIT_E_ARG
    assert _decode_merged(lib, K, V, out=FAKE + 8) == _lib.VIT_E_ALIGN
    assert _decode_merged(lib, V, K) == _lib.VIT_E_ARG
    assert _decode_merged(lib, K, V, counters=None) == _lib.VIT_E_ARG
    assert _decode_merged(lib, K, V, counters=FAKE + 4) == _lib.VIT_E_ALIGN
    assert _lib.MERGE_MAX_SPLITS == 64 and _lib.MERGE_MAX_PARTIALS == 128
    assert _decode_merged(lib, K, V, ns=65) == _lib.VIT_E_UNSUPPORTED            # 2 rows x 65 splits
    assert _decode_merged(lib, K, V, hq=16, ns=17) == _lib.VIT_E_UNSUPPORTED     # 8 rows x 17 splits
    assert _decode_merged(lib, K, V, hq=8, q_len=2, ns=17) == _lib.VIT_E_UNSUPPORTED  # 4 x 2 rows x 17
    assert _decode_merged(lib, K, _plane(side=1, codec=3, signs=None)) == _lib.VIT_E_ARG  # rotated V, no signs


def test_merge_fits_matches_the_limits():
    import quantized_kv_cache_append_amd as vit

    assert vit.merge_fits(32, 8, 1, 16)           # the 16-split ladder: 4 rows x 16
    assert vit.merge_fits(40, 8, 3, 8)            # 15 rows x 8 = 120
    assert not vit.merge_fits(40, 8, 3, 9)        # 135
    assert not vit.merge_fits(16, 2, 1, 128)      # 8 rows x 128
    assert not vit.merge_fits(4, 4, 1, 65)        # 65 splits
    assert vit.merge_fits(16, 2, 1, 1)            # one split: nothing to merge


def _transcode(lib, src, dst, n_rows=(10, 10)):
    arr = None if n_rows is None else (ctypes.c_int64 * len(n_rows))(*n_rows)
    return lib.vit_kv_transcode(ctypes.byref(src), ctypes.byref(dst), arr, None)


def test_transcode_validation(lib):
    """Codec pairs, matching geometry, disjoint arrays and row counts are all
    checked on the host (no compute: every call fails or has no rows)."""
    S16 = 0x1000000  # f16 plane: codes 2 x 2 x 512 x 256 B = 512 KiB
    src = _plane(codec=0, codes=S16, scales=None, norms=None)
    dst = _plane(codec=1, codes=0x2000000, scales=0x3000000, norms=None)
    assert _transcode(lib, src, dst, n_rows=(0, 0)) == _lib.VIT_OK       # nothing to do
    assert _transcode(lib, src, dst, n_rows=(513, 0)) == _lib.VIT_E_CAPACITY
    assert _transcode(lib, src, dst, n_rows=(-1, 0)) == _lib.VIT_E_CAPACITY
    assert _transcode(lib, src, dst, n_rows=None) == _lib.VIT_E_ARG
    # overlapping arrays: the destination codes inside the source codes
    assert _transcode(lib, src, _plane(codec=1, codes=S16 + 0x40000, scales=0x3000000, norms=None)) == _lib.VIT_E_ARG
    # destination scales inside the source codes
    assert _transcode(lib, src, _plane(codec=1, codes=0x2000000, scales=S16 + 0x100, norms=None)) == _lib.VIT_E_ARG
    # geometry and side must match
    assert _transcode(lib, src, _plane(codec=1, side=1, codes=0x2000000, scales=0x3000000, norms=None)) == _lib.VIT_E_ARG
    assert _transcode(lib, src, _plane(codec=1, H=4, codes=0x2000000, scales=0x3000000, norms=None)) == _lib.VIT_E_ARG
    assert _transcode(lib, src, _plane(codec=1, cap=1024, codes=0x2000000, scales=0x3000000, norms=None)) == _lib.VIT_E_ARG
    # only degrade steps from an exactly decodable source
    q8 = _plane(codec=1, codes=0x4000000, scales=0x5000000, norms=None)
    q4 = _plane(codec=2, codes=0x6000000, scales=0x7000000, norms=None)
    r4 = _plane(codec=3, codes=0x8000000, scales=0x9000000, norms=0xA000000, signs=ctypes.addressof(_SIGNS))
    f16b = _plane(codec=0, codes=0xB000000, scales=None, norms=None)
    for a, b in ((q4, q8), (q8, f16b), (r4, q4), (q4, r4), (src, f16b), (q8, _plane(codec=1, codes=0xC000000,
                                                                                        scales=0xD000000, norms=None))):
        assert _transcode(lib, a, b) == _lib.VIT_E_UNSUPPORTED
    for a, b in ((src, q8), (src, q4), (src, r4), (q8, q4), (q8, r4)):
        assert _transcode(lib, a, b, n_rows=(0, 0)) == _lib.VIT_OK


def test_classic_next_step_matches_the_oracle():
    """The C controller step against oracle.vbr.classic_next_step on random
    ladder states, price orders, pinned sides and floors (host logic only)."""
    from oracle import vbr

    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(11)
    ladder = ["f16", "q8_0", "q4_0"]
    for trial in range(300):
        n = int(rng.integers(1, 48))
        state = [ladder[i] for i in rng.integers(0, 3, n)]
        order = [int(i) for i in rng.permutation(n)]
        movable = None if trial % 3 == 0 else [bool(x) for x in rng.random(n) < 0.8]
        floor = None if trial % 2 else float(rng.choice([4.5, 6.0, 8.5, 10.25, 12.0, 15.5]))
        assert vit.vit_vbr_classic_next_step(state, order, movable, floor) == \
            vbr.classic_next_step(state, order, movable, floor), (state, order, movable, floor)
    # a whole schedule, stepped through the C function
    state, order = ["f16"] * 32, [int(i) for i in rng.permutation(32)]
    steps = []
    while (st := vit.vit_vbr_classic_next_step(state, order, floor_bpv=6.0)) is not None:
        state[st[0]] = st[1]
        steps.append(st)
    assert steps == vbr.classic_schedule(["f16"] * 32, order, floor_bpv=6.0)


def test_classic_next_step_validation(lib):
    t, c = ctypes.c_int32(), ctypes.c_int32()

    def call(codecs, order, n=None):
        n = len(codecs) if n is None else n
        ca = (ctypes.c_int32 * max(1, len(codecs)))(*codecs)
        oa = (ctypes.c_int32 * max(1, len(order)))(*order)
        return lib.vit_vbr_classic_next_step(n, ca, oa, None, 0.0, ctypes.byref(t), ctypes.byref(c))

    assert call([0, 1], [1, 0]) == _lib.VIT_OK and (t.value, c.value) == (0, 1)
    assert call([0, 3], [0, 1]) == _lib.VIT_E_ARG   # rot4 is not on the classic ladder
    assert call([0, 0], [0, 0]) == _lib.VIT_E_ARG   # not a permutation
    assert call([0, 0], [0, 2]) == _lib.VIT_E_ARG
    assert call([], [], n=0) == _lib.VIT_E_ARG
    assert call([2, 2], [0, 1]) == _lib.VIT_OK and t.value == -1  # nothing left to degrade


def test_probe_validation(lib):
    """Attention-probe scores: K plane only, G <= 16, 1 <= seq_len <= capacity,
    finite scale and decay, aligned buffers (no compute: every case fails)."""
    K = _plane(side=0)

    def call(k=K, hq=4, seq_len=(10, 10), scale=0.088, decay=0.9, ws=FAKE, scores=FAKE, q=FAKE):
        arr = (ctypes.c_int64 * len(seq_len))(*seq_len)
        return lib.vit_attn_probe_scores(ctypes.byref(k), q, hq, arr, scale, decay, ws, scores, None)

    assert call(k=_plane(side=1)) == _lib.VIT_E_ARG
    assert call(hq=3) == _lib.VIT_E_ARG
    assert call(hq=34) == _lib.VIT_E_UNSUPPORTED          # G = 17
    assert call(seq_len=(0, 10)) == _lib.VIT_E_ARG
    assert call(seq_len=(513, 10)) == _lib.VIT_E_CAPACITY
    assert call(scale=float("inf")) == _lib.VIT_E_ARG
    assert call(decay=float("nan")) == _lib.VIT_E_ARG
    assert call(ws=None) == _lib.VIT_E_ARG
    assert call(ws=FAKE + 16) == _lib.VIT_E_ALIGN
    assert call(scores=FAKE + 4) == _lib.VIT_E_ALIGN
    assert lib.vit_attn_probe_workspace_bytes(2, 4, 512) == 2 * 4 * 512 * 4 + 2 * 4 * 64 * 2 * 4
    assert lib.vit_attn_probe_workspace_bytes(2, 300, 512) == 0


def test_select_evictions_validation(lib):
    def call(seq_len=(10, 10), ns=2, nr=2, ne=3, rows=FAKE, nout=FAKE, scores=FAKE, cap=512, ws=FAKE):
        arr = (ctypes.c_int64 * len(seq_len))(*seq_len)
        return lib.vit_probe_select_evictions(scores, len(seq_len), cap, arr, ns, nr, ne, rows, nout, ws, None)

    assert call(seq_len=(513, 1)) == _lib.VIT_E_CAPACITY
    assert call(seq_len=(-1, 1)) == _lib.VIT_E_CAPACITY
    assert call(ns=-1) == _lib.VIT_E_ARG
    assert call(ne=-2) == _lib.VIT_E_ARG
    assert call(rows=None) == _lib.VIT_E_ARG
    assert call(nout=None) == _lib.VIT_E_ARG
    assert call(scores=None) == _lib.VIT_E_ARG
    assert call(rows=FAKE + 4) == _lib.VIT_E_ALIGN
    assert call(ws=None) == _lib.VIT_E_ARG
    assert call(ws=FAKE + 64) == _lib.VIT_E_ALIGN
    assert call(seq_len=(1,) * 65) == _lib.VIT_E_UNSUPPORTED
    assert lib.vit_probe_select_workspace_bytes(3) == 3 * (3 * 2048 + 256 * 2) * 4
    assert lib.vit_probe_select_workspace_bytes(0) == 0


def test_reduce_validation(lib):
    V = _plane(side=1)
    r = lib.vit_attn_splitk_reduce
    assert r(FAKE, 2, 4, 128, 1, ctypes.byref(V), FAKE, None) == _lib.VIT_E_ARG
    assert r(FAKE, 2, 4, 64, 4, ctypes.byref(V), FAKE, None) == _lib.VIT_E_UNSUPPORTED
    assert r(None, 2, 4, 128, 4, ctypes.byref(V), FAKE, None) == _lib.VIT_E_ARG
    assert r(FAKE, 2, 4, 128, 4, ctypes.byref(_plane(side=1, codec=3)), FAKE, None) == _lib.VIT_E_ARG
    assert r(FAKE + 4, 2, 4, 128, 4, ctypes.byref(V), FAKE, None) == _lib.VIT_E_ALIGN


def test_arm_kernel_events_validation(lib):
    assert lib.vit_arm_kernel_events(FAKE, None) == _lib.VIT_E_ARG
    assert lib.vit_arm_kernel_events(None, FAKE) == _lib.VIT_E_ARG
    assert lib.vit_arm_kernel_events(None, None) == _lib.VIT_OK
    # armed fake events are consumed by the next decode call even when it fails
    # validation, so they are never handed to the runtime
    assert lib.vit_arm_kernel_events(FAKE, FAKE) == _lib.VIT_OK
    assert _decode(lib, _plane(side=0), _plane(side=1), ns=0) == _lib.VIT_E_ARG
    assert lib.vit_arm_kernel_events(None, None) == _lib.VIT_OK


# ------------------------------------------------------------- host layout
@pytest.mark.parametrize("codec", ["f16", "q8_0", "q4_0", "rot4", "rot3"])
@pytest.mark.parametrize("side", ["k", "v"])
def test_layout_is_a_bijection(codec, side):
    rng = np.random.default_rng(3)
    S, H, cap = 2, 3, 256
    if codec == "f16":
        codes = rng.integers(0, 65536, (S, H, cap, 128)).astype(np.uint16)
    elif codec == "q8_0":
        codes = rng.integers(-127, 128, (S, H, cap, 128)).astype(np.int8)
    else:
        codes = rng.integers(0, 8 if codec == "rot3" else 16, (S, H, cap, 128)).astype(np.uint8)
    raw = np.zeros(S * H * cap * layout.ROW_BYTES[codec], np.uint8)
    layout.pack_codes(codec, side, codes, raw)
    back = layout.unpack_codes(codec, side, raw, S, H, cap)
    assert np.array_equal(back, codes)


def test_k_layout_16_byte_units_are_contiguous_per_lane():
    """Each wave-wide 16-byte load of a K tile covers 1 KB of contiguous bytes:
    unit (half, c) of lane l = 16 g + r sits at ((half*CB + c)*64 + l)*16 and
    holds chunk g (CHB = RB/16 canonical bytes) of each of the 4/CB blocks of
    unit c, in block order (include/vit.h, K-side tile)."""
    for codec in ("f16", "q8_0", "q4_0", "rot4"):
        rb = layout.ROW_BYTES[codec]
        perm = layout._k_perm(codec)
        cb = rb // 64
        bpu, chb = 4 // cb, rb // 16
        offs = np.sort(perm.reshape(-1))
        assert np.array_equal(offs, np.arange(32 * rb))
        for p in range(32):
            h, r = p >> 4, p & 15
            for g in range(4):
                for c in range(cb):
                    unit = ((h * cb + c) * 64 + 16 * g + r) * 16
                    for bb in range(bpu):
                        for k in range(chb):
                            byte = (c * bpu + bb) * (rb // 4) + g * chb + k
                            assert perm[p, byte] == unit + bb * chb + k


@pytest.mark.parametrize("side", ["k", "v"])
def test_scales_layout_roundtrip(side):
    rng = np.random.default_rng(4)
    s = rng.integers(0, 65536, (2, 3, 256, 4)).astype(np.uint16)
    assert np.array_equal(layout.unpack_scales(side, layout.pack_scales(side, s), 2, 3, 256), s)


def test_no_kernel_spills_to_scratch():
    """The build records the compiler's resource usage per kernel: no kernel
    may use scratch memory (register spills cost the decode its stream
    rate), and every decode instantiation must fit two 8-wave workgroups'
    worth of waves per SIMD, the occupancy its launch is planned for."""
    import json
    import os

    from quantized_kv_cache_append_amd import build

    if not os.path.exists(build.RESOURCES):
        pytest.skip("library not built here")
    res = json.load(open(build.RESOURCES))
    spilled = {k: v["scratch"] for k, v in res.items() if v.get("scratch", 0) or v.get("vgpr_spill", 0)}
    assert not spilled, f"kernels with scratch: {spilled}"
    decode = {k: v for k, v in res.items() if "decode_kernel" in k}
    assert len(decode) == 75, "5 K codecs x 5 V codecs x 3 row layouts"
    assert all(v["waves_per_simd"] >= 2 for v in decode.values())

