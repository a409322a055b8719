"""GPU parity of vit_attn_decode_merged (decode attention and its split merge
in one launch: the last workgroup of each (sequence, KV head) merges that
head's partials) against the two-call path (vit_attn_decode_mq +
vit_attn_splitk_reduce) and against the oracle's decode_multi_reference.

Bar: the output equals the two-call output bit for bit (the merge shares the
reduce kernel's arithmetic), is within 2e-3 x RMS of the oracle, the arrival
counters are back at zero after every call, and the partials the call leaves
in the workspace reduce to the same output.  Covers both rotated V codecs
(inverse WHT after the merge), query rows per KV head from 1 to 16, split
counts 2..64 up to the 128-partial-row limit, splits that own no tile, fused
appends whose rows straddle splits, several calls in a row on one counter
buffer, and the batched and low-bit workloads at full size with the default
split count.
"""

import math

import numpy as np
import pytest

import synth
from gpu_helpers import append_rows, check_close, fill_plane_synth, make_plane, say, torch_cuda
from oracle import attention

D = 128


def _rows(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    ch = rng.choice(D, 2, replace=False)
    x[..., ch] *= 20.0
    return x


def _setup(kc, vc, G, q_len, lens, fused, seed, S=2, H=2, cap=512):
    """Planes holding the rows before the new ones (all rows without a fused
    append), the host rows, device queries and the new rows."""
    torch = torch_cuda()
    rng = np.random.default_rng(seed)
    ks = rng.integers(0, 256, 16, dtype=np.uint8) if kc in ("rot4", "rot3") else None
    vs = rng.integers(0, 256, 16, dtype=np.uint8) if vc in ("rot4", "rot3") else None
    K = make_plane(kc, "k", S, H, cap, ks)
    V = make_plane(vc, "v", S, H, cap, vs)
    Lmax = max(lens)
    kx = _rows(rng, (S, Lmax, H, D))
    vx = _rows(rng, (S, Lmax, H, D))
    q = _rows(rng, (S, q_len, H * G, D))
    knd = vnd = None
    if fused:
        P = max(lens) - q_len
        if P > 0:
            append_rows(K, kx[:, :P], [0] * S)
            append_rows(V, vx[:, :P], [0] * S)
        knd = torch.from_numpy(np.ascontiguousarray(np.stack([kx[s, lens[s] - q_len:lens[s]] for s in range(S)]))).cuda()
        vnd = torch.from_numpy(np.ascontiguousarray(np.stack([vx[s, lens[s] - q_len:lens[s]] for s in range(S)]))).cuda()
    else:
        append_rows(K, kx, [0] * S)
        append_rows(V, vx, [0] * S)
    return K, V, kx, vx, ks, vs, q, torch.from_numpy(q).cuda(), knd, vnd


def _two_calls(vit, torch, K, V, qd, Hq, q_len, lens, knd, vnd, n_splits):
    S = K.n_seqs
    ws = torch.empty(vit.vit_attn_workspace_bytes(S, Hq * q_len, D, n_splits), dtype=torch.uint8, device="cuda")
    out = torch.full((S, q_len, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    vit.vit_attn_decode_mq(K, V, qd, Hq, q_len, lens, knd, vnd, None, n_splits, ws, out)
    if n_splits > 1:
        vit.vit_attn_splitk_reduce(ws, S, Hq * q_len, D, n_splits, V, out)
    return out


def _merged(vit, torch, K, V, qd, Hq, q_len, lens, knd, vnd, n_splits, counters, ws=None):
    S = K.n_seqs
    if ws is None:
        ws = torch.empty(vit.vit_attn_workspace_bytes(S, Hq * q_len, D, n_splits), dtype=torch.uint8, device="cuda")
    out = torch.full((S, q_len, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    vit.vit_attn_decode_merged(K, V, qd, Hq, q_len, lens, out, ws, counters, knd, vnd, None, n_splits)
    return out, ws


CASES = [
    # kc, vc, G, q_len, lens, n_splits, fused
    ("q8_0", "q8_0", 4, 1, [300, 37], 4, True),     # batched-like; the 37-row sequence leaves 2 splits empty
    ("q4_0", "rot4", 5, 1, [512, 200], 8, False),   # G 5 (low-bit), rotated V: WHT after the merge
    ("f16", "q4_0", 1, 1, [129, 480], 64, False),   # 64 splits, most of them empty for 129 rows
    ("rot4", "rot3", 8, 1, [260, 33], 16, True),    # 8 rows x 16 splits = the 128-row limit
    ("rot3", "f16", 4, 4, [200, 100], 8, True),     # 16 rows (two chained hi/lo MFMAs) x 8
    ("q8_0", "rot4", 2, 3, [97, 31], 3, True),      # 6 rows; new rows straddle tiles of two splits
    ("q4_0", "q8_0", 16, 1, [500, 511], 2, False),  # 16 query heads per KV head, 2 splits
    ("rot4", "q4_0", 4, 1, [512, 512], 2, True),    # the fused append's tile is the last of split 1
]
# a split of 32 tiles: the new rows' tile is past every wave's first slots,
# so the other waves prefetch while the rows are encoded
LATE = [
    ("q8_0", "f16", 4, 1, [2000, 1500], 2, True),
    ("q4_0", "q4_0", 4, 3, [2048, 1111], 2, True),
]


@pytest.mark.gpu
@pytest.mark.parametrize("kc,vc,G,q_len,lens,n_splits,fused,cap", [c + (512,) for c in CASES] + [c + (2048,) for c in LATE])
def test_merged_equals_two_calls(kc, vc, G, q_len, lens, n_splits, fused, cap):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    say(f"[merged] K={kc} V={vc} G={G} q_len={q_len} lens={lens} splits={n_splits} fused={fused} cap={cap}")
    K, V, kx, vx, ks, vs, q, qd, knd, vnd = _setup(kc, vc, G, q_len, lens, fused, seed=900 + 7 * G + q_len, cap=cap)
    Hq = K.n_kv_heads * G
    assert vit.merge_fits(Hq, K.n_kv_heads, q_len, n_splits)
    two = _two_calls(vit, torch, K, V, qd, Hq, q_len, lens, knd, vnd, n_splits)
    counters = vit.merge_counters(K)
    for rep in range(2):  # the second call finds the counters its predecessor left at zero
        one, ws = _merged(vit, torch, K, V, qd, Hq, q_len, lens, knd, vnd, n_splits, counters)
        torch.cuda.synchronize()
        assert torch.equal(one, two), f"call {rep}: merged output differs from decode + reduce"
        assert int(counters.abs().sum()) == 0, f"call {rep}: arrival counters not back at zero"
    # the partials left in the workspace reduce to the same rows
    again = torch.full_like(two, float("nan"))
    vit.vit_attn_splitk_reduce(ws, K.n_seqs, Hq * q_len, D, n_splits, V, again)
    torch.cuda.synchronize()
    assert torch.equal(again, two)
    got = one.cpu().numpy()
    ref = np.zeros_like(got, dtype=np.float64)
    for s in range(K.n_seqs):
        L = lens[s]
        for h in range(K.n_kv_heads):
            ref[s, :, h * G:(h + 1) * G] = attention.decode_multi_reference(
                q[s, :, h * G:(h + 1) * G], kx[s, :L, h], vx[s, :L, h], kc, vc, 1.0 / math.sqrt(D), ks, vs)
    check_close(got, ref, f"merged K={kc} V={vc} G={G} q_len={q_len}")


@pytest.mark.gpu
def test_merged_calls_of_different_shapes_share_counters():
    """One counter buffer (zeroed once) serves calls of different geometry and
    split count in a row: each equals its two-call result."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    counters = torch.zeros(64, dtype=torch.int32, device="cuda")
    shapes = [  # kc, vc, G, q_len, lens, n_splits, S, H
        ("q8_0", "q4_0", 4, 1, [400, 130, 64], 6, 3, 2),
        ("rot4", "f16", 2, 2, [250], 32, 1, 4),
        ("f16", "rot3", 8, 1, [511, 3], 5, 2, 1),
        ("q8_0", "q4_0", 4, 1, [400, 130, 64], 6, 3, 2),
    ]
    for i, (kc, vc, G, q_len, lens, ns, S, H) in enumerate(shapes):
        say(f"[merged] shared counters, call {i}: K={kc} V={vc} S={S} H={H} G={G} splits={ns}")
        K, V, kx, vx, ks, vs, q, qd, knd, vnd = _setup(kc, vc, G, q_len, lens, True, seed=1300 + i, S=S, H=H)
        Hq = H * G
        two = _two_calls(vit, torch, K, V, qd, Hq, q_len, lens, knd, vnd, ns)
        one, _ = _merged(vit, torch, K, V, qd, Hq, q_len, lens, knd, vnd, ns, counters)
        torch.cuda.synchronize()
        assert torch.equal(one, two), f"call {i}"
        assert int(counters.abs().sum()) == 0


def _full_size(cfg, unit_count=2):
    """A workload's cache at full size with its new token appended by the
    call, at the library's default split count: merged == two calls bit for
    bit, and sampled units within tolerance of the oracle."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    c = synth.CONFIGS[cfg]
    S, Hq, H, cap, L = c["seqs"], c["hq"], c["hkv"], c["capacity"], c["ctx"]
    G = Hq // H
    kc, vc = c["k_codec"], c["v_codec"]
    ns = vit.vit_attn_default_splits(S, H, Hq, L)
    assert vit.merge_fits(Hq, H, 1, ns), f"{cfg}: {ns} splits"
    say(f"[merged] {cfg} full size: S={S} Hq={Hq} Hkv={H} L={L} {kc}/{vc} splits={ns}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.SEED_ID[cfg] + 2000)
    K = make_plane(kc, "k", S, H, cap, poison=False)
    V = make_plane(vc, "v", S, H, cap, poison=False)
    units = [(s, h) for s in range(S) for h in range(H)][::max(1, S * H // unit_count)][:unit_count]
    for side, P in (("k", K), ("v", V)):
        fill_plane_synth(P, cfg, 0, side, 0, L - 1, units, torch, gen)
    q = torch.randn((S, 1, Hq, D), generator=gen, device="cuda")
    kn = torch.randn((S, 1, H, D), generator=gen, device="cuda")
    vn = torch.randn((S, 1, H, D), generator=gen, device="cuda")
    two = _two_calls(vit, torch, K, V, q, Hq, 1, [L] * S, kn, vn, ns)
    counters = vit.merge_counters(K)
    one, _ = _merged(vit, torch, K, V, q, Hq, 1, [L] * S, kn, vn, ns, counters)
    torch.cuda.synchronize()
    assert torch.equal(one, two), f"{cfg}: merged output differs from decode + reduce"
    assert int(counters.abs().sum()) == 0
    got = one.cpu().numpy()[:, 0]
    qh = q.cpu().numpy()[:, 0]
    knh, vnh = kn.cpu().numpy()[:, 0], vn.cpu().numpy()[:, 0]
    for s, h in units:
        kr = np.concatenate([synth.kv_rows(cfg, "k", 0, s, h, 0, L - 1), knh[s, h][None]], 0)
        vr = np.concatenate([synth.kv_rows(cfg, "v", 0, s, h, 0, L - 1), vnh[s, h][None]], 0)
        ref = attention.decode_multi_reference(qh[s, h * G:(h + 1) * G][None], kr, vr, kc, vc, 1.0 / math.sqrt(D))
        check_close(got[s, h * G:(h + 1) * G], ref[0], f"merged {cfg} unit ({s},{h})")


@pytest.mark.gpu
@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", ["batched", "lowbit"])
def test_merged_full_size(cfg):
    _full_size(cfg)
