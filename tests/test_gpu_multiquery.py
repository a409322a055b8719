"""GPU parity of vit_attn_decode_mq (several new tokens per sequence, causal
among themselves) + vit_attn_splitk_reduce against the oracle's
decode_multi_reference.

Bar: max |o_gpu - o_ref| <= 2e-3 x RMS(o_ref) per call.  Covers both wave
layouts (4 and 8 query rows), two row groups (G * q_len = 16), fused appends
whose new rows straddle tiles owned by different splits (codes checked
bit-exact), q_len = 1 against vit_attn_decode, and the verify steps bench.py
times at full size (sampled (sequence, KV head) units, the library's default
split count).
"""

import math

import numpy as np
import pytest

import synth
from gpu_helpers import append_rows, check_close, compare_plane_rows, fill_plane_synth, make_plane, say, torch_cuda
from oracle import attention

D = 128


def _rows(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    ch = rng.choice(D, 2, replace=False)
    x[..., ch] *= 20.0
    return x


def _run(kc, vc, G, q_len, lens, n_splits, fused, seed, S=2, H=2, cap=512):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(seed)
    ks = rng.integers(0, 256, 16, dtype=np.uint8) if kc in ("rot4", "rot3") else None
    vs = rng.integers(0, 256, 16, dtype=np.uint8) if vc in ("rot4", "rot3") else None
    K = make_plane(kc, "k", S, H, cap, ks)
    V = make_plane(vc, "v", S, H, cap, vs)
    Lmax = max(lens)
    kx = _rows(rng, (S, Lmax, H, D))
    vx = _rows(rng, (S, Lmax, H, D))
    Hq = H * G
    q = _rows(rng, (S, q_len, Hq, D))
    if fused:
        # one call writes every sequence's rows before its q_len new ones; a
        # sequence with a shorter prefix gets junk rows past it, which the
        # fused append of the decode call must overwrite
        n_pre = [l - q_len for l in lens]
        P = max(n_pre)
        if P > 0:
            pk = _rows(rng, (S, P, H, D))
            pv = _rows(rng, (S, P, H, D))
            for s in range(S):
                pk[s, :n_pre[s]] = kx[s, :n_pre[s]]
                pv[s, :n_pre[s]] = vx[s, :n_pre[s]]
            append_rows(K, pk, [0] * S)
            append_rows(V, pv, [0] * S)
        k_new = np.stack([kx[s, lens[s] - q_len:lens[s]] for s in range(S)])  # [S][q_len][H][D]
        v_new = np.stack([vx[s, lens[s] - q_len:lens[s]] for s in range(S)])
        knd = torch.from_numpy(np.ascontiguousarray(k_new)).cuda()
        vnd = torch.from_numpy(np.ascontiguousarray(v_new)).cuda()
    else:
        append_rows(K, kx, [0] * S)
        append_rows(V, vx, [0] * S)
        knd = vnd = None
    out = vit.decode(K, V, torch.from_numpy(q).cuda(), Hq, lens, k_new=knd, v_new=vnd, n_splits=n_splits,
                     q_len=q_len)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert got.shape == (S, q_len, Hq, D)
    ref = np.zeros_like(got, dtype=np.float64)
    for s in range(S):
        L = lens[s]
        for h in range(H):
            ref[s, :, h * G:(h + 1) * G] = attention.decode_multi_reference(
                q[s, :, h * G:(h + 1) * G], kx[s, :L, h], vx[s, :L, h], kc, vc, 1.0 / math.sqrt(D), ks, vs)
    return got, ref, (K, V, kx, vx, ks, vs)


CASES = [
    # kc, vc, G, q_len, lens, n_splits, fused
    ("q8_0", "q8_0", 4, 2, [300, 37], 3, True),    # 8 rows: wide layout; new rows 35, 36 cross no tile
    ("q4_0", "q4_0", 4, 4, [129, 66], 2, True),    # 16 rows: two row groups; rows 126..128 straddle tiles 3/4
    ("rot4", "q4_0", 2, 3, [96, 33], 2, True),     # 6 rows; rows 30..32 straddle tiles 0/1 (two splits)
    ("f16", "rot4", 1, 4, [5, 260], 5, True),      # 4 rows: narrow layout; a 5-row sequence
    ("q8_0", "f16", 8, 2, [70, 200], 1, False),   # 16 rows, one split (normalised output straight from decode)
    ("rot4", "rot4", 4, 3, [31, 97], 4, True),     # 12 rows
    ("rot3", "rot3", 2, 4, [64, 130], 3, True),    # 8 rows, 3-bit rotated K and V
    ("rot3", "q8_0", 4, 4, [40, 300], 2, True),    # 16 rows
]


@pytest.mark.gpu
@pytest.mark.parametrize("kc,vc,G,q_len,lens,n_splits,fused", CASES)
def test_multi_token_decode(kc, vc, G, q_len, lens, n_splits, fused):
    say(f"[decode-mq] K={kc} V={vc} G={G} q_len={q_len} lens={lens} splits={n_splits} fused={fused}")
    got, ref, (K, V, kx, vx, ks, vs) = _run(kc, vc, G, q_len, lens, n_splits, fused, seed=700 + G * 10 + q_len)
    check_close(got, ref, f"K={kc} V={vc} G={G} q_len={q_len}")
    if fused:
        # the fused rows are stored exactly as vit_kv_append_quant stores them
        view_k, view_v = K.host_view(), V.host_view()
        for s in range(len(lens)):
            for h in range(K.n_kv_heads):
                idx = np.arange(lens[s] - q_len, lens[s])
                compare_plane_rows(K, view_k, s, h, idx, kx[s, idx, h])
                compare_plane_rows(V, view_v, s, h, idx, vx[s, idx, h])


@pytest.mark.gpu
def test_single_token_mq_equals_decode():
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    say("[decode-mq] q_len 1 vs vit_attn_decode")
    rng = np.random.default_rng(77)
    S, H, G, cap = 2, 2, 4, 512
    K = make_plane("q8_0", "k", S, H, cap)
    V = make_plane("q4_0", "v", S, H, cap)
    append_rows(K, _rows(rng, (S, 200, H, D)), [0] * S)
    append_rows(V, _rows(rng, (S, 200, H, D)), [0] * S)
    q = torch.from_numpy(_rows(rng, (S, H * G, D))).cuda()
    a = vit.decode(K, V, q, H * G, [200, 150], n_splits=3)
    b = vit.decode(K, V, q.reshape(S, 1, H * G, D), H * G, [200, 150], n_splits=3, q_len=1)
    torch.cuda.synchronize()
    a, b = a.cpu().numpy(), b.cpu().numpy()[:, 0]
    rms = float(np.sqrt(np.mean(a.astype(np.float64) ** 2)))
    assert np.max(np.abs(a - b)) <= 1e-5 * rms


def _run_workload_verify(cfg, q_len, units):
    """A workload's cache at full size, q_len new tokens per sequence appended
    by the decode call, as bench.py --q-len runs it; the sampled units are
    checked against the oracle over the same synth rows."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    c = synth.CONFIGS[cfg]
    S, Hq, H, cap, L = c["seqs"], c["hq"], c["hkv"], c["capacity"], c["ctx"]
    G = Hq // H
    kc, vc = synth.codec_map(cfg)[0]
    ks = synth.sign_mask(cfg, 0, "k") if kc in ("rot4", "rot3") else None
    vs = synth.sign_mask(cfg, 0, "v") if vc in ("rot4", "rot3") else None
    say(f"[verify {c['name']}] K={kc} V={vc} q_len={q_len} units={units}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1000 + synth.SEED_ID[cfg])
    K = make_plane(kc, "k", S, H, cap, ks)
    V = make_plane(vc, "v", S, H, cap, vs)
    fill_plane_synth(K, cfg, 0, "k", 0, L - q_len, units, torch, gen)
    fill_plane_synth(V, cfg, 0, "v", 0, L - q_len, units, torch, gen)
    k_new = torch.randn((S, q_len, H, D), generator=gen, device="cuda")
    v_new = torch.randn((S, q_len, H, D), generator=gen, device="cuda")
    for (s, h) in units:
        k_new[s, :, h] = torch.from_numpy(synth.kv_rows(cfg, "k", 0, s, h, L - q_len, q_len)).cuda()
        v_new[s, :, h] = torch.from_numpy(synth.kv_rows(cfg, "v", 0, s, h, L - q_len, q_len)).cuda()
    q = np.random.default_rng(4242 + synth.SEED_ID[cfg]).standard_normal((S, q_len, Hq, D)).astype(np.float32)
    ns = vit.vit_attn_default_splits(S, H, Hq, L)
    out = vit.decode(K, V, torch.from_numpy(q).cuda(), Hq, [L] * S, k_new=k_new, v_new=v_new, n_splits=ns,
                     q_len=q_len)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gots, refs = [], []
    for (s, h) in units:
        kr = synth.kv_rows(cfg, "k", 0, s, h, 0, L)
        vr = synth.kv_rows(cfg, "v", 0, s, h, 0, L)
        refs.append(attention.decode_multi_reference(q[s, :, h * G:(h + 1) * G], kr, vr, kc, vc,
                                                     1.0 / math.sqrt(D), ks, vs))
        gots.append(got[s, :, h * G:(h + 1) * G])
    check_close(np.stack(gots), np.stack(refs), f"{c['name']} verify q_len={q_len} splits={ns}")
    del K, V
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_workload_batched_verify4():
    _run_workload_verify("batched", 4, [(0, 0), (5, 3)])


@pytest.mark.gpu
def test_workload_lowbit_verify3():
    _run_workload_verify("lowbit", 3, [(2, 6)])


@pytest.mark.gpu
def test_workload_rotated_verify2():
    _run_workload_verify("rotated", 2, [(0, 1)])
