"""Seeded randomized GPU parity over many small shapes (the cases are fixed by
the seed, so the test is repeatable):

* vit_kv_append_quant_multi with random plane counts, codecs, sides,
  sequence and KV-head counts, capacities, start rows and row counts must
  leave every plane exactly as per-plane vit_kv_append_quant calls do, and
  hold the oracle's encoding of the appended rows;
* vit_attn_decode_merged with random codec pairs, GQA ratios, new-token
  counts, lengths (ragged across sequences, some below one tile) and split
  counts must equal decode + reduce bit for bit and lie within 2e-3 x RMS of
  the oracle.
"""

import math

import numpy as np
import pytest

from gpu_helpers import append_rows, check_close, compare_plane_rows, make_plane, say, torch_cuda
from oracle import attention

D = 128
CODECS = ["f16", "q8_0", "q4_0", "rot4", "rot3"]


def _signs(rng, codec):
    return rng.integers(0, 256, 16, dtype=np.uint8) if codec in ("rot4", "rot3") else None


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(12))
def test_fuzz_append_multi(case):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(7000 + case)
    n_planes = int(rng.integers(1, 9))
    S, H = int(rng.integers(1, 5)), int(rng.integers(1, 4))
    cap = 256 * int(rng.integers(1, 4))
    T = int(rng.integers(1, 160))
    pos0 = [int(rng.integers(0, cap - T + 1)) for _ in range(S)]
    kinds = [(CODECS[int(rng.integers(0, 5))], ("k", "v")[int(rng.integers(0, 2))]) for _ in range(n_planes)]
    say(f"[fuzz-append] case {case}: {n_planes} planes {kinds} S={S} H={H} cap={cap} T={T} pos0={pos0}")
    pairs = []
    for codec, side in kinds:
        sg = _signs(rng, codec)
        pairs.append((make_plane(codec, side, S, H, cap, sg), make_plane(codec, side, S, H, cap, sg)))
    xs = [(rng.standard_normal((S, T, H, D)) * rng.lognormal(0, 1, (S, T, H, 1))).astype(np.float32)
          for _ in kinds]
    srcs = [torch.from_numpy(x).cuda() for x in xs]
    vit.vit_kv_append_quant_multi([m for m, _ in pairs], srcs, pos0)
    for (_, single), src in zip(pairs, srcs):
        vit.vit_kv_append_quant(single, src, pos0)
    torch.cuda.synchronize()
    for i, ((multi, single), x) in enumerate(zip(pairs, xs)):
        for a, b in zip(multi.tensors(), single.tensors()):
            assert bool((a == b).all()), f"case {case} plane {i} {kinds[i]}: multi != single"
        view = multi.host_view()
        for s in range(S):
            for h in range(H):
                compare_plane_rows(multi, view, s, h, pos0[s] + np.arange(T), x[s, :, h])


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(16))
def test_fuzz_decode_merged(case):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(9000 + case)
    kc, vc = CODECS[int(rng.integers(0, 5))], CODECS[int(rng.integers(0, 5))]
    S, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    q_len = int(rng.integers(1, 5))
    G = int(rng.integers(1, 16 // q_len + 1))
    cap = 256 * int(rng.integers(1, 5))
    lens = [int(rng.integers(q_len, cap + 1)) for _ in range(S)]
    rows = G * q_len
    max_ns = min(64, 128 // rows)
    ns = int(rng.integers(2, max_ns + 1))
    fused = bool(rng.integers(0, 2))
    Hq = H * G
    say(f"[fuzz-decode] case {case}: K={kc} V={vc} S={S} H={H} G={G} q_len={q_len} lens={lens} splits={ns} "
        f"fused={fused}")
    ks, vs = _signs(rng, kc), _signs(rng, vc)
    K, V = make_plane(kc, "k", S, H, cap, ks), make_plane(vc, "v", S, H, cap, vs)
    Lmax = max(lens)
    kx = rng.standard_normal((S, Lmax, H, D)).astype(np.float32)
    vx = rng.standard_normal((S, Lmax, H, D)).astype(np.float32)
    q = rng.standard_normal((S, q_len, Hq, D)).astype(np.float32)
    knd = vnd = None
    if fused:
        # the rows before each sequence's new tokens are stored first (a
        # sequence with fewer of them also gets some of its new-token rows,
        # with the same values the decode call stores again)
        _fill_exact(K, V, kx, vx, [lens[s] - q_len for s in range(S)])
        knd = torch.from_numpy(np.ascontiguousarray(
            np.stack([kx[s, lens[s] - q_len:lens[s]] for s in range(S)]))).cuda()
        vnd = torch.from_numpy(np.ascontiguousarray(
            np.stack([vx[s, lens[s] - q_len:lens[s]] for s in range(S)]))).cuda()
    else:
        _fill_exact(K, V, kx, vx, lens)
    qd = torch.from_numpy(q).cuda()
    ws = torch.empty(vit.vit_attn_workspace_bytes(S, Hq * q_len, D, ns), dtype=torch.uint8, device="cuda")
    two = torch.full((S, q_len, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    vit.vit_attn_decode_mq(K, V, qd, Hq, q_len, lens, knd, vnd, None, ns, ws, two)
    vit.vit_attn_splitk_reduce(ws, S, Hq * q_len, D, ns, V, two)
    counters = vit.merge_counters(K)
    one = torch.full_like(two, float("nan"))
    vit.vit_attn_decode_merged(K, V, qd, Hq, q_len, lens, one, ws, counters, knd, vnd, None, ns)
    torch.cuda.synchronize()
    assert torch.equal(one, two), f"case {case}: merged != decode + reduce"
    assert int(counters.abs().sum()) == 0
    got = one.cpu().numpy()
    ref = np.zeros_like(got, dtype=np.float64)
    for s in range(S):
        L = lens[s]
        for h in range(H):
            ref[s, :, h * G:(h + 1) * G] = attention.decode_multi_reference(
                q[s, :, h * G:(h + 1) * G], kx[s, :L, h], vx[s, :L, h], kc, vc, 1.0 / math.sqrt(D), ks, vs)
    check_close(got, ref, f"fuzz decode case {case} K={kc} V={vc}")


def _fill_exact(K, V, kx, vx, counts):
    """Store rows 0 .. counts[s]-1 of every sequence s: one call over the
    longest count, the rows past a sequence's count taken from its own data
    too (they are never read: each sequence attends only its own length)."""
    n = max(counts)
    if n > 0:
        append_rows(K, kx[:, :n], [0] * K.n_seqs)
        append_rows(V, vx[:, :n], [0] * V.n_seqs)
