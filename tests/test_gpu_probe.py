"""GPU parity of the attention-probe cell scores (vit_attn_probe_scores)
against oracle.probe, and of the eviction choice (vit_probe_select_evictions),
which must equal the oracle's exactly on the same fp32 scores.

Scores bar: every cell within 1e-4 relative (+ 1e-6 of the largest score) of
the fp64 definition.  The logits carry the decode path's operand error
(2^-21 relative: exact K codes, fp16 hi + lo query), then fp32 exp2 and
sums, so the error is a few 1e-6 relative.  Cells at or past L: unchanged.
"""

import math

import numpy as np
import pytest

import synth
from gpu_helpers import append_rows, fill_plane_synth, make_plane, say, torch_cuda
from oracle import probe

D = 128
SCALE = 1.0 / math.sqrt(D)


def _rows(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    ch = rng.choice(D, 2, replace=False)
    x[..., ch] *= 12.0
    return x


def _check_scores(got, prev, mass, decay, L, what):
    exp = decay * prev[:L].astype(np.float64) + mass
    err = np.abs(got[:L].astype(np.float64) - exp)
    bound = 1e-4 * np.abs(exp) + 1e-6 * np.abs(exp).max()
    worst = int(np.argmax(err - bound))
    say(f"  {what}: max rel err {float(np.max(err / np.maximum(np.abs(exp), 1e-30))):.2e}")
    assert np.all(err <= bound), f"{what}: cell {worst} got {got[worst]} expected {exp[worst]}"
    assert np.array_equal(got[L:], prev[L:]), f"{what}: cells past L changed"


@pytest.mark.gpu
@pytest.mark.parametrize("kc", ["f16", "q8_0", "q4_0", "rot4", "rot3"])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_probe_scores_match_oracle(kc, G):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    say(f"[probe] K={kc} G={G}")
    rng = np.random.default_rng(300 + 10 * G + ["f16", "q8_0", "q4_0", "rot4", "rot3"].index(kc))
    S, H, cap = 3, 2, 512
    lens = [300, 37, 1]
    ks = rng.integers(0, 256, 16, dtype=np.uint8) if kc in ("rot4", "rot3") else None
    K = make_plane(kc, "k", S, H, cap, ks)
    kx = _rows(rng, (S, cap, H, D))
    append_rows(K, kx, [0] * S)
    Hq = G * H
    q = _rows(rng, (S, Hq, D)) * 0.5
    prev = rng.random((S, cap)).astype(np.float32)
    scores = torch.from_numpy(prev.copy()).cuda()
    vit.vit_attn_probe_scores(K, torch.from_numpy(q).cuda(), Hq, lens, scores, decay=0.8)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    for s in range(S):
        L = lens[s]
        mass = probe.cell_mass(q[s], np.stack([kx[s, :L, h] for h in range(H)]), kc, SCALE, ks)
        _check_scores(got[s], prev[s], mass, 0.8, L, f"K={kc} G={G} seq {s}")


@pytest.mark.gpu
def test_probe_two_events_decay():
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(31)
    S, H, cap, G = 2, 2, 256, 4
    K = make_plane("q8_0", "k", S, H, cap)
    kx = _rows(rng, (S, cap, H, D))
    append_rows(K, kx, [0] * S)
    q1, q2 = _rows(rng, (S, G * H, D)), _rows(rng, (S, G * H, D))
    scores = torch.zeros((S, cap), dtype=torch.float32, device="cuda")
    vit.vit_attn_probe_scores(K, torch.from_numpy(q1).cuda(), G * H, [200, 256], scores, decay=0.5)
    vit.vit_attn_probe_scores(K, torch.from_numpy(q2).cuda(), G * H, [200, 256], scores, decay=0.5)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    for s, L in enumerate([200, 256]):
        keys = np.stack([kx[s, :L, h] for h in range(H)])
        m1 = probe.cell_mass(q1[s], keys, "q8_0", SCALE)
        m2 = probe.cell_mass(q2[s], keys, "q8_0", SCALE)
        first = probe.decay_update(np.zeros(L), m1, 0.5)
        _check_scores(got[s], np.concatenate([first.astype(np.float32), np.zeros(cap - L, np.float32)]),
                      m2, 0.5, L, f"two events seq {s}")


def _run_probe_workload(cfg, seqs):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    c = synth.CONFIGS[cfg]
    S, Hq, H, cap, L = c["seqs"], c["hq"], c["hkv"], c["capacity"], c["ctx"]
    kc = synth.codec_map(cfg)[0][0]
    ks = synth.sign_mask(cfg, 0, "k") if kc in ("rot4", "rot3") else None
    say(f"[probe {c['name']}] K={kc} S={S} Hq={Hq} L={L} sampled seqs {seqs}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2000 + synth.SEED_ID[cfg])
    K = make_plane(kc, "k", S, H, cap, ks)
    fill_plane_synth(K, cfg, 0, "k", 0, L, [(s, h) for s in seqs for h in range(H)], torch, gen)
    torch.cuda.empty_cache()
    q = np.stack([synth.q_rows(cfg, 0, s, Hq) for s in range(S)])
    scores = torch.zeros((S, cap), dtype=torch.float32, device="cuda")
    vit.vit_attn_probe_scores(K, torch.from_numpy(q).cuda(), Hq, [L] * S, scores, decay=0.9)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    for s in seqs:
        keys = np.stack([synth.kv_rows(cfg, "k", 0, s, h, 0, L) for h in range(H)])
        mass = probe.cell_mass(q[s], keys, kc, SCALE, ks)
        _check_scores(got[s], np.zeros(cap, np.float32), mass, 0.9, L, f"{c['name']} seq {s}")
    del K
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_probe_batched_workload():
    _run_probe_workload("batched", [0, 5])


@pytest.mark.gpu
def test_probe_rotated_workload():
    _run_probe_workload("rotated", [0])


# ------------------------------------------------------------------ select
def _select(torch, vit, scores_np, lens, ns, nr, ne):
    rows, n = vit.vit_probe_select_evictions(torch.from_numpy(scores_np).cuda(), lens, ns, nr, ne)
    torch.cuda.synchronize()
    return rows.cpu().numpy(), n.cpu().numpy()


@pytest.mark.gpu
def test_select_evictions_matches_oracle():
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(41)
    cap = 2048
    for trial in range(12):
        S = int(rng.integers(1, 5))
        kind = trial % 3
        if kind == 0:
            sc = rng.integers(0, 7, (S, cap)).astype(np.float32)  # heavy ties
        elif kind == 1:
            sc = rng.standard_normal((S, cap)).astype(np.float32)  # negatives too
            sc[:, ::7] = 0.0
            sc[:, 3::7] = -0.0
        else:
            sc = rng.random((S, cap)).astype(np.float32) ** 4
        lens = [int(x) for x in rng.integers(0, cap + 1, S)]
        ns, nr = (int(x) for x in rng.integers(0, 300, 2))
        ne = int(rng.integers(0, 1500))
        say(f"[select] trial {trial} S={S} lens={lens} sink={ns} recent={nr} evict={ne}")
        rows, n = _select(torch, vit, sc, lens, ns, nr, ne)
        for s in range(S):
            ref = probe.select_evictions(sc[s].astype(np.float64), lens[s], ns, nr, ne)
            assert n[s] == len(ref), (trial, s)
            assert rows[s, :len(ref)].tolist() == ref, (trial, s)
            assert np.all(rows[s, len(ref):] == -1)


@pytest.mark.gpu
def test_select_evictions_edges_and_full_slot():
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    sc = np.zeros((2, 256), np.float32)
    rows, n = _select(torch, vit, sc, [256, 10], 8, 8, 5)
    assert n.tolist() == [5, 0] and rows[0].tolist() == [8, 9, 10, 11, 12] and rows[1].tolist() == [-1] * 5
    rows, n = _select(torch, vit, sc, [256, 256], 0, 0, 0)
    assert n.tolist() == [0, 0]
    # a 200,704-cell slot with 64 distinct score values
    rng = np.random.default_rng(43)
    cap = 200704
    sc = (rng.integers(0, 64, (2, cap)) / 64.0).astype(np.float32)
    lens = [cap, 150001]
    rows, n = _select(torch, vit, sc, lens, 4, 256, 5000)
    for s in range(2):
        ref = probe.select_evictions(sc[s].astype(np.float64), lens[s], 4, 256, 5000)
        assert n[s] == 5000 and rows[s].tolist() == ref


@pytest.mark.gpu
def test_select_evictions_ties_across_blocks():
    """Several 1024-cell blocks per sequence; the tied target key's cells span
    blocks, so each block's share of them depends on the blocks before it."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(47)
    cap = 30000
    sc = np.ones((3, cap), np.float32)                               # all equal
    sc[1] = (rng.integers(0, 3, cap) / 4.0).astype(np.float32)       # three values
    sc[2] = rng.random(cap).astype(np.float32)
    sc[2, 5000:21000:3] = 0.125                                       # a tie run across blocks
    lens = [cap, 29999, 25001]
    for ne in (1, 4095, 4097, 9000, 12000, 30000):
        rows, n = _select(torch, vit, sc, lens, 17, 5, ne)
        for s in range(3):
            ref = probe.select_evictions(sc[s].astype(np.float64), lens[s], 17, 5, ne)
            assert n[s] == len(ref), (ne, s)
            assert rows[s, :len(ref)].tolist() == ref, (ne, s)


@pytest.mark.gpu
def test_select_evictions_both_forms_at_the_threshold():
    """A longest middle range of 8192 cells takes the one-workgroup form
    (keys in LDS), 8193 the multi-block form; both must equal the oracle."""
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(53)
    cap = 8704
    sc = (rng.integers(0, 50, (2, cap)) / 16.0).astype(np.float32)  # many ties
    sc[1] = rng.standard_normal(cap).astype(np.float32)
    for lens in ([8192, 5000], [8193, 5000]):
        for ne in (1, 700, 4096, 9000):
            say(f"[select-threshold] lens={lens} evict={ne}")
            rows, n = _select(torch, vit, sc, lens, 0, 0, ne)
            for s in range(2):
                ref = probe.select_evictions(sc[s].astype(np.float64), lens[s], 0, 0, ne)
                assert n[s] == len(ref), (lens, ne, s)
                assert rows[s, :len(ref)].tolist() == ref, (lens, ne, s)
                assert np.all(rows[s, len(ref):] == -1)
