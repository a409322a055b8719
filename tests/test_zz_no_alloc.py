"""GPU check of vit_attn_decode_noalloc (the decode whose split partials live
in the library's static device scratch) against the existing entry points,
vit_attn_decode_mq + vit_attn_splitk_reduce with a caller workspace.

Two calls in a row, the second with a smaller input (fewer sequences, rows,
splits; several new tokens), then a third with one split (no scratch use).
The decode's summation order is fixed, so the two entry points must agree
bit for bit; both are also held to the oracle's bar (max |o - ref| <=
2e-3 x RMS(ref)).
"""

import math

import numpy as np
import pytest

from gpu_helpers import append_rows, check_close, make_plane, say, torch_cuda
from oracle import attention

D = 128


def _rows(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    x[..., rng.choice(D, 2, replace=False)] *= 20.0
    return x


def _case(kc, vc, S, H, G, q_len, lens, n_splits, fused, seed):
    torch = torch_cuda()
    import quantized_kv_cache_append_amd as vit

    rng = np.random.default_rng(seed)
    ks = rng.integers(0, 256, 16, dtype=np.uint8) if kc in ("rot4", "rot3") else None
    vs = rng.integers(0, 256, 16, dtype=np.uint8) if vc in ("rot4", "rot3") else None
    cap = 256 * ((max(lens) + 255) // 256)
    K = make_plane(kc, "k", S, H, cap, ks)
    V = make_plane(vc, "v", S, H, cap, vs)
    Lmax = max(lens)
    kx, vx = _rows(rng, (S, Lmax, H, D)), _rows(rng, (S, Lmax, H, D))
    Hq = H * G
    q = torch.from_numpy(_rows(rng, (S, q_len, Hq, D))).cuda()
    if fused:
        append_rows(K, kx, [0] * S)
        append_rows(V, vx, [0] * S)
        knew = torch.from_numpy(np.ascontiguousarray(np.stack([kx[s, lens[s] - q_len:lens[s]] for s in range(S)]))).cuda()
        vnew = torch.from_numpy(np.ascontiguousarray(np.stack([vx[s, lens[s] - q_len:lens[s]] for s in range(S)]))).cuda()
    else:
        append_rows(K, kx, [0] * S)
        append_rows(V, vx, [0] * S)
        knew = vnew = None
    # the existing entry points with a caller workspace
    ref_out = vit.decode(K, V, q, Hq, lens, k_new=knew, v_new=vnew, n_splits=n_splits, q_len=q_len)
    # the entry point that allocates nothing (out is the caller's)
    out = torch.full((S, q_len, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    vit.vit_attn_decode_noalloc(K, V, q, Hq, q_len, lens, out, k_new=knew, v_new=vnew, n_splits=n_splits)
    torch.cuda.synchronize()
    got, want = out.cpu().numpy(), ref_out.cpu().numpy()
    assert np.array_equal(got, want), f"noalloc differs from the workspace path: {np.max(np.abs(got - want))}"
    ref = np.zeros(got.shape, dtype=np.float64)
    qh = q.cpu().numpy()
    for s in range(S):
        for h in range(H):
            ref[s, :, h * G:(h + 1) * G] = attention.decode_multi_reference(
                qh[s, :, h * G:(h + 1) * G], kx[s, :lens[s], h], vx[s, :lens[s], h], kc, vc, 1.0 / math.sqrt(D), ks, vs)
    check_close(got, ref, f"noalloc K={kc} V={vc} S={S} G={G} q_len={q_len} splits={n_splits}")


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_path():
    # call 1: the larger input (3 x 32 rows x 8 splits of partials)
    say("[noalloc] call 1: q8_0/rot4, S 3, G 4, 8 splits, fused append")
    _case("q8_0", "rot4", 3, 2, 4, 1, [3000, 1500, 777], 8, True, seed=11)
    # call 2: smaller (2 x 16 rows x 3 splits), two new tokens, another codec pair
    say("[noalloc] call 2: f16/q4_0, S 2, G 4, q_len 2, 3 splits")
    _case("f16", "q4_0", 2, 1, 4, 2, [700, 130], 3, False, seed=12)
    # call 3: one split, the normalised output straight from the decode
    say("[noalloc] call 3: rot3/q8_0, S 1, G 8, 1 split")
    _case("rot3", "q8_0", 1, 2, 8, 1, [400], 1, True, seed=13)
