"""Shared helpers of the GPU parity tests (not a test module).

Inputs come from ``synth`` (seeded) or from seeded numpy generators; expected
values come only from ``oracle``.  The HIP path is reached only through the
C ABI (``quantized_kv_cache_append_amd``)."""

import math
import sys

import numpy as np
import pytest

import oracle
from oracle import attention, codecs

TOL = 2e-3  # max |o - ref| <= TOL * RMS(ref)


def torch_cuda():
    import torch

    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU visible")
    return torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_plane(codec, side, S, H, cap, signs=None, poison=True):
    from quantized_kv_cache_append_amd import KVPlane

    p = KVPlane(codec, side, S, H, cap, signs)
    if poison:
        for t in p.tensors():
            t.fill_(-1)  # all bits set: 0xFF codes, NaN fp16 scales / norms
    return p


def append_rows(plane, rows_host, pos0, stream=None):
    """rows_host fp32 [S, T, H, 128] -> device -> vit_kv_append_quant."""
    import torch

    from quantized_kv_cache_append_amd import vit_kv_append_quant

    src = torch.from_numpy(np.ascontiguousarray(rows_host, dtype=np.float32)).cuda()
    vit_kv_append_quant(plane, src, pos0, stream=stream)
    return src


def fill_plane_synth(plane, cfg, layer, side, start, count, units, torch, gen):
    """Rows start..start+count-1 of every (seq, head) of a workload plane:
    the seeded synth rows for the sampled units, seeded device normals
    elsewhere; then one vit_kv_append_quant call."""
    import synth
    from quantized_kv_cache_append_amd import vit_kv_append_quant

    S, H = plane.n_seqs, plane.n_kv_heads
    src = torch.randn((S, count, H, 128), generator=gen, device="cuda", dtype=torch.float32)
    for (s, h) in units:
        src[s, :, h] = torch.from_numpy(synth.kv_rows(cfg, side, layer, s, h, start, count)).cuda()
    vit_kv_append_quant(plane, src, [start] * S)
    return src


def unit_view(plane, s, h):
    """Logical contents of one (sequence, KV head) stream of a plane (the
    slice of each array that holds it), as host_view shapes them with S = H = 1."""
    from quantized_kv_cache_append_amd import layout

    cap = plane.capacity
    u = s * plane.n_kv_heads + h
    rb = plane.codes.numel() // (plane.n_seqs * plane.n_kv_heads * cap)
    out = {"codes": layout.unpack_codes(plane.codec, plane.side,
                                        plane.codes[u * cap * rb:(u + 1) * cap * rb].cpu().numpy(), 1, 1, cap)[0, 0]}
    if plane.scales is not None:
        raw = plane.scales[u * cap * 4:(u + 1) * cap * 4].cpu().numpy().view(np.uint16)
        out["scales"] = layout.unpack_scales(plane.side, raw, 1, 1, cap)[0, 0]
    if plane.norms is not None:
        out["norms"] = layout.unpack_norms(plane.norms[u * cap:(u + 1) * cap].cpu().numpy().view(np.uint16), 1, 1, cap)[0, 0]
    return out


def oracle_quant(codec, rows, signs):
    """Oracle codes of rows [N, 128] as (codes, scales, norms) arrays."""
    q = codecs.quantize(codec, rows, signs)
    return q["codes"], q.get("scales"), q.get("norms")


def compare_plane_rows(plane, view, s, h, rows_idx, rows_fp32):
    """Bit-exact comparison of rows of one (seq, head) against the oracle."""
    c, sc, nm = oracle_quant(plane.codec, rows_fp32, plane.signs)
    got = view["codes"][s, h, rows_idx]
    if plane.codec == "q8_0":
        got = got.astype(np.int8)
    bad = np.argwhere(got != c)
    assert bad.size == 0, f"{plane.codec}/{plane.side} code mismatch at rows {rows_idx[bad[:5, 0]]} ch {bad[:5, 1]}"
    if sc is not None:
        assert np.array_equal(view["scales"][s, h, rows_idx], sc), f"{plane.codec} scale mismatch"
    if nm is not None:
        assert np.array_equal(view["norms"][s, h, rows_idx], nm), f"{plane.codec} norm mismatch"


def ref_unit(q_rows, k_rows, v_rows, kc, vc, scale, ks=None, vs=None):
    return attention.decode_reference(q_rows, k_rows, v_rows, kc, vc, scale, ks, vs)


def check_close(got, ref, what, tol=TOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = math.sqrt(float(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref)))
    say(f"  {what}: max|err| / rms = {err / rms:.3e} (rms {rms:.3e})")
    assert err <= tol * rms, f"{what}: max err {err:.3e} > {tol} x rms {rms:.3e}"
    return err / rms


__all__ = ["oracle", "torch_cuda", "say", "make_plane", "append_rows", "fill_plane_synth", "unit_view", "compare_plane_rows",
           "ref_unit", "check_close", "TOL"]
