"""KV byte accounting: bits/value per codec, bytes per row, per-token sizes.

Closed forms that the pages print and that this model must reproduce:
* bits/value: f16 16, q8_0 8.5, q4_0 4.5, turbo4 4.125, turbo8 8.125
  (buun-llama-cpp page, "Codecs" table);
* tq3_0 at 3.5 bits is "~22% smaller than q4_0" (Randozart/VITRIOL page,
  "What sets VITRIOL apart" table); rot3 is that 3.5 bits/value class;
* VBR aggregate bits/value 15.75 then 15.51 for the first two degrade steps
  and 160 / 600 steps for 16 / 60 attention layers (buun-llama-cpp page,
  "VBR -- Variable Bit-Rate KV Cache");
* K f16 + V q8_0 costs 24.5 KiB/token where f16/f16 costs 32; 3 x 262,144
  tokens need 18.4 GiB and 49,152 tokens 1,176 MiB (serverAppConfigs commit
  log, tests/frank_small_unit.bats page).
"""

BLOCK = 32
HEAD_DIM = 128

# bits per value of each codec (codes + per-block scale + per-row norm)
BPV = {
    "f16": 16.0,
    "q8_0": 8.0 + 16.0 / BLOCK,                     # 8.5
    "q4_0": 4.0 + 16.0 / BLOCK,                     # 4.5
    "rot4": 4.0 + 16.0 / BLOCK + 16.0 / HEAD_DIM,   # 4.625: scale per 32 + norm per row
    "rot3": 3.0 + 16.0 / BLOCK,                     # 3.5: scale per 32, no norm
    # rotated codecs of the pages' ladder that carry one fp16 norm per 128 values
    "turbo8": 8.0 + 16.0 / HEAD_DIM,                # 8.125
    "turbo4": 4.0 + 16.0 / HEAD_DIM,                # 4.125
    "tq3_0": 3.5,
}

# the degrade ladder named on the buun-llama-cpp page (f16 plus five rungs)
VBR_LADDER = ("f16", "turbo8", "turbo4", "turbo3_tcq", "turbo2_tcq", "turbo1_tcq")


def row_bytes(codec, head_dim=HEAD_DIM):
    """Bytes of one (token, head) row: codes + scales (+ norm)."""
    return int(round(BPV[codec] * head_dim / 8))


def plane_bytes(codec, n_seqs, n_kv_heads, capacity, head_dim=HEAD_DIM):
    return n_seqs * n_kv_heads * capacity * row_bytes(codec, head_dim)


def kv_bytes_per_token(codec_map, n_kv_heads, head_dim=HEAD_DIM):
    """Bytes per token over all layers for a per-(layer, side) codec map
    [(k_codec, v_codec), ...]."""
    return sum(n_kv_heads * (row_bytes(k, head_dim) + row_bytes(v, head_dim)) for k, v in codec_map)


def aggregate_bpv(tensor_codecs):
    """Mean bits/value over equally sized (layer, side) tensors."""
    return sum(BPV[c] for c in tensor_codecs) / len(tensor_codecs)


def vbr_steps(n_attn_layers, n_rungs=len(VBR_LADDER) - 1):
    """One degrade step moves one (layer, side) tensor down one rung."""
    return n_attn_layers * 2 * n_rungs


def decode_kv_read_bytes(k_codec, v_codec, n_seqs, n_kv_heads, attended_len, head_dim=HEAD_DIM):
    """Algorithmic KV bytes one decode step must read: every attended row of
    every (sequence, KV head) once, K and V, codes + scales + norms."""
    return n_seqs * n_kv_heads * attended_len * (row_bytes(k_codec, head_dim) + row_bytes(v_codec, head_dim))
