"""Host-side view of the physical plane layout (numpy only).

The kernels store each (sequence, KV head) stream as 32-row tiles whose byte
order serves coalesced MFMA operand loads (include/vit.h, "Physical layout").
These functions translate between that order and logical per-row codes
(``codes[..., row, channel]``, ``scales[..., row, block]``, ``norms[..., row]``)
so that tests and tools can read or seed planes.  They run on host copies of
the plane arrays; nothing here is on the decode path.
"""

import numpy as np

ROW_BYTES = {"f16": 256, "q8_0": 128, "q4_0": 64, "rot4": 64, "rot3": 48}
TILE = 32
D = 128


def _k_perm(codec):
    """Physical byte offset (within a tile) of each canonical row byte [32, RB].

    Unit (h, c, g, r) holds chunk g (bytes [g*CHB, (g+1)*CHB) of the block's
    canonical bytes) of each of the 4/CB blocks of unit c, in block order."""
    rb = ROW_BYTES[codec]
    cb = rb // 64
    bpu, chb = 4 // cb, 4 * cb
    p = np.arange(TILE)[:, None]
    byte = np.arange(rb)[None, :]
    b = byte // (rb // 4)
    wb = byte % (rb // 4)
    g = wb // chb
    c = b // bpu
    i = (b % bpu) * chb + wb % chb
    h = p >> 4
    r = p & 15
    return (((h * cb + c) * 4 + g) * 16 + r) * 16 + i


def _v_map(codec):
    """(byte offset, nibble shift) of code (row p, channel ch) in a V tile [32,128]."""
    p = np.arange(TILE)[:, None]
    ch = np.arange(D)[None, :]
    nt, n, g8, j = ch >> 4, ch & 15, p >> 3, p & 7
    shift = np.zeros((TILE, D), dtype=np.int64)
    if codec == "f16":
        off = ((nt * 4 + g8) * 16 + n) * 16 + 2 * j
    elif codec == "q8_0":
        p8 = (j & 4) | ((j & 1) << 1) | ((j >> 1) & 1)
        off = (((nt >> 1) * 4 + g8) * 16 + n) * 16 + 8 * (nt & 1) + p8
    else:
        base = (((nt >> 2) * 4 + g8) * 16 + n) * 16 + 4 * (nt & 3)
        if codec == "q4_0":
            off = base + (((j & 1) << 1) | ((j >> 1) & 1))
            shift = (j >> 2) * 4 + 0 * ch
        else:
            off = base + (j >> 1)
            shift = (j & 1) * 4 + 0 * ch
    return np.broadcast_to(off, (TILE, D)), np.broadcast_to(shift, (TILE, D))


def _rot3_bitpos(side):
    """Bit offset (within a tile) of the 3-bit code of (row p, channel ch)
    [32, 128], code bit k at offset + k (little-endian bit order)."""
    p = np.arange(TILE)[:, None]
    ch = np.arange(D)[None, :]
    if side == "k":
        # unit (h, g, r) of 12 bytes; block b's group at byte 3b, code j at bit 3j
        h, r, b, g, j = p >> 4, p & 15, ch >> 5, (ch & 31) >> 3, ch & 7
        return ((((h * 4 + g) * 16 + r) * 12 + 3 * b) * 8 + 3 * j).astype(np.int64)
    # unit (u, g8, n16) of 12 bytes; N-tile (ch >> 4) & 3 at byte 3c, row j at bit 3j
    u, g8, n16, c, j = ch >> 6, p >> 3, ch & 15, (ch >> 4) & 3, p & 7
    return (((((u * 4 + g8) * 16 + n16) * 12) + 3 * c) * 8 + 3 * j).astype(np.int64)


def _rot3_unpack(side, tiles):
    bits = np.unpackbits(tiles, axis=-1, bitorder="little")
    pos = _rot3_bitpos(side)
    c = bits[..., pos] | (bits[..., pos + 1] << 1) | (bits[..., pos + 2] << 2)
    return c.astype(np.uint8)


def _rot3_pack(side, codes_tiles, tiles):
    """codes_tiles [..., 32, 128] -> tiles [..., 32 * 48] (every bit rewritten)."""
    pos = _rot3_bitpos(side)
    bits = np.zeros(tiles.shape[:-1] + (tiles.shape[-1] * 8,), dtype=np.uint8)
    c = np.asarray(codes_tiles, dtype=np.uint8)
    for k in range(3):
        bits[..., pos + k] = (c >> k) & 1
    tiles[...] = np.packbits(bits, axis=-1, bitorder="little")


def _canon_to_codes(codec, rows):
    """Canonical row bytes [..., RB] -> logical codes [..., 128]."""
    if codec == "f16":
        return np.ascontiguousarray(rows).view(np.uint16)
    if codec == "q8_0":
        return np.ascontiguousarray(rows).view(np.int8)
    r = rows.reshape(rows.shape[:-1] + (4, 16))
    return np.concatenate([r & 15, r >> 4], axis=-1).reshape(rows.shape[:-1] + (D,))


def _codes_to_canon(codec, codes):
    if codec == "f16":
        return np.ascontiguousarray(codes, dtype=np.uint16).view(np.uint8)
    if codec == "q8_0":
        return np.ascontiguousarray(codes, dtype=np.int8).view(np.uint8)
    c = np.asarray(codes, dtype=np.uint8).reshape(codes.shape[:-1] + (4, 32))
    return (c[..., :16] | (c[..., 16:] << 4)).reshape(codes.shape[:-1] + (64,))


def unpack_codes(codec, side, raw, n_seqs, n_kv_heads, capacity):
    """Physical code bytes -> logical codes [S, H, capacity, 128]
    (uint16 fp16 bits for f16, int8 for q8_0, 0..15 for q4_0 / rot4, 0..7
    for rot3)."""
    rb = ROW_BYTES[codec]
    tiles = np.asarray(raw, dtype=np.uint8).reshape(n_seqs, n_kv_heads, capacity // TILE, TILE * rb)
    if codec == "rot3":
        return _rot3_unpack(side, tiles).reshape(n_seqs, n_kv_heads, capacity, D)
    if side == "k":
        rows = tiles[..., _k_perm(codec)].reshape(n_seqs, n_kv_heads, capacity, rb)
        return _canon_to_codes(codec, rows)
    off, shift = _v_map(codec)
    if codec == "f16":
        lo = tiles[..., off].astype(np.uint16)
        hi = tiles[..., off + 1].astype(np.uint16)
        return (lo | (hi << 8)).reshape(n_seqs, n_kv_heads, capacity, D)
    if codec == "q8_0":
        return tiles[..., off].view(np.int8).reshape(n_seqs, n_kv_heads, capacity, D)
    return ((tiles[..., off] >> shift) & 15).astype(np.uint8).reshape(n_seqs, n_kv_heads, capacity, D)


def pack_codes(codec, side, codes, raw):
    """Write logical codes [S, H, capacity, 128] into physical bytes ``raw``
    (a writable uint8 array of the plane's code size), in place."""
    codes = np.asarray(codes)
    S, H, cap, _ = codes.shape
    rb = ROW_BYTES[codec]
    tiles = raw.reshape(S, H, cap // TILE, TILE * rb)
    if codec == "rot3":
        _rot3_pack(side, codes.reshape(S, H, cap // TILE, TILE, D), tiles)
        return raw
    if side == "k":
        canon = _codes_to_canon(codec, codes).reshape(S, H, cap // TILE, TILE, rb)
        tiles[..., _k_perm(codec)] = canon
        return raw
    off, shift = _v_map(codec)
    c = codes.reshape(S, H, cap // TILE, TILE, D)
    if codec == "f16":
        c16 = c.astype(np.uint16)
        tiles[..., off] = (c16 & 0xFF).astype(np.uint8)
        tiles[..., off + 1] = (c16 >> 8).astype(np.uint8)
    elif codec == "q8_0":
        tiles[..., off] = c.astype(np.int8).view(np.uint8)
    else:
        # two codes share a byte: build each byte from its two nibbles
        t = np.zeros_like(tiles)
        np.add.at(t, (Ellipsis, off), (c.astype(np.uint8) & 15) << shift.astype(np.uint8))
        tiles[...] = t
    return raw


def unpack_scales(side, raw, n_seqs, n_kv_heads, capacity):
    """fp16 scale bits -> [S, H, capacity, 4].  K side: stored [S][H][cap][4];
    V side: stored [S][H][cap/32][4][32]."""
    s = np.asarray(raw, dtype=np.uint16)
    if side == "k":
        return s.reshape(n_seqs, n_kv_heads, capacity, 4)
    s = s.reshape(n_seqs, n_kv_heads, capacity // TILE, 4, TILE)
    return np.ascontiguousarray(s.transpose(0, 1, 2, 4, 3)).reshape(n_seqs, n_kv_heads, capacity, 4)


def pack_scales(side, scales):
    s = np.asarray(scales, dtype=np.uint16)
    S, H, cap, _ = s.shape
    if side == "k":
        return np.ascontiguousarray(s).reshape(-1)
    return np.ascontiguousarray(s.reshape(S, H, cap // TILE, TILE, 4).transpose(0, 1, 2, 4, 3)).reshape(-1)


def unpack_norms(raw, n_seqs, n_kv_heads, capacity):
    return np.asarray(raw, dtype=np.uint16).reshape(n_seqs, n_kv_heads, capacity)
