// Append: quantize new K or V rows and store them in a cache plane; and the
// VBR degrade step, which re-encodes the rows a plane holds into a plane of
// a codec with fewer bits per value.
//
// Compiled with -ffp-contract=off: the encoders' fp32 operation order is part
// of the codec formats (codes and fp16 scales are bit-exact), so no multiply
// may fuse with an add.
//
// Append's work split: one wave per (8-row group, KV head, sequence), four
// groups per workgroup.  The wave loads all of its rows first (so their
// loads are in flight together), encodes them together (each encoder step is
// issued for all rows before the next; lane l holds channels l and l + 64 of
// a row), and stores them (store_group).
#include "decode_impl.h"

namespace vit {

// K side, a whole 8-row group (not rot3): the 8 rows' canonical bytes go to
// LDS together (4-bit codecs pair their nibbles by a lane exchange first),
// one wave fence, then lane l stores unit l % (4 CB) of row l / (4 CB), so one
// 16-byte store instruction covers 4 (f16), 8 (q8_0) or all 8 (4-bit) rows.
// The 8 rows' 32 fp16 scales (K: [row][block], contiguous) go out as four
// 16-byte stores from lanes 0 and 32, the rot4 norms as one from lane 0.
template <int CODEC>
__device__ inline void store_k_group(uint8_t* tbase, uint16_t* scales, uint16_t* norms, int64_t g0, int pbase,
                                     const RowCodes (&rc)[8], int lane, uint8_t (*rowbuf)[256]) {
  // row r's canonical bytes at kb + r * KS: the padding makes the unit reads
  // of a store instruction (several rows at once) fall in distinct LDS banks
  // (4-bit: all 32 lanes of a half-wave; q8_0: at most 2 lanes per bank)
  constexpr int KS = CODEC == F16 ? 256 : (CODEC == Q8_0 ? 144 : 80);
  uint8_t* kb = &rowbuf[0][0];
  if constexpr (CODEC == Q4_0 || CODEC == ROT4) {
    // canonical byte 16b + j = code j | code j + 16 << 4 of block b: lane
    // 32h + j (j < 16) holds channel j of blocks h (c0) and 2 + h (c1), and
    // its xor-16 partner channel j + 16
    uint32_t hi0[8], hi1[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      hi0[r] = xshfl<16>(rc[r].c0);
      hi1[r] = xshfl<16>(rc[r].c1);
    }
    if ((lane & 16) == 0) {
      const int j = lane & 15, h = lane >> 5;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        kb[r * KS + 16 * h + j] = static_cast<uint8_t>((rc[r].c0 & 15u) | ((hi0[r] & 15u) << 4));
        kb[r * KS + 16 * (2 + h) + j] = static_cast<uint8_t>((rc[r].c1 & 15u) | ((hi1[r] & 15u) << 4));
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if constexpr (CODEC == F16) {
        reinterpret_cast<uint16_t*>(kb + r * KS)[lane] = static_cast<uint16_t>(rc[r].c0);
        reinterpret_cast<uint16_t*>(kb + r * KS)[lane + 64] = static_cast<uint16_t>(rc[r].c1);
      } else {
        kb[r * KS + lane] = static_cast<uint8_t>(rc[r].c0);
        kb[r * KS + lane + 64] = static_cast<uint8_t>(rc[r].c1);
      }
    }
  }
  wave_lds_fence();
  // unit (c, g): chunk g (CHB bytes) of each of the BPU blocks of unit c
  constexpr int CB = units_per_block(CODEC);
  constexpr int BPU = 4 / CB, CHB = 4 * CB, LPR = 4 * CB;  // LPR: lanes (units) per row
  constexpr int RPP = 64 / LPR;                               // rows per store instruction
#pragma unroll
  for (int r0 = 0; r0 < 8; r0 += RPP) {
    const int r = r0 + lane / LPR;
    if (r < 8) {
      const int u = lane % LPR;
      const int g = u / CB, c = u % CB;
      uint32_t w[4];
#pragma unroll
      for (int bb = 0; bb < BPU; ++bb)
#pragma unroll
        for (int k = 0; k < CHB / 4; ++k)
          w[bb * (CHB / 4) + k] =
              *reinterpret_cast<const uint32_t*>(kb + r * KS + (c * BPU + bb) * 16 * CB + g * CHB + 4 * k);
      *reinterpret_cast<u32x4*>(tbase + k_unit_offset(CODEC, pbase + r, g, c)) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
  if constexpr (has_scales(CODEC)) {
    // lane 0 holds blocks 0 and 2 of every row, lane 32 blocks 1 and 3
    uint32_t own0[8], own1[8], oth0[8], oth1[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      own0[r] = rc[r].s0;
      own1[r] = rc[r].s1;
      oth0[r] = static_cast<uint32_t>(__shfl_xor(static_cast<int>(own0[r]), 32, kWave));
      oth1[r] = static_cast<uint32_t>(__shfl_xor(static_cast<int>(own1[r]), 32, kWave));
    }
    if ((lane & 31) == 0) {
      const bool upper = lane != 0;  // lane 32: rows 4..7, and its own blocks are 1 and 3
      uint32_t row[4][2];            // [row i of this lane's four][word]: blocks (0, 1), (2, 3)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a0 = upper ? own0[4 + i] : own0[i], a1 = upper ? own1[4 + i] : own1[i];
        const uint32_t b0 = upper ? oth0[4 + i] : oth0[i], b1 = upper ? oth1[4 + i] : oth1[i];
        const uint32_t blk0 = upper ? b0 : a0, blk1 = upper ? a0 : b0;
        const uint32_t blk2 = upper ? b1 : a1, blk3 = upper ? a1 : b1;
        row[i][0] = blk0 | (blk1 << 16);
        row[i][1] = blk2 | (blk3 << 16);
      }
      u32x4* dst = reinterpret_cast<u32x4*>(scales + k_scale_index(g0 + (upper ? 4 : 0), 0));
      dst[0] = u32x4{row[0][0], row[0][1], row[1][0], row[1][1]};
      dst[1] = u32x4{row[2][0], row[2][1], row[3][0], row[3][1]};
    }
  }
  if constexpr (has_norms(CODEC)) {
    if (lane == 0) {
      uint32_t nv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) nv[r] = rc[r].norm;
      const u32x4 u = {nv[0] | (nv[1] << 16), nv[2] | (nv[3] << 16), nv[4] | (nv[5] << 16), nv[6] | (nv[7] << 16)};
      *reinterpret_cast<u32x4*>(norms + g0) = u;
    }
  }
}

// Store the encoded rows g0 .. g0+7 (one 8-row group, g0 % 8 == 0) of one
// (sequence, KV head) stream; only rows with live[r] are written.  A whole
// group goes out together: K rows through LDS (store_k_group; rot3 K rows one
// by one); on the V side a channel's 8 rows form one column unit, assembled
// in registers and written whole.  A group cut by the range edge goes row by
// row and keeps the rows outside it (read-modify-write of the shared 4-bit
// and 3-bit V words).
template <int CODEC, int SIDE>
__device__ inline void store_group(uint8_t* codes, uint16_t* scales, uint16_t* norms, int64_t g0,
                                   const RowCodes (&rc)[8], const bool (&live)[8], int lane, uint8_t (*rowbuf)[256]) {
  bool all = true;
#pragma unroll
  for (int r = 0; r < 8; ++r) all = all && live[r];
  if (!all || (SIDE == 0 && CODEC == ROT3)) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (live[r]) store_row<CODEC, SIDE>(codes, scales, norms, g0 + r, rc[r], lane, rowbuf[r]);
    return;
  }
  // the whole group is in range: write units, scales and norms whole
  const int64_t tile = g0 >> 5;
  const int pbase = static_cast<int>(g0 & 31);  // 0, 8, 16 or 24
  uint8_t* tbase = codes + tile * tile_code_bytes(CODEC);
  if constexpr (SIDE == 0) {
    store_k_group<CODEC>(tbase, scales, norms, g0, pbase, rc, lane, rowbuf);
    return;
  }
  if constexpr (CODEC == ROT3) {
    // lane l: the 24-bit groups of channels l and l + 64 over the 8 rows;
    // lane n16 < 16 writes units (u, g8, n16), channels 64u + 16c + n16
    uint32_t gv[2] = {0u, 0u};
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      gv[0] |= (rc[r].c0 & 7u) << (3 * r);
      gv[1] |= (rc[r].c1 & 7u) << (3 * r);
    }
    uint32_t g[2][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      g[0][c] = static_cast<uint32_t>(__shfl(static_cast<int>(gv[0]), 16 * c + (lane & 15), kWave));
      g[1][c] = static_cast<uint32_t>(__shfl(static_cast<int>(gv[1]), 16 * c + (lane & 15), kWave));
    }
    if (lane < 16) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint32_t w[3];
        rot3_unit_words(g[u], w);
        int bit;
        uint32_t* dst = reinterpret_cast<uint32_t*>(tbase + v3_group_offset(pbase, 64 * u + lane, &bit));
        dst[0] = w[0];
        dst[1] = w[1];
        dst[2] = w[2];
      }
    }
  } else {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int ch = lane + 64 * half;
      uint32_t c[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) c[r] = half ? rc[r].c1 : rc[r].c0;
      int sh;
      const int off0 = v_code_offset(CODEC, pbase, ch, &sh);
      if constexpr (CODEC == F16) {
        const u32x4 u = {c[0] | (c[1] << 16), c[2] | (c[3] << 16), c[4] | (c[5] << 16), c[6] | (c[7] << 16)};
        *reinterpret_cast<u32x4*>(tbase + off0) = u;
      } else if constexpr (CODEC == Q8_0) {
        // row r goes to byte P8[r] = {0,2,1,3,4,6,5,7}[r] of the 8-byte unit
        const uint32_t lo = (c[0] & 0xFFu) | ((c[2] & 0xFFu) << 8) | ((c[1] & 0xFFu) << 16) | ((c[3] & 0xFFu) << 24);
        const uint32_t hi = (c[4] & 0xFFu) | ((c[6] & 0xFFu) << 8) | ((c[5] & 0xFFu) << 16) | ((c[7] & 0xFFu) << 24);
        *reinterpret_cast<u32x2*>(tbase + off0) = u32x2{lo, hi};
      } else {
        uint32_t w = 0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int off = v_code_offset(CODEC, pbase + r, ch, &sh);
          w |= (c[r] & 0xFu) << (((off & 3) << 3) + sh);
        }
        *reinterpret_cast<uint32_t*>(tbase + (off0 & ~3)) = w;
      }
    }
  }
  if constexpr (has_scales(CODEC)) {
    // lane 0 holds blocks 0 and 2, lane 32 blocks 1 and 3 (uniform per half-wave)
    if ((lane & 31) == 0) {
      const int b0 = lane >> 5;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t sv[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) sv[r] = half ? rc[r].s1 : rc[r].s0;
        const u32x4 u = {sv[0] | (sv[1] << 16), sv[2] | (sv[3] << 16), sv[4] | (sv[5] << 16), sv[6] | (sv[7] << 16)};
        *reinterpret_cast<u32x4*>(scales + v_scale_index(tile, b0 + 2 * half, pbase)) = u;
      }
    }
  }
  if constexpr (has_norms(CODEC)) {
    if (lane == 0) {
      uint32_t nv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) nv[r] = rc[r].norm;
      const u32x4 u = {nv[0] | (nv[1] << 16), nv[2] | (nv[3] << 16), nv[4] | (nv[5] << 16), nv[6] | (nv[7] << 16)};
      *reinterpret_cast<u32x4*>(norms + g0) = u;
    }
  }
}

// One 8-row group of one (sequence, KV head) stream: load the rows, encode
// them together, store them (rows outside [p_begin, p_begin + n_tokens) are
// neither encoded into the plane nor written).
template <int CODEC, int SIDE>
__device__ __forceinline__ void append_group(void* codes_base, uint16_t* scales_base, uint16_t* norms_base,
                                             const float* src_base, int64_t capacity, const uint32_t (&signs)[4],
                                             int64_t p_begin, int n_tokens, int n_kv_heads, int seq, int head,
                                             int64_t g, int lane, uint8_t (*rowbuf)[256]) {
  const int64_t p_end = p_begin + n_tokens;
  const int64_t g_first_row = g * 8;
  if (g_first_row >= p_end) return;  // past this sequence's range (uniform per wave)

  constexpr int RB = row_code_bytes(CODEC);
  const int64_t ph = static_cast<int64_t>(seq) * n_kv_heads + head;
  uint8_t* codes = static_cast<uint8_t*>(codes_base) + ph * capacity * RB;
  uint16_t* scales = has_scales(CODEC) ? scales_base + ph * capacity * 4 : nullptr;
  uint16_t* norms = has_norms(CODEC) ? norms_base + ph * capacity : nullptr;

  bool live[8];
  float x0[8], x1[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int64_t p = g_first_row + r;
    live[r] = p >= p_begin && p < p_end;
    // rows outside the range read a row inside it (clamped) and are not stored
    const int64_t pc = p < p_begin ? p_begin : (p >= p_end ? p_end - 1 : p);
    const float* src = src_base + ((static_cast<int64_t>(seq) * n_tokens + (pc - p_begin)) * n_kv_heads + head) * kD;
    x0[r] = src[lane];
    x1[r] = src[lane + 64];
  }
  RowCodes rc[8];
  encode_rows<CODEC, 8>(x0, x1, lane, signs, rc);
  store_group<CODEC, SIDE>(codes, scales, norms, g_first_row, rc, live, lane, rowbuf);
}

template <int CODEC, int SIDE>
__global__ __launch_bounds__(64 * kAppendWaves) void append_kernel(AppendArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int head = blockIdx.y;
  const int seq = blockIdx.z;
  const int64_t p_begin = a.pos0[seq];
  // every scalar argument in one round trip (fetched where each is first
  // used, they were waited for one after another)
  __asm__ volatile("" ::"s"(p_begin), "s"(a.n_tokens), "s"(a.n_kv_heads), "s"(a.capacity), "s"(a.src), "s"(a.codes),
                   "s"(a.scales), "s"(a.norms), "s"(a.signs[0]), "s"(a.signs[1]), "s"(a.signs[2]), "s"(a.signs[3]));
  const int64_t g = (p_begin >> 3) + static_cast<int64_t>(blockIdx.x) * kAppendWaves + wave;  // 8-row group
  const uint32_t signs[4] = {a.signs[0], a.signs[1], a.signs[2], a.signs[3]};
  __shared__ uint8_t rowbuf[kAppendWaves][8][256];
  append_group<CODEC, SIDE>(a.codes, a.scales, a.norms, a.src, a.capacity, signs, p_begin, a.n_tokens, a.n_kv_heads,
                            seq, head, g, lane, rowbuf[wave]);
}

// Several planes in one launch: blockIdx.z = plane * n_seqs + sequence, and
// each workgroup runs the encoder of its plane's codec and side (uniform
// per workgroup), so the launch's fixed start cost is paid once.
__global__ __launch_bounds__(64 * kAppendWaves) void append_multi_kernel(AppendMultiArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int head = blockIdx.y;
  const int pl = static_cast<int>(blockIdx.z) / a.n_seqs;
  const int seq = static_cast<int>(blockIdx.z) - pl * a.n_seqs;
  const AppendPlane& P = a.planes[pl];
  const int64_t p_begin = a.pos0[seq];
  __asm__ volatile("" ::"s"(p_begin), "s"(a.n_tokens), "s"(a.n_kv_heads), "s"(P.capacity), "s"(P.src), "s"(P.codes),
                   "s"(P.scales), "s"(P.norms), "s"(P.codec_side), "s"(P.signs[0]), "s"(P.signs[1]),
                   "s"(P.signs[2]), "s"(P.signs[3]));  // one round trip, as in append_kernel
  const int64_t g = (p_begin >> 3) + static_cast<int64_t>(blockIdx.x) * kAppendWaves + wave;
  const uint32_t signs[4] = {P.signs[0], P.signs[1], P.signs[2], P.signs[3]};
  __shared__ uint8_t rowbuf[kAppendWaves][8][256];
#define VIT_APPEND_GROUP(C, S)                                                                                    \
  case (C)*2 + (S):                                                                                               \
    append_group<C, S>(P.codes, P.scales, P.norms, P.src, P.capacity, signs, p_begin, a.n_tokens, a.n_kv_heads,  \
                       seq, head, g, lane, rowbuf[wave]);                                                         \
    break;
  switch (P.codec_side) {
    VIT_APPEND_GROUP(F16, 0)
    VIT_APPEND_GROUP(F16, 1)
    VIT_APPEND_GROUP(Q8_0, 0)
    VIT_APPEND_GROUP(Q8_0, 1)
    VIT_APPEND_GROUP(Q4_0, 0)
    VIT_APPEND_GROUP(Q4_0, 1)
    VIT_APPEND_GROUP(ROT4, 0)
    VIT_APPEND_GROUP(ROT4, 1)
    VIT_APPEND_GROUP(ROT3, 0)
    VIT_APPEND_GROUP(ROT3, 1)
    default:
      break;
  }
#undef VIT_APPEND_GROUP
}

// Re-encode (a VBR degrade step): one workgroup per 32-row tile of one
// (sequence, KV head) stream.  The source tile (codes and scales) is staged
// in LDS with 16-byte loads; wave w then decodes rows 8w .. 8w+7 (lane l:
// channels l and l + 64) to their values, which are exact in fp32 (an fp16
// value, or an integer code times an fp16 scale), encodes them as append
// does, and stores the group.  Rows at or past n_rows are neither decoded
// nor written.
template <int SRC, int DST, int SIDE>
__global__ __launch_bounds__(64 * kAppendWaves) void transcode_kernel(TranscodeArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t tile = blockIdx.x;
  const int head = blockIdx.y;
  const int seq = blockIdx.z;
  const int64_t n = a.n_rows[seq];
  // every scalar argument in one round trip, as in append_kernel
  __asm__ volatile("" ::"s"(n), "s"(a.n_kv_heads), "s"(a.capacity), "s"(a.src_codes), "s"(a.src_scales), "s"(a.codes),
                   "s"(a.scales), "s"(a.norms), "s"(a.signs[0]), "s"(a.signs[1]), "s"(a.signs[2]), "s"(a.signs[3]));
  const int64_t row0 = tile * kTile;
  if (row0 >= n) return;  // uniform per workgroup

  const int64_t ph = static_cast<int64_t>(seq) * a.n_kv_heads + head;
  __shared__ u32x4 stile[tile_code_bytes(SRC) / 16];
  __shared__ uint16_t sscale[128];
  __shared__ uint8_t rowbuf[kAppendWaves][8][256];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.src_codes + ph * a.capacity * row_code_bytes(SRC) +
                                                      tile * tile_code_bytes(SRC));
    for (int i = tid; i < tile_code_bytes(SRC) / 16; i += 64 * kAppendWaves) stile[i] = __builtin_nontemporal_load(src + i);
    if constexpr (has_scales(SRC)) {
      // the tile's 128 scales are contiguous on both sides: K [row][block],
      // V [block][row]
      const u32x4* ssrc = reinterpret_cast<const u32x4*>(a.src_scales + ph * a.capacity * 4 + tile * 128);
      if (tid < 16) reinterpret_cast<u32x4*>(sscale)[tid] = __builtin_nontemporal_load(ssrc + tid);
    }
  }
  __syncthreads();
  const int64_t g0 = row0 + 8 * wave;
  if (g0 >= n) return;  // no live row in this wave's group (uniform per wave)

  const uint8_t* t8 = reinterpret_cast<const uint8_t*>(stile);
  bool live[8];
  float x0[8], x1[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int p = 8 * wave + r;  // row within the tile
    live[r] = row0 + p < n;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int ch = lane + 64 * half;
      float v;
      if constexpr (SRC == F16) {
        int sh;
        const int off = SIDE == 0 ? k_canon_offset(F16, p, 2 * ch) : v_code_offset(F16, p, ch, &sh);
        v = f16_to_float(*reinterpret_cast<const uint16_t*>(t8 + off));
      } else {
        const int b = ch >> 5;
        const float d = f16_to_float(sscale[SIDE == 0 ? p * 4 + b : b * 32 + p]);
        int code;
        if constexpr (SRC == Q8_0) {
          int sh;
          const int off = SIDE == 0 ? k_canon_offset(Q8_0, p, ch) : v_code_offset(Q8_0, p, ch, &sh);
          code = static_cast<int8_t>(t8[off]);
        } else {  // Q4_0: canonical byte 16b + (j & 15), high nibble for j >= 16
          int sh = ((ch & 31) >> 4) * 4;
          const int off = SIDE == 0 ? k_canon_offset(Q4_0, p, 16 * b + (ch & 15)) : v_code_offset(Q4_0, p, ch, &sh);
          code = static_cast<int>((t8[off] >> sh) & 0xFu) - 8;
        }
        v = static_cast<float>(code) * d;  // exact: <= 19 significant bits
      }
      v = live[r] ? v : 0.0f;  // rows past n_rows (any bits) are encoded as zeros and not stored
      if (half) x1[r] = v;
      else x0[r] = v;
    }
  }
  RowCodes rc[8];
  encode_rows<DST, 8>(x0, x1, lane, a.signs, rc);
  constexpr int RB = row_code_bytes(DST);
  uint8_t* codes = static_cast<uint8_t*>(a.codes) + ph * a.capacity * RB;
  uint16_t* scales = has_scales(DST) ? a.scales + ph * a.capacity * 4 : nullptr;
  uint16_t* norms = has_norms(DST) ? a.norms + ph * a.capacity : nullptr;
  store_group<DST, SIDE>(codes, scales, norms, g0, rc, live, lane, rowbuf[wave]);
}

#define VIT_APPEND_CASE(C, S)                                                   \
  case (C)*2 + (S):                                                             \
    hipExtLaunchKernelGGL((append_kernel<C, S>), grid, dim3(64 * kAppendWaves), 0, stream, ev.start, ev.stop, 0, \
                          args);                                                \
    break;

hipError_t launch_append(int codec, int side, dim3 grid, hipStream_t stream, const AppendArgs& args,
                         const KernelEvents& ev) {
  switch (codec * 2 + side) {
    VIT_APPEND_CASE(F16, 0)
    VIT_APPEND_CASE(F16, 1)
    VIT_APPEND_CASE(Q8_0, 0)
    VIT_APPEND_CASE(Q8_0, 1)
    VIT_APPEND_CASE(Q4_0, 0)
    VIT_APPEND_CASE(Q4_0, 1)
    VIT_APPEND_CASE(ROT4, 0)
    VIT_APPEND_CASE(ROT4, 1)
    VIT_APPEND_CASE(ROT3, 0)
    VIT_APPEND_CASE(ROT3, 1)
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_append_multi(dim3 grid, hipStream_t stream, const AppendMultiArgs& args, const KernelEvents& ev) {
  hipExtLaunchKernelGGL(append_multi_kernel, grid, dim3(64 * kAppendWaves), 0, stream, ev.start, ev.stop, 0, args);
  return hipGetLastError();
}

// The degrade steps: f16 -> q8_0 / q4_0 / rot4 / rot3, q8_0 -> q4_0 / rot4 /
// rot3, q4_0 -> rot3.
#define VIT_TRANSCODE_CASE(S, D)                                                                         \
  case (S)*8 + (D):                                                                                      \
    if (side == 0)                                                                                       \
      hipExtLaunchKernelGGL((transcode_kernel<S, D, 0>), grid, dim3(64 * kAppendWaves), 0, stream,      \
                            ev.start, ev.stop, 0, args);                                                 \
    else                                                                                                 \
      hipExtLaunchKernelGGL((transcode_kernel<S, D, 1>), grid, dim3(64 * kAppendWaves), 0, stream,      \
                            ev.start, ev.stop, 0, args);                                                 \
    break;

hipError_t launch_transcode(int src_codec, int dst_codec, int side, dim3 grid, hipStream_t stream,
                            const TranscodeArgs& args, const KernelEvents& ev) {
  switch (src_codec * 8 + dst_codec) {
    VIT_TRANSCODE_CASE(F16, Q8_0)
    VIT_TRANSCODE_CASE(F16, Q4_0)
    VIT_TRANSCODE_CASE(F16, ROT4)
    VIT_TRANSCODE_CASE(F16, ROT3)
    VIT_TRANSCODE_CASE(Q8_0, Q4_0)
    VIT_TRANSCODE_CASE(Q8_0, ROT4)
    VIT_TRANSCODE_CASE(Q8_0, ROT3)
    VIT_TRANSCODE_CASE(Q4_0, ROT3)
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vit
