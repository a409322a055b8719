// Device-side definitions shared by the append, decode and reduce kernels:
// vector types, codec constants, the physical plane layout and the wave-level
// encode helpers.  gfx950 only (wave64, MFMA 16x16x32 f16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vit {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Codec { F16 = 0, Q8_0 = 1, Q4_0 = 2, ROT4 = 3 };

constexpr int kD = 128;      // head_dim
constexpr int kTile = 32;    // rows per tile
constexpr int kWave = 64;

// code bytes per row and 16-byte units per 32-value block ("CB")
__host__ __device__ constexpr int row_code_bytes(int c) { return c == F16 ? 256 : (c == Q8_0 ? 128 : 64); }
__host__ __device__ constexpr int units_per_block(int c) { return row_code_bytes(c) / 64; }
__host__ __device__ constexpr int tile_code_bytes(int c) { return kTile * row_code_bytes(c); }
__host__ __device__ constexpr bool has_scales(int c) { return c != F16; }
__host__ __device__ constexpr bool has_norms(int c) { return c == ROT4; }

// ---------------------------------------------------------------------------
// The rot4 levels: the 16-level Lloyd-Max quantizer for N(0,1) (J. Max 1960),
// stored as fp16 bit patterns in increasing order, and the fp32 midpoints of
// adjacent stored levels used as decision thresholds.
__device__ constexpr uint16_t kLevelBits[16] = {
    0xc177, 0xc023, 0xbe79, 0xbd06, 0xbb8a, 0xb941, 0xb635, 0xb01c,
    0x301c, 0x3635, 0x3941, 0x3b8a, 0x3d06, 0x3e79, 0x4023, 0x4177};
__device__ constexpr float kThresholds[15] = {
    -0x1.334p+1f, -0x1.d7ep+0f, -0x1.6fep+0f, -0x1.196p+0f, -0x1.996p-1f,
    -0x1.0b7p-1f, -0x1.086p-2f, 0.0f, 0x1.086p-2f, 0x1.0b7p-1f,
    0x1.996p-1f, 0x1.196p+0f, 0x1.6fep+0f, 0x1.d7ep+0f, 0x1.334p+1f};

// ---------------------------------------------------------------------------
// Physical layout (see include/vit.h).  Offsets are within one 32-row tile.

// K side: row p of the tile, block b, 16-byte unit c of that block's bytes.
// Rows 16h .. 16h+15 form half h; lane 16b + r of a wave-wide 16-byte load of
// (half h, unit c) reads row 16h + r, block b.
__host__ __device__ inline int k_unit_offset(int codec, int p, int b, int c) {
  const int h = p >> 4;
  const int r = p & 15;
  const int cb = units_per_block(codec);
  return (((h * cb + c) * 4 + b) * 16 + r) * 16;
}

// V side: byte offset of the code of (row p, channel ch) and, for 4-bit
// codecs, the nibble shift (0 or 4).  F16 codes take 2 bytes at the offset.
__host__ __device__ inline int v_code_offset(int codec, int p, int ch, int* shift) {
  const int nt = ch >> 4, n = ch & 15, g8 = p >> 3, j = p & 7;
  *shift = 0;
  if (codec == F16) return ((nt * 4 + g8) * 16 + n) * 16 + 2 * j;
  if (codec == Q8_0) {
    const int p8 = (j & 4) | ((j & 1) << 1) | ((j >> 1) & 1);  // {0,2,1,3,4,6,5,7}
    return (((nt >> 1) * 4 + g8) * 16 + n) * 16 + 8 * (nt & 1) + p8;
  }
  const int base = (((nt >> 2) * 4 + g8) * 16 + n) * 16 + 4 * (nt & 3);
  if (codec == Q4_0) {
    *shift = (j >> 2) * 4;
    return base + (((j & 1) << 1) | ((j >> 1) & 1));  // {0,2,1,3,0,2,1,3}
  }
  *shift = (j & 1) * 4;  // ROT4
  return base + (j >> 1);
}

// scales of one stream: K side in row order [row][block]; V side
// block-major inside each tile [tile][block][32].
__host__ __device__ inline int64_t k_scale_index(int64_t row, int b) { return row * 4 + b; }
__host__ __device__ inline int64_t v_scale_index(int64_t tile, int b, int p) { return tile * 128 + b * 32 + p; }

// ---------------------------------------------------------------------------
// Scalar helpers (encode side: every operation is one IEEE binary32 rounding).

__device__ inline uint16_t f16_bits(float x) {
  const _Float16 h = static_cast<_Float16>(x);  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ inline float f16_to_float(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// Correctly rounded fp32 square root of a finite x >= 0.  The hardware
// square root is within one ulp; the result is moved to a neighbour when the
// exact residual x - y*y' (one fma, whose sign is exact) shows the true root
// lies past the midpoint between the two.  Tiny inputs are scaled by 2^64
// (exact) so that the hardware sees a normal number.
__device__ inline float sqrt_rn(float x) {
  if (x == 0.0f) return x;
  const bool tiny = x < 0x1p-100f;
  const float xs = tiny ? x * 0x1p+64f : x;
  float y = __builtin_amdgcn_sqrtf(xs);
  const float ydn = __uint_as_float(__float_as_uint(y) - 1u);
  const float yup = __uint_as_float(__float_as_uint(y) + 1u);
  const float rdn = __builtin_fmaf(-ydn, y, xs);
  const float rup = __builtin_fmaf(-yup, y, xs);
  if (rdn <= 0.0f) y = ydn;
  else if (rup > 0.0f) y = yup;
  return tiny ? y * 0x1p-32f : y;
}

__device__ inline float recip_or_zero(float d) { return d != 0.0f ? 1.0f / d : 0.0f; }

template <typename T>
__device__ inline T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, kWave);
}

// ---------------------------------------------------------------------------
// Wave-level row encoders.  Lane l holds channels l (x0) and l + 64 (x1).
// Every encoder body disables fp contraction: the operation order of the
// codec definitions is part of the format, whatever flags the including
// translation unit uses.
// Blocks: x0 is in block l>>5, x1 in block 2 + (l>>5); the 32 lanes of a
// half-wave hold one block, so block reductions are xor-shuffles 16..1.

struct RowCodes {
  uint32_t c0, c1;     // codes of channels l and l+64 (fp16 bits, int8 as uint8, nibble)
  uint16_t s0, s1;     // fp16 scales of the blocks of x0 and x1
  uint16_t norm;       // rot4 row norm
};

__device__ inline float block_max_abs(float v) {
  float a = fabsf(v);
  for (int m = 16; m >= 1; m >>= 1) a = fmaxf(a, shfl_xor(a, m));
  return a;
}

__device__ inline RowCodes encode_f16(float x0, float x1) {
#pragma clang fp contract(off)
  RowCodes r{};
  r.c0 = f16_bits(x0);
  r.c1 = f16_bits(x1);
  return r;
}

__device__ inline int8_t q8_code(float x, float inv) {
#pragma clang fp contract(off)
  float c = roundf(x * inv);  // round half away from zero
  c = fminf(fmaxf(c, -127.0f), 127.0f);
  return static_cast<int8_t>(c);
}

__device__ inline RowCodes encode_q8_0(float x0, float x1) {
#pragma clang fp contract(off)
  RowCodes r{};
  const float d0 = block_max_abs(x0) / 127.0f;
  const float d1 = block_max_abs(x1) / 127.0f;
  const float i0 = recip_or_zero(d0), i1 = recip_or_zero(d1);
  r.c0 = static_cast<uint8_t>(q8_code(x0, i0));
  r.c1 = static_cast<uint8_t>(q8_code(x1, i1));
  r.s0 = f16_bits(d0);
  r.s1 = f16_bits(d1);
  return r;
}

// q4_0 block scale from the first element of largest magnitude.
__device__ inline float q4_block_scale(float x, int lane) {
#pragma clang fp contract(off)
  // key: |x| bits (monotone for non-negative floats) high, inverted index low,
  // so the max picks the largest magnitude and, among equals, the first index.
  const uint32_t j = static_cast<uint32_t>(lane & 31);
  uint64_t key = (static_cast<uint64_t>(__float_as_uint(fabsf(x))) << 32) | (31u - j);
  for (int m = 16; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor(key, m);
    key = o > key ? o : key;
  }
  const uint32_t amax_bits = static_cast<uint32_t>(key >> 32);
  const int src = (lane & 32) | static_cast<int>(31u - static_cast<uint32_t>(key & 0xffffffffu));
  const float m = __shfl(x, src, kWave);
  return amax_bits == 0u ? 0.0f : m / -8.0f;
}

__device__ inline uint32_t q4_code(float x, float inv) {
#pragma clang fp contract(off)
  float c = roundf(x * inv) + 8.0f;
  c = fminf(fmaxf(c, 0.0f), 15.0f);
  return static_cast<uint32_t>(c);
}

__device__ inline RowCodes encode_q4_0(float x0, float x1, int lane) {
#pragma clang fp contract(off)
  RowCodes r{};
  const float d0 = q4_block_scale(x0, lane);
  const float d1 = q4_block_scale(x1, lane);
  r.c0 = q4_code(x0, recip_or_zero(d0));
  r.c1 = q4_code(x1, recip_or_zero(d1));
  r.s0 = f16_bits(d0);
  r.s1 = f16_bits(d1);
  return r;
}

__device__ inline uint32_t rot4_index(float t) {
  uint32_t idx = 0;
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    const float th = kThresholds[k];
    idx += (t > th) ? 1u : 0u;
    idx += (t == th && t >= 0.0f) ? 1u : 0u;
  }
  return idx;
}

// signs: the 128-bit mask as 4 words; bit j set => channel j negated.
__device__ inline RowCodes encode_rot4(float x0, float x1, int lane, const uint32_t signs[4]) {
#pragma clang fp contract(off)
  RowCodes r{};
  const int ch0 = lane, ch1 = lane + 64;
  float w0 = ((signs[ch0 >> 5] >> (ch0 & 31)) & 1u) ? -x0 : x0;
  float w1 = ((signs[ch1 >> 5] >> (ch1 & 31)) & 1u) ? -x1 : x1;
  // Walsh-Hadamard stages h = 1..32 across lanes, then h = 64 inside the lane.
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const float p0 = shfl_xor(w0, h);
    const float p1 = shfl_xor(w1, h);
    if (lane & h) {
      w0 = p0 - w0;
      w1 = p1 - w1;
    } else {
      w0 = w0 + p0;
      w1 = w1 + p1;
    }
  }
  {
    const float a = w0 + w1, b = w0 - w1;
    w0 = a;
    w1 = b;
  }
  // row norm: stride-halving tree of the squares of the input row
  const float sq0 = x0 * x0;
  const float sq1 = x1 * x1;
  float ss = sq0 + sq1;
  for (int m = 32; m >= 1; m >>= 1) ss = ss + shfl_xor(ss, m);
  const float n = sqrt_rn(ss);
  r.norm = f16_bits(n);
  const float g = n > 0.0f ? 1.0f / n : 0.0f;
  const float u0 = w0 * g;
  const float u1 = w1 * g;
  // per-block RMS of the whitened values
  const float uu0 = u0 * u0;
  const float uu1 = u1 * u1;
  float b0 = uu0, b1 = uu1;
  for (int m = 16; m >= 1; m >>= 1) {
    b0 = b0 + shfl_xor(b0, m);
    b1 = b1 + shfl_xor(b1, m);
  }
  const float r0 = sqrt_rn(b0 * 0.03125f);
  const float r1 = sqrt_rn(b1 * 0.03125f);
  r.s0 = f16_bits(r0);
  r.s1 = f16_bits(r1);
  const float ib0 = r0 > 0.0f ? 1.0f / r0 : 0.0f;
  const float ib1 = r1 > 0.0f ? 1.0f / r1 : 0.0f;
  r.c0 = rot4_index(u0 * ib0);
  r.c1 = rot4_index(u1 * ib1);
  return r;
}

template <int CODEC>
__device__ inline RowCodes encode_row(float x0, float x1, int lane, const uint32_t signs[4]) {
  if constexpr (CODEC == F16) return encode_f16(x0, x1);
  else if constexpr (CODEC == Q8_0) return encode_q8_0(x0, x1);
  else if constexpr (CODEC == Q4_0) return encode_q4_0(x0, x1, lane);
  else return encode_rot4(x0, x1, lane, signs);
}

}  // namespace vit
