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

enum Codec { F16 = 0, Q8_0 = 1, Q4_0 = 2, ROT4 = 3, ROT3 = 4 };

constexpr int kD = 128;      // head_dim
constexpr int kTile = 32;    // rows per tile
constexpr int kWave = 64;

// code bytes per row and 16-byte units per 32-value block ("CB"; rot3 rows
// of 48 bytes use 12-byte units instead, see below)
__host__ __device__ constexpr int row_code_bytes(int c) {
  return c == F16 ? 256 : (c == Q8_0 ? 128 : (c == ROT3 ? 48 : 64));
}
__host__ __device__ constexpr int units_per_block(int c) { return c == ROT3 ? 1 : row_code_bytes(c) / 64; }
__host__ __device__ constexpr int tile_code_bytes(int c) { return kTile * row_code_bytes(c); }
__host__ __device__ constexpr bool has_scales(int c) { return c != F16; }
__host__ __device__ constexpr bool has_norms(int c) { return c == ROT4; }
// codes in the Walsh-Hadamard-rotated domain (queries rotate with the keys,
// outputs rotate back)
__host__ __device__ constexpr bool rotated(int c) { return c == ROT4 || c == ROT3; }

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

// The rot3 levels: the 8-level Lloyd-Max quantizer for N(0,1) (Max 1960) as
// fp16 bit patterns, increasing, and the fp32 midpoints of adjacent levels.
__device__ constexpr uint16_t kLevelBits3[8] = {0xc04e, 0xbd60, 0xba0c, 0xb3d8, 0x33d8, 0x3a0c, 0x3d60, 0x404e};
__device__ constexpr float kThresholds3[7] = {-0x1.bf8p+0f, -0x1.0ccp+0f, -0x1.004p-1f, 0.0f,
                                              0x1.004p-1f,  0x1.0ccp+0f,  0x1.bf8p+0f};

// ---------------------------------------------------------------------------
// Physical layout (see include/vit.h).  Offsets are within one 32-row tile.

// K side: row p of the tile, chunk g (0..3) of unit c.  A row's canonical
// bytes (codes in channel order; 4-bit codes packed as in q4_0) are cut into
// blocks of 16 * CB bytes (CB = units_per_block) and each block into four
// chunks of 4 * CB bytes; unit c of the row holds chunk g of its blocks
// c * BPU .. c * BPU + BPU - 1 (BPU = 4 / CB), 16 bytes.  Rows 16h .. 16h+15
// form half h; lane 16g + r of a wave-wide 16-byte load of (half h, unit c)
// reads row 16h + r, chunk g.
__host__ __device__ inline int k_unit_offset(int codec, int p, int g, int c) {
  const int h = p >> 4;
  const int r = p & 15;
  const int cb = units_per_block(codec);
  return (((h * cb + c) * 4 + g) * 16 + r) * 16;
}

// K side: tile offset of canonical byte k of row p.
__host__ __device__ inline int k_canon_offset(int codec, int p, int k) {
  const int cb = units_per_block(codec), bpu = 4 / cb, chb = 4 * cb;
  const int blk = k / (16 * cb), off = k % (16 * cb);
  return k_unit_offset(codec, p, off / chb, blk / bpu) + (blk % bpu) * chb + off % chb;
}

// rot3 K side: the 12-byte unit of (row p, chunk g): 24-bit groups of blocks
// 0..3 at bytes 3b; group (b, g) holds channels 32b + 8g + j (j < 8), code j
// at bits 3j.  Rows 16h .. 16h+15 form half h; lane 16g + r of a wave-wide
// 12-byte load of half h reads row 16h + r, chunk g.
__host__ __device__ inline int k3_unit_offset(int p, int g) {
  return (((p >> 4) * 4 + g) * 16 + (p & 15)) * 12;
}

// rot3 V side: the 12-byte unit (u, 8-row group g8, n16) holds the 24-bit
// groups of channels 64u + 16c + n16 (c < 4) at bytes 3c, the code of row
// 8 g8 + j at bits 3j.  Lane 16 g8 + n16 of a wave-wide 12-byte load u reads
// unit (u, g8, n16).  Returns the group's byte offset; *bit = 3j.
__host__ __device__ inline int v3_group_offset(int p, int ch, int* bit) {
  *bit = 3 * (p & 7);
  return (((ch >> 6) * 4 + (p >> 3)) * 16 + (ch & 15)) * 12 + 3 * ((ch >> 4) & 3);
}

// V side: byte offset of the code of (row p, channel ch) and, for 4-bit
// codecs, the nibble shift (0 or 4).  F16 codes take 2 bytes at the offset.
// (rot3: v3_group_offset.)
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

// Exchange with lane l ^ M.  Within 16-lane rows the moves are DPP (1, 2:
// quad permutes; 8: a row rotation by 8, which is the xor-8 pairing);
// 4 and 16 use ds_swizzle's xor mode (inside 32-lane groups); 32 uses
// ds_bpermute.  Pure data movement: the encoders' arithmetic is unchanged.
template <int M>
__device__ inline uint32_t xshfl(uint32_t v) {
  if constexpr (M == 1) return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, true);
  else if constexpr (M == 2) return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, true);
  else if constexpr (M == 8) return __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xF, 0xF, true);
  else if constexpr (M == 4) return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x101F));
  else if constexpr (M == 16) return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x401F));
  else return static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), M, kWave));
}
template <int M>
__device__ inline float xshfl(float v) {
  return __uint_as_float(xshfl<M>(__float_as_uint(v)));
}

// ---------------------------------------------------------------------------
// Wave-level row encoders, R rows at a time (each step is issued for every
// row before the next step, so the rows' lane exchanges overlap).  Lane l
// holds channels l (x0) and l + 64 (x1) of each row.  Every encoder body
// disables fp contraction: the operation order of the codec definitions is
// part of the format, whatever flags the including translation unit uses.
// Blocks: x0 is in block l>>5, x1 in block 2 + (l>>5); the 32 lanes of a
// half-wave hold one block, so block reductions are xor exchanges 16..1.

struct RowCodes {
  uint32_t c0, c1;     // codes of channels l and l+64 (fp16 bits, int8 as uint8, nibble)
  uint16_t s0, s1;     // fp16 scales of the blocks of x0 and x1
  uint16_t norm;       // rot4 row norm
};

template <int M, int N>
__device__ inline void sum_step(float (&a)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] = a[i] + xshfl<M>(a[i]);
}

// Maxima of non-negative floats as unsigned integers: for x, y >= +0 the
// bit patterns order like the values, so max(bits) is the bits of the float
// maximum (the encoders' inputs are finite).  The float form would first
// quiet each exchanged operand (an extra max per value in IEEE mode), and the
// integer max takes the lane exchange as a DPP operand.
template <int M, int N>
__device__ inline void umax_step(uint32_t (&a)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t o = xshfl<M>(a[i]);
    a[i] = a[i] > o ? a[i] : o;
  }
}
template <int N>
__device__ inline void half_wave_umax(uint32_t (&a)[N]) {
  umax_step<16>(a);
  umax_step<8>(a);
  umax_step<4>(a);
  umax_step<2>(a);
  umax_step<1>(a);
}

// |x| maxima of the blocks: a[i] <- max over the lane's 32-lane half-wave
template <int N>
__device__ inline void block_max_abs(float (&a)[N]) {
  uint32_t u[N];
#pragma unroll
  for (int i = 0; i < N; ++i) u[i] = __float_as_uint(a[i]) & 0x7FFFFFFFu;  // |x|
  half_wave_umax(u);
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] = __uint_as_float(u[i]);
}

// Per lane: b where lane bit set in `mask` (a constant lane pattern), else a.
__device__ inline float lane_select(uint64_t mask, float a, float b) {
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(mask));
  return r;
}

// N block quantities v[i] that every lane of a half-wave holds (the same
// value on all 32 lanes, e.g. after a block reduction) mapped through f once
// per slot instead of on every lane: lane i (and i + 16) of each half-wave
// evaluates slot i, and ds_bpermute hands both results back to every lane.
// f(v, a, b) writes two results; for other slot counts than 8 and 16 the
// direct per-lane evaluation is used.  The arithmetic of f is unchanged,
// only where it runs.  (A full-wave quantity, the same on all 64 lanes,
// works too.)
template <int N, class F>
__device__ inline void per_slot(const float (&v)[N], int lane, F f, float (&a)[N], float (&b)[N]) {
  if constexpr (N != 8 && N != 16) {
#pragma unroll
    for (int i = 0; i < N; ++i) f(v[i], a[i], b[i]);
  } else {
    // v[lane % N] by a binary tree of selects on the bits of lane % N
    // (explicit v_cndmask with constant lane masks: written as ?:, the
    // selects become a lane-indexed stack array in scratch memory)
    constexpr uint64_t kBit[4] = {0xAAAAAAAAAAAAAAAAull, 0xCCCCCCCCCCCCCCCCull, 0xF0F0F0F0F0F0F0F0ull,
                                  0xFF00FF00FF00FF00ull};
    float t[N];
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = v[i];
#pragma unroll
    for (int level = 0, n = N; n > 1; ++level, n >>= 1)
#pragma unroll
      for (int i = 0; i < n / 2; ++i) t[i] = lane_select(kBit[level], t[2 * i], t[2 * i + 1]);
    float A, B;
    f(t[0], A, B);
    const int base = lane & 32;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      a[i] = __shfl(A, base | i, kWave);
      b[i] = __shfl(B, base | i, kWave);
    }
  }
}

template <int R>
__device__ inline void encode_f16(const float (&x0)[R], const float (&x1)[R], RowCodes (&rc)[R]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rc[r] = RowCodes{};
    rc[r].c0 = f16_bits(x0[r]);
    rc[r].c1 = f16_bits(x1[r]);
  }
}

__device__ inline int8_t q8_code(float x, float inv) {
#pragma clang fp contract(off)
  float c = roundf(x * inv);  // round half away from zero
  c = fminf(fmaxf(c, -127.0f), 127.0f);
  return static_cast<int8_t>(c);
}

template <int R>
__device__ inline void encode_q8_0(const float (&x0)[R], const float (&x1)[R], int lane, RowCodes (&rc)[R]) {
#pragma clang fp contract(off)
  float m[2 * R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[2 * r] = x0[r];
    m[2 * r + 1] = x1[r];
  }
  block_max_abs(m);
  // d = amax / 127 and 1/d once per (row, block); the fp16 bits of d travel
  // as a float
  float sb[2 * R], inv[2 * R];
  per_slot(m, lane, [](float amax, float& bits, float& iv) {
#pragma clang fp contract(off)
    const float d = amax / 127.0f;
    bits = __uint_as_float(f16_bits(d));
    iv = recip_or_zero(d);
  }, sb, inv);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rc[r] = RowCodes{};
    rc[r].c0 = static_cast<uint8_t>(q8_code(x0[r], inv[2 * r]));
    rc[r].c1 = static_cast<uint8_t>(q8_code(x1[r], inv[2 * r + 1]));
    rc[r].s0 = static_cast<uint16_t>(__float_as_uint(sb[2 * r]));
    rc[r].s1 = static_cast<uint16_t>(__float_as_uint(sb[2 * r + 1]));
  }
}

// q4_0: the signed value m of the first element of largest magnitude in
// each block (channel order = lane order within the half-wave): the block
// max |x|, then a ballot of the lanes holding it and the first of them.
template <int N>
__device__ inline void q4_block_signed_max(const float (&x)[N], int lane, float (&m)[N]) {
  uint32_t a[N], mx[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    a[i] = __float_as_uint(x[i]) & 0x7FFFFFFFu;  // |x| as bits
    mx[i] = a[i];
  }
  half_wave_umax(mx);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint64_t eq = __builtin_amdgcn_ballot_w64(a[i] == mx[i]);
    // a half-wave's mask is never 0: its maximum is one of its values
    const uint32_t half = lane < 32 ? static_cast<uint32_t>(eq) : static_cast<uint32_t>(eq >> 32);
    m[i] = __shfl(x[i], (lane & 32) | static_cast<int>(__builtin_ctz(half)), kWave);
  }
}

__device__ inline uint32_t q4_code(float x, float inv) {
#pragma clang fp contract(off)
  float c = roundf(x * inv) + 8.0f;
  c = fminf(fmaxf(c, 0.0f), 15.0f);
  return static_cast<uint32_t>(c);
}

template <int R>
__device__ inline void encode_q4_0(const float (&x0)[R], const float (&x1)[R], int lane, RowCodes (&rc)[R]) {
#pragma clang fp contract(off)
  float x[2 * R], m[2 * R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    x[2 * r] = x0[r];
    x[2 * r + 1] = x1[r];
  }
  q4_block_signed_max(x, lane, m);
  // d = m / -8 (+0 for a zero block, where m is +-0) and 1/d once per
  // (row, block); the fp16 bits of d travel as a float
  float sb[2 * R], inv[2 * R];
  per_slot(m, lane, [](float mm, float& bits, float& iv) {
#pragma clang fp contract(off)
    const float d = mm == 0.0f ? 0.0f : mm / -8.0f;
    bits = __uint_as_float(f16_bits(d));
    iv = recip_or_zero(d);
  }, sb, inv);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rc[r] = RowCodes{};
    rc[r].c0 = q4_code(x0[r], inv[2 * r]);
    rc[r].c1 = q4_code(x1[r], inv[2 * r + 1]);
    rc[r].s0 = static_cast<uint16_t>(__float_as_uint(sb[2 * r]));
    rc[r].s1 = static_cast<uint16_t>(__float_as_uint(sb[2 * r + 1]));
  }
}

// idx = #{k : th_k < t} + #{k : th_k == t and t >= 0} (a tie goes to the
// level farther from zero).  The thresholds are symmetric (th_k = -th_{14-k},
// th_7 = 0), so with c = #{k >= 8 : th_k <= |t|} this is 8 + c for t >= 0
// (-0 included) and 7 - c for t < 0.
__device__ inline uint32_t rot4_index(float t) {
  const float a = fabsf(t);
  uint32_t c = 0;
#pragma unroll
  for (int k = 8; k < 15; ++k) c += kThresholds[k] <= a ? 1u : 0u;
  return t >= 0.0f ? 8u + c : 7u - c;
}

// One Walsh-Hadamard stage across lanes for every row: lanes with bit h set
// take (partner - own), the others (own + partner), both written as
// partner + (+-own): x - y and x + (-y) are the same IEEE operation, signed
// zeros included, and the sum takes the lane exchange as a DPP operand.
template <int H, int R>
__device__ inline void wht_stage(float (&w0)[R], float (&w1)[R], int lane) {
#pragma clang fp contract(off)
  const uint32_t neg = (lane & H) != 0 ? 0x80000000u : 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    w0[r] = xshfl<H>(w0[r]) + __uint_as_float(__float_as_uint(w0[r]) ^ neg);
    w1[r] = xshfl<H>(w1[r]) + __uint_as_float(__float_as_uint(w1[r]) ^ neg);
  }
}

// A block's RMS r = sqrt(sum * (1/32)) as fp16 bits and its reciprocal
// (0 for r == 0), the per-block step of rot4 and rot3.
__device__ inline void block_rms(float sum, float& bits, float& ib) {
#pragma clang fp contract(off)
  const float r = sqrt_rn(sum * 0.03125f);
  bits = __uint_as_float(f16_bits(r));
  ib = r > 0.0f ? 1.0f / r : 0.0f;
}

// Sign flip and unnormalised Walsh-Hadamard transform of R rows: w = H (s . x).
// signs: the 128-bit mask as 4 words; bit j set => channel j negated.
template <int R>
__device__ inline void rotate_rows(const float (&x0)[R], const float (&x1)[R], int lane, const uint32_t signs[4],
                                   float (&w0)[R], float (&w1)[R]) {
#pragma clang fp contract(off)
  const int ch0 = lane, ch1 = lane + 64;
  const bool neg0 = ((signs[ch0 >> 5] >> (ch0 & 31)) & 1u) != 0;
  const bool neg1 = ((signs[ch1 >> 5] >> (ch1 & 31)) & 1u) != 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    w0[r] = neg0 ? -x0[r] : x0[r];
    w1[r] = neg1 ? -x1[r] : x1[r];
  }
  // Walsh-Hadamard stages h = 1..32 across lanes, then h = 64 inside the lane.
  wht_stage<1>(w0, w1, lane);
  wht_stage<2>(w0, w1, lane);
  wht_stage<4>(w0, w1, lane);
  wht_stage<8>(w0, w1, lane);
  wht_stage<16>(w0, w1, lane);
  wht_stage<32>(w0, w1, lane);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float a = w0[r] + w1[r], b = w0[r] - w1[r];
    w0[r] = a;
    w1[r] = b;
  }
}

template <int R>
__device__ inline void encode_rot4(const float (&x0)[R], const float (&x1)[R], int lane, const uint32_t signs[4],
                                   RowCodes (&rc)[R]) {
#pragma clang fp contract(off)
  float w0[R], w1[R];
  rotate_rows(x0, x1, lane, signs, w0, w1);
  // row norm: stride-halving tree of the squares of the input row
  float ss[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float sq0 = x0[r] * x0[r];
    const float sq1 = x1[r] * x1[r];
    ss[r] = sq0 + sq1;
  }
  sum_step<32>(ss);
  sum_step<16>(ss);
  sum_step<8>(ss);
  sum_step<4>(ss);
  sum_step<2>(ss);
  sum_step<1>(ss);
  // n = ||x||, its fp16 bits and g = 1/n once per row
  float nb[R], gr[R];
  per_slot(ss, lane, [](float s2, float& bits, float& g) {
#pragma clang fp contract(off)
    const float n = sqrt_rn(s2);
    bits = __uint_as_float(f16_bits(n));
    g = n > 0.0f ? 1.0f / n : 0.0f;
  }, nb, gr);
  float u[2 * R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rc[r] = RowCodes{};
    rc[r].norm = static_cast<uint16_t>(__float_as_uint(nb[r]));
    u[2 * r] = w0[r] * gr[r];
    u[2 * r + 1] = w1[r] * gr[r];
  }
  // per-block RMS of the whitened values
  float b[2 * R];
#pragma unroll
  for (int i = 0; i < 2 * R; ++i) b[i] = u[i] * u[i];
  sum_step<16>(b);
  sum_step<8>(b);
  sum_step<4>(b);
  sum_step<2>(b);
  sum_step<1>(b);
  float sb[2 * R], ib[2 * R];
  per_slot(b, lane, block_rms, sb, ib);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rc[r].s0 = static_cast<uint16_t>(__float_as_uint(sb[2 * r]));
    rc[r].s1 = static_cast<uint16_t>(__float_as_uint(sb[2 * r + 1]));
    rc[r].c0 = rot4_index(u[2 * r] * ib[2 * r]);
    rc[r].c1 = rot4_index(u[2 * r + 1] * ib[2 * r + 1]);
  }
}

// The rot3 index: #{k : th_k < t} + #{k : th_k == t and t >= 0} over the 7
// symmetric thresholds (th_3 = 0), i.e. 4 + #{k >= 4 : th_k <= |t|} for
// t >= 0 (-0 included) and 3 minus that count for t < 0.
__device__ inline uint32_t rot3_index(float t) {
  const float a = fabsf(t);
  uint32_t c = 0;
#pragma unroll
  for (int k = 4; k < 7; ++k) c += kThresholds3[k] <= a ? 1u : 0u;
  return t >= 0.0f ? 4u + c : 3u - c;
}

// rot3: rotate, then per block the RMS of the rotated values is the fp16
// scale and t = w / RMS picks one of 8 levels (no row norm).
template <int R>
__device__ inline void encode_rot3(const float (&x0)[R], const float (&x1)[R], int lane, const uint32_t signs[4],
                                   RowCodes (&rc)[R]) {
#pragma clang fp contract(off)
  float w0[R], w1[R];
  rotate_rows(x0, x1, lane, signs, w0, w1);
  float b[2 * R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    b[2 * r] = w0[r] * w0[r];
    b[2 * r + 1] = w1[r] * w1[r];
  }
  sum_step<16>(b);
  sum_step<8>(b);
  sum_step<4>(b);
  sum_step<2>(b);
  sum_step<1>(b);
  float sb[2 * R], ib[2 * R];
  per_slot(b, lane, block_rms, sb, ib);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rc[r] = RowCodes{};
    rc[r].s0 = static_cast<uint16_t>(__float_as_uint(sb[2 * r]));
    rc[r].s1 = static_cast<uint16_t>(__float_as_uint(sb[2 * r + 1]));
    rc[r].c0 = rot3_index(w0[r] * ib[2 * r]);
    rc[r].c1 = rot3_index(w1[r] * ib[2 * r + 1]);
  }
}

template <int CODEC, int R>
__device__ inline void encode_rows(const float (&x0)[R], const float (&x1)[R], int lane, const uint32_t signs[4],
                                   RowCodes (&rc)[R]) {
  if constexpr (CODEC == F16) encode_f16(x0, x1, rc);
  else if constexpr (CODEC == Q8_0) encode_q8_0(x0, x1, lane, rc);
  else if constexpr (CODEC == Q4_0) encode_q4_0(x0, x1, lane, rc);
  else if constexpr (CODEC == ROT4) encode_rot4(x0, x1, lane, signs, rc);
  else encode_rot3(x0, x1, lane, signs, rc);
}

// In-place unnormalised WHT of n_rows rows of 128 floats in LDS (16-byte
// aligned), by every thread of a workgroup of NTHREADS: stages h = 1, 2,
// ..., 64 in that order, each pair (i, i + h) becoming (x + y, x - y).
// Stages 1..8 run in registers on 16 consecutive channels per thread, then
// stages 16..64 on 8 channels 16 apart: two barriers instead of one per stage,
// with the same operations in the same order.
template <int NTHREADS>
__device__ inline void wht128_lds(float* rows, int n_rows, int tid) {
  for (int u = tid; u < n_rows * 8; u += NTHREADS) {  // (row, 16-channel group)
    float4v* p = reinterpret_cast<float4v*>(rows + (u >> 3) * 128 + (u & 7) * 16);
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4v w = p[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * q + j] = w[j];
    }
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (!(i & h)) {
          const float x = v[i], y = v[i + h];
          v[i] = x + y;
          v[i + h] = x - y;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = float4v{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
  }
  __syncthreads();
  for (int u = tid; u < n_rows * 16; u += NTHREADS) {  // (row, channel within the groups)
    float* p = rows + (u >> 4) * 128 + (u & 15);
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = p[16 * k];
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (!(k & h)) {
          const float x = v[k], y = v[k + h];
          v[k] = x + y;
          v[k + h] = x - y;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) p[16 * k] = v[k];
  }
  __syncthreads();
}

template <int CODEC>
__device__ inline RowCodes encode_row(float x0, float x1, int lane, const uint32_t signs[4]) {
  const float a[1] = {x0}, b[1] = {x1};
  RowCodes rc[1];
  encode_rows<CODEC, 1>(a, b, lane, signs, rc);
  return rc[0];
}

}  // namespace vit
