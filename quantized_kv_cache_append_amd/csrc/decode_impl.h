// Flash-decode attention over a quantized KV plane pair, for gfx950.
//
// One workgroup of 8 waves per (split, KV head, sequence), the only one on
// its compute unit.  Split s owns the 32-row tiles s, s + n_splits, ...;
// wave w of the workgroup takes every 8th of them, starting at the w-th,
// handles all query rows of the KV head, keeps its own online softmax state
// and prefetches its next tiles into registers while it computes the current
// one.  The waves are merged through LDS at the end, in a fixed order, so
// the result is bitwise repeatable.
//
// Both products run on MFMA 16x16x32 f16 with exact operands:
//   * K and V codes are exact in fp16 (f16 values, int8 / 4-bit integers,
//     fp16 rot4 levels), and every per-block scale is applied in fp32;
//   * the query and the probabilities are split into fp16 hi + lo parts,
//     so operand rounding stays near 2^-21 relative.
// MFMA m's B operand in S^T = Q K^T is block m of 16 K rows (lane group q,
// lanes 16q..16q+15, holds its 8-channel chunk q); each output lane gets,
// for one cached row, per-block partial dot products, which it scales by
// the fp32 block scales and sums in registers.  P is regrouped through a
// small per-wave LDS buffer into the P.V operand, where the V block scale
// folds into P per block.  Three row layouts share this scheme, by the
// number of query rows per KV head (G, or G * q_len for several new tokens):
//   <= 4 rows: (query row, block) rows, zero outside their block's MFMA,
//              hi and lo in separate MFMAs;
//   <= 8 rows: (query, hi/lo part) rows, one MFMA per block;
//   <= 16 rows: query rows, hi and lo in two chained MFMAs.
#pragma once

#include "merge.h"
#include "vit_device.h"
#include "vit_launch.h"

namespace vit {

__device__ inline float4v mfma16(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// --- exact fp16 conversions of packed codes ---------------------------------
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
__device__ inline half2v h2_bits(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// (x & mask) | bits in one v_and_or_b32 (gfx9 VOP3 takes no literal, so the
// mask comes in a VGPR and the constant bits in an SGPR).
__device__ inline uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
  uint32_t r;
  __asm__("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(mask), "s"(bits));
  return r;
}
__device__ inline uint32_t bits_h2(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// a times the fp16 in half HI of w, in fp32: one v_fma_mix_f32 (exact
// product, one rounding, the same value as converting the fp16 first).
template <int HI>
__device__ inline float mul_f16(float a, uint32_t w) {
  float r;
  if constexpr (HI) __asm__("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(w));
  else __asm__("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(w));
  return r;
}

// eight int8 codes (two words) -> fp16, element order (b0, b2, b1, b3) of each
// word.  v_perm_b32 builds the fp16 bit patterns 0x64 | (c ^ 0x80), i.e. the
// values 1024 + c + 128, and one packed subtract of 1152 per pair is exact:
// per four codes one xor, two perms, two subtracts.  (Keeping the 1152 in the
// operand and removing it after the product is not exact enough: the MFMA's
// f16 accumulation then loses the low bits of the code terms.)
__device__ inline half8 q8_unpack(uint32_t w0, uint32_t w1) {
  const uint32_t a = w0 ^ 0x80808080u, b = w1 ^ 0x80808080u;
  const half2v k = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  u32x4 r;
  r[0] = bits_h2(h2_bits(__builtin_amdgcn_perm(0x64646464u, a, 0x04020400u)) - k);  // bytes 0, 2
  r[1] = bits_h2(h2_bits(__builtin_amdgcn_perm(0x64646464u, a, 0x04030401u)) - k);  // bytes 1, 3
  r[2] = bits_h2(h2_bits(__builtin_amdgcn_perm(0x64646464u, b, 0x04020400u)) - k);
  r[3] = bits_h2(h2_bits(__builtin_amdgcn_perm(0x64646464u, b, 0x04030401u)) - k);
  return __builtin_bit_cast(half8, r);
}

// eight 4-bit codes (offset 8) -> fp16 pairs, element order
// (lo b0, lo b2, lo b1, lo b3, hi b0, hi b2, hi b1, hi b3).
__device__ inline half8 q4_unpack(uint32_t w) {
  const half2v k_lo = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
  const half2v s_hi = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
  const half2v k_hi = {static_cast<_Float16>(-72.0f), static_cast<_Float16>(-72.0f)};
  const uint32_t w8 = w >> 8;
  const half2v a = h2_bits(and_or(w, 0x000F000Fu, 0x64006400u)) - k_lo;
  const half2v b = h2_bits(and_or(w8, 0x000F000Fu, 0x64006400u)) - k_lo;
  const half2v c = h2_bits(and_or(w, 0x00F000F0u, 0x64006400u)) * s_hi + k_hi;
  const half2v d = h2_bits(and_or(w8, 0x00F000F0u, 0x64006400u)) * s_hi + k_hi;
  half8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// rot4 level table in LDS: byte b of packed indices -> the fp16 pair
// (level[b & 15], level[b >> 4]).  It is replicated once per lane (entry b of
// lane l at word 64 b + l), so the 64 lookups of one instruction always fall
// in distinct banks however the code bytes are distributed.
struct Lut {
  const uint32_t* words;   // rot4: 256 * 64 words
  const uint32_t* words3;  // rot3: 64 * 64 words
  uint32_t lane4;          // 4 * lane: the lane's byte offset within an entry
};

// Fill the lane-replicated table (entry b = level pair (b & 15, b >> 4) of
// lane l at word 64 b + l) with NTHREADS threads, a multiple of 256; lv is
// kLevelBits[lane & 15], loaded early by the caller.  Word 4 (tid + NTHREADS
// i) + j (j < 4) is entry e = (tid + NTHREADS i) / 16 of lane 4 (tid % 16) + j:
// low level (tid / 16) % 16, high level tid / 256 + (NTHREADS / 256) i, the
// same for the whole wave.
template <int NTHREADS>
__device__ inline void fill_rot4_lut(uint32_t* lut, int tid, uint32_t lv) {
  static_assert(NTHREADS % 256 == 0 && NTHREADS <= 4096, "table fill: whole 256-thread groups");
  const uint32_t lo = static_cast<uint32_t>(__shfl(static_cast<int>(lv), (tid >> 4) & 15));
  const int hb = __builtin_amdgcn_readfirstlane(tid >> 8);
#pragma unroll
  for (int i = 0; i < 4096 / NTHREADS; ++i) {
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lv), hb + (NTHREADS / 256) * i));
    const uint32_t e = lo | (hi << 16);
    *reinterpret_cast<u32x4*>(&lut[4 * (tid + NTHREADS * i)]) = u32x4{e, e, e, e};
  }
}

// The rot3 table: entry e (6 bits) = level pair (e & 7, e >> 3) of lane l at
// word 64 e + l, filled with NTHREADS threads (a multiple of 128); lv3 is
// kLevelBits3[lane & 7].  Word 4 (tid + NTHREADS i) + j is entry
// (tid + NTHREADS i) / 16: low level (tid / 16) % 8, high level
// tid / 128 + (NTHREADS / 128) i, the same for the whole wave.
template <int NTHREADS>
__device__ inline void fill_rot3_lut(uint32_t* lut3, int tid, uint32_t lv3) {
  static_assert(NTHREADS % 128 == 0 && NTHREADS <= 1024, "table fill: whole 128-thread groups");
  const uint32_t lo = static_cast<uint32_t>(__shfl(static_cast<int>(lv3), (tid >> 4) & 7));
  const int hb = __builtin_amdgcn_readfirstlane(tid >> 7);
#pragma unroll
  for (int i = 0; i < 1024 / NTHREADS; ++i) {
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lv3), hb + (NTHREADS / 128) * i));
    const uint32_t e = lo | (hi << 16);
    *reinterpret_cast<u32x4*>(&lut3[4 * (tid + NTHREADS * i)]) = u32x4{e, e, e, e};
  }
}

// eight rot3 indices (a 24-bit group, code j at bits 3j) -> fp16 levels in
// order j: four 6-bit fields, each one lookup at 256 * field + 4 * lane.
__device__ inline half8 rot3_unpack(uint32_t g, const Lut& lut) {
  const char* base = reinterpret_cast<const char*>(lut.words3);
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p)
    r[p] = *reinterpret_cast<const uint32_t*>(base + ((__builtin_amdgcn_ubfe(g, 6 * p, 6) << 8) | lut.lane4));
  return __builtin_bit_cast(half8, r);
}

// 24-bit group i (< 4) of a 12-byte rot3 unit held in u[0..2]
__device__ inline uint32_t rot3_group(const u32x4& u, int i) {
  return i == 0 ? u[0] : i == 1 ? __builtin_amdgcn_alignbit(u[1], u[0], 24)
                       : i == 2 ? __builtin_amdgcn_alignbit(u[2], u[1], 16) : u[2] >> 8;
}

// eight rot4 indices -> fp16 levels, element order (lo b0, hi b0, lo b1,
// hi b1, ...).  One v_perm_b32 per byte builds its table address
// 256 * byte + 4 * lane.
__device__ inline half8 rot4_unpack(uint32_t w, const Lut& lut) {
  const char* base = reinterpret_cast<const char*>(lut.words);
  u32x4 r;
  r[0] = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(w, lut.lane4, 0x0C0C0400u));
  r[1] = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(w, lut.lane4, 0x0C0C0500u));
  r[2] = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(w, lut.lane4, 0x0C0C0600u));
  r[3] = *reinterpret_cast<const uint32_t*>(base + __builtin_amdgcn_perm(w, lut.lane4, 0x0C0C0700u));
  return __builtin_bit_cast(half8, r);
}

// Channel (within the row) of element j of the K operand of MFMA m in lane
// group g: MFMA m covers block m, lane group g its chunk g (8 channels).
template <int KC>
__device__ inline int k_chan(int g, int m, int j) {
  if constexpr (KC == F16) {
    return 32 * m + 8 * g + j;
  } else if constexpr (KC == Q8_0) {
    const int p8 = (j & 4) | ((j & 1) << 1) | ((j >> 1) & 1);
    return 32 * m + 8 * g + p8;
  } else if constexpr (KC == Q4_0) {
    const int byte = ((j & 1) << 1) | ((j >> 1) & 1);
    return 32 * m + 4 * g + byte + ((j >> 2) << 4);
  } else if constexpr (KC == ROT4) {
    return 32 * m + 4 * g + (j >> 1) + ((j & 1) << 4);
  } else {  // ROT3: chunk g of block m is channels 32m + 8g .. 32m + 8g + 7
    return 32 * m + 8 * g + j;
  }
}

template <int KC>
__device__ inline half8 unpack_k(const u32x4* units, int m, const Lut& lut) {
  if constexpr (KC == F16) {
    return __builtin_bit_cast(half8, units[m]);
  } else if constexpr (KC == Q8_0) {
    const u32x4 u = units[m >> 1];
    return (m & 1) ? q8_unpack(u[2], u[3]) : q8_unpack(u[0], u[1]);
  } else if constexpr (KC == Q4_0) {
    return q4_unpack(units[0][m]);
  } else if constexpr (KC == ROT4) {
    return rot4_unpack(units[0][m], lut);
  } else {
    return rot3_unpack(rot3_group(units[0], m), lut);
  }
}

// V operand of N-tile nt (channels 16nt..16nt+15): element j = row 8q + j.
template <int VC>
__device__ inline half8 unpack_v(const u32x4* vd, int nt, const Lut& lut) {
  if constexpr (VC == F16) {
    return __builtin_bit_cast(half8, vd[nt]);
  } else if constexpr (VC == Q8_0) {
    const u32x4 u = vd[nt >> 1];
    return (nt & 1) ? q8_unpack(u[2], u[3]) : q8_unpack(u[0], u[1]);
  } else if constexpr (VC == Q4_0) {
    return q4_unpack(vd[nt >> 2][nt & 3]);
  } else if constexpr (VC == ROT4) {
    return rot4_unpack(vd[nt >> 2][nt & 3], lut);
  } else {  // ROT3: 12-byte unit nt / 4, group nt % 4
    return rot3_unpack(rot3_group(vd[nt >> 2], nt & 3), lut);
  }
}

// one 12-byte rot3 unit (4-byte aligned) into components 0..2; nothing past
// it is read
__device__ inline u32x4 load_unit12(const uint8_t* p) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
  return u32x4{__builtin_nontemporal_load(w), __builtin_nontemporal_load(w + 1), __builtin_nontemporal_load(w + 2), 0u};
}

template <int C>
constexpr int v_loads() {
  return C == F16 ? 8 : (C == Q8_0 ? 4 : 2);
}

// DPP moves within 16-lane rows: quad_perm [1,0,3,2], [2,3,0,1], row_ror 4, 8.
template <int CTRL>
__device__ inline float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ inline float row16_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x124>(v));
  return fmaxf(v, dpp<0x128>(v));
}
__device__ inline float row16_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x124>(v);
  return v + dpp<0x128>(v);
}

// x + nb * (fp16 in half HI of w), in fp32, one rounding: one v_fma_mix_f32
// (the fp16 operand is converted exactly).
template <int HI>
__device__ inline float fma_f16(uint32_t w, float nb, float x) {
  float r;
  if constexpr (HI) __asm__("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(nb), "v"(x));
  else __asm__("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(nb), "v"(x));
  return r;
}

// Part of the hi/lo fp16 split of a pair (x0, x1): nb = 0 gives the hi part
// fp16(x) toward zero, nb = -1 the lo part fp16(x - hi) (x - hi is exact).
// Four operations per pair: two conversions and two v_fma_mix_f32.
__device__ inline uint32_t split_part(float x0, float x1, float nb) {
  const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x0, x1));
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(fma_f16<0>(hi, nb, x0), fma_f16<1>(hi, nb, x1)));
}

// hi + lo fp16 split of two fp32 values: hi = fp16(x) toward zero (so x - hi
// is exact in fp32), lo = fp16(x - hi); |x - hi - lo| <= 2^-21 |x| + 2^-25.
__device__ inline void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x0, x1));
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(fma_f16<0>(hi, -1.0f, x0), fma_f16<1>(hi, -1.0f, x1)));
}
__device__ inline void split8(const float v[8], half8& hi, half8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t hh, ll;
    split_pair(v[2 * i], v[2 * i + 1], hh, ll);
    h[i] = hh;
    l[i] = ll;
  }
  hi = __builtin_bit_cast(half8, h);
  lo = __builtin_bit_cast(half8, l);
}

// LDS traffic that stays inside one wave (written and read back by lanes of
// the same wave) needs ordering, not a workgroup barrier.
__device__ inline void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Registers of one 32-row tile for one lane.  The cache is streamed once per
// call, so every tile load is a nontemporal (streaming) load.
template <int KC, int VC, int NT>
struct TileRegs {
  u32x4 kd[2][units_per_block(KC)];  // K units of halves 0 and 1
  u32x4 vd[v_loads<VC>()];           // V column units
  u32x2 ks[2];                       // K scales of this lane's row in each half
  uint32_t kn[2];                    // K norms (rot4)
  u32x4 vs[NT >= 2 ? 4 : 1];         // V scales, rows 8q .. 8q+7: block (lane & 3)
                                     // for 4 query rows per wave, blocks 0..3 for 8 or 16
  u32x4 vn;                          // V norms (rot4), rows 8q .. 8q+7
};

template <int KC, int VC, int NT>
__device__ inline void load_tile(TileRegs<KC, VC, NT>& r, int t, int lane, const uint8_t* kbase,
                                 const uint8_t* vbase, const uint16_t* ksb, const uint16_t* knb,
                                 const uint16_t* vsb, const uint16_t* vnb) {
  constexpr int KCB = units_per_block(KC);
  const uint8_t* kt = kbase + static_cast<int64_t>(t) * tile_code_bytes(KC);
  const uint8_t* vt = vbase + static_cast<int64_t>(t) * tile_code_bytes(VC);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (KC == ROT3) {
      r.kd[h][0] = load_unit12(kt + (h * 64 + lane) * 12);
    } else {
#pragma unroll
      for (int c = 0; c < KCB; ++c)
        r.kd[h][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kt + ((h * KCB + c) * 64 + lane) * 16));
    }
  }
#pragma unroll
  for (int i = 0; i < v_loads<VC>(); ++i) {
    if constexpr (VC == ROT3) r.vd[i] = load_unit12(vt + (i * 64 + lane) * 12);
    else r.vd[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vt + (i * 64 + lane) * 16));
  }
  const int n16 = lane & 15, qg = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(t) * kTile;
  if constexpr (has_scales(KC)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      r.ks[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(ksb + (row0 + 16 * h + n16) * 4));
  }
  if constexpr (has_norms(KC)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) r.kn[h] = __builtin_nontemporal_load(knb + row0 + 16 * h + n16);
  }
  if constexpr (has_scales(VC)) {
#pragma unroll
    for (int b = 0; b < (NT >= 2 ? 4 : 1); ++b)
      r.vs[b] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(vsb + row0 * 4 + (NT >= 2 ? b : (lane & 3)) * 32 + 8 * qg));
  }
  if constexpr (has_norms(VC)) r.vn = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vnb + row0 + 8 * qg));
}

// Tiles kept in flight ahead of the one being used: two for the 4-bit pairs
// with 4 query rows per wave (a tile is ~4.6 KB); one when a tile already
// carries >= 6 KB per wave or when 8 query rows leave no registers for more.
template <int KC, int VC, int NT>
constexpr int prefetch_depth() {
  return (NT == 1 && tile_code_bytes(KC) + tile_code_bytes(VC) <= 4096) ? 2 : 1;
}

// rot3: the 24-bit group of 8 consecutive lanes' 3-bit codes (lane 8k + j
// contributes code j at bits 3j); every lane of the 8 gets the group.
__device__ inline uint32_t rot3_group8(uint32_t code, int lane) {
  uint32_t v = (code & 7u) << (3 * (lane & 7));
  v |= xshfl<1>(v);
  v |= xshfl<2>(v);
  v |= xshfl<4>(v);
  return v;
}

// rot3: three dwords of a 12-byte unit from its four 24-bit groups
__device__ inline void rot3_unit_words(const uint32_t (&g)[4], uint32_t (&w)[3]) {
  w[0] = g[0] | (g[1] << 24);
  w[1] = (g[1] >> 8) | (g[2] << 16);
  w[2] = (g[2] >> 16) | (g[3] << 8);
}

// Store one encoded row p of a (sequence, KV head) stream from a single wave:
// scales, norm and codes (K: canonical bytes staged in `rowbuf`, 256 bytes of
// LDS private to the wave, then 16-byte units; V: the row's code in each
// channel's column unit, a read-modify-write for the 4-bit codecs).
template <int C, int SIDE>
__device__ inline void store_row(uint8_t* codes, uint16_t* scales, uint16_t* norms, int64_t p,
                                 const RowCodes& rc, int lane, uint8_t* rowbuf) {
  const int64_t tile = p >> 5;
  const int pt = static_cast<int>(p & 31);
  if constexpr (has_scales(C)) {
    if ((lane & 31) == 0) {
      const int b0 = lane >> 5;
      if constexpr (SIDE == 0) {
        scales[k_scale_index(p, b0)] = rc.s0;
        scales[k_scale_index(p, 2 + b0)] = rc.s1;
      } else {
        scales[v_scale_index(tile, b0, pt)] = rc.s0;
        scales[v_scale_index(tile, 2 + b0, pt)] = rc.s1;
      }
    }
  }
  if constexpr (has_norms(C)) {
    if (lane == 0) norms[p] = rc.norm;
  }
  uint8_t* tbase = codes + tile * tile_code_bytes(C);
  if constexpr (C == ROT3) {
    if constexpr (SIDE == 0) {
      // channel groups of 8: lane l holds channels l (blocks 0, 1) and l + 64
      // (blocks 2, 3); lanes 8k .. 8k+7 form group k of each half.  Unit
      // (p, g): blocks 0..3 of chunk g = groups of lanes 8g (c0, c1) and
      // 8g + 32 (c0, c1)
      const uint32_t g0 = rot3_group8(rc.c0, lane);
      const uint32_t g1 = rot3_group8(rc.c1, lane);
      const uint32_t h0 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(g0), 32, kWave));
      const uint32_t h1 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(g1), 32, kWave));
      if (lane < 32 && (lane & 7) == 0) {
        const uint32_t g[4] = {g0, h0, g1, h1};
        uint32_t w[3];
        rot3_unit_words(g, w);
        uint32_t* dst = reinterpret_cast<uint32_t*>(tbase + k3_unit_offset(pt, lane >> 3));
        dst[0] = w[0];
        dst[1] = w[1];
        dst[2] = w[2];
      }
    } else {
      // one lane per unit (u, pt / 8, n16) rewrites row pt's four fields:
      // channels 64u + 16c + n16, c < 4 (several channels share its words)
      uint32_t cc[2][4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        cc[0][c] = static_cast<uint32_t>(__shfl(static_cast<int>(rc.c0), 16 * c + (lane & 15), kWave));
        cc[1][c] = static_cast<uint32_t>(__shfl(static_cast<int>(rc.c1), 16 * c + (lane & 15), kWave));
      }
      if (lane < 16) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          int bit;
          const int off = v3_group_offset(pt, 64 * u + lane, &bit);  // group c = 0 of the unit
          uint32_t* wp = reinterpret_cast<uint32_t*>(tbase + off);
          uint32_t d[3] = {wp[0], wp[1], wp[2]};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int P = 24 * c + bit;  // bit position in the 96-bit unit
            const int lo = P >> 5, sh = P & 31;
            const uint32_t v = cc[u][c] & 7u;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
              if (k == lo) d[k] = (d[k] & ~(7u << sh)) | (v << sh);
              if (k == lo + 1 && sh > 29) d[k] = (d[k] & ~(7u >> (32 - sh))) | (v >> (32 - sh));
            }
          }
          wp[0] = d[0];
          wp[1] = d[1];
          wp[2] = d[2];
        }
      }
    }
    return;
  }
  if constexpr (SIDE == 0) {
    // canonical row bytes in LDS, then 16-byte units to their tile slots
    if constexpr (C == F16) {
      reinterpret_cast<uint16_t*>(rowbuf)[lane] = static_cast<uint16_t>(rc.c0);
      reinterpret_cast<uint16_t*>(rowbuf)[lane + 64] = static_cast<uint16_t>(rc.c1);
    } else if constexpr (C == Q8_0) {
      rowbuf[lane] = static_cast<uint8_t>(rc.c0);
      rowbuf[lane + 64] = static_cast<uint8_t>(rc.c1);
    } else {
      rowbuf[128 + lane] = static_cast<uint8_t>(rc.c0);
      rowbuf[192 + lane] = static_cast<uint8_t>(rc.c1);
      wave_lds_fence();
      const int b = lane >> 4, j = lane & 15;
      rowbuf[lane] = static_cast<uint8_t>(rowbuf[128 + 32 * b + j] | (rowbuf[128 + 32 * b + j + 16] << 4));
    }
    wave_lds_fence();
    // unit (c, g): chunk g (CHB bytes) of each of the BPU blocks of unit c
    constexpr int CB = units_per_block(C);
    constexpr int BPU = 4 / CB, CHB = 4 * CB;
    if (lane < 4 * CB) {
      const int g = lane / CB, c = lane % CB;
      uint32_t w[4];
#pragma unroll
      for (int bb = 0; bb < BPU; ++bb)
#pragma unroll
        for (int k = 0; k < CHB / 4; ++k)
          w[bb * (CHB / 4) + k] =
              *reinterpret_cast<const uint32_t*>(rowbuf + (c * BPU + bb) * 16 * CB + g * CHB + 4 * k);
      *reinterpret_cast<u32x4*>(tbase + k_unit_offset(C, pt, g, c)) = u32x4{w[0], w[1], w[2], w[3]};
    }
  } else {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int ch = lane + 64 * half;
      const uint32_t code = half ? rc.c1 : rc.c0;
      int sh;
      const int off = v_code_offset(C, pt, ch, &sh);
      if constexpr (C == F16) {
        *reinterpret_cast<uint16_t*>(tbase + off) = static_cast<uint16_t>(code);
      } else if constexpr (C == Q8_0) {
        tbase[off] = static_cast<uint8_t>(code);
      } else {
        // the channel's 8 rows share one aligned word; only this row changes
        uint32_t* wp = reinterpret_cast<uint32_t*>(tbase + (off & ~3));
        const int bit = ((off & 3) << 3) + sh;
        *wp = (*wp & ~(0xFu << bit)) | ((code & 0xFu) << bit);
      }
    }
  }
}

// Quantize one new row and store it (the fused append of the decode call).
template <int C, int SIDE>
__device__ inline void append_one_row(uint8_t* codes, uint16_t* scales, uint16_t* norms, int64_t p,
                                      const float* src, int lane, const uint32_t signs[4], uint8_t* rowbuf) {
  const RowCodes rc = encode_row<C>(src[lane], src[lane + 64], lane, signs);
  store_row<C, SIDE>(codes, scales, norms, p, rc, lane, rowbuf);
}

// Per-wave online-softmax state for 4*NT query rows.
template <int NT>
struct WaveState {
  float m_run[NT];        // running max (base 2) of the lane's query row
  float l_run[NT];        // lane-partial running sum
  float4v oacc[8];        // P.V accumulators of N-tile c: rows (query row, block)
                          // for 4 query rows, (query row, hi/lo part) for 8
  // The softmax reference is m_run + vexp: p = 2^(s - m_run - vexp), so the
  // P.V operand p * f (f = V block factor) carries 2^-vexp and stays in the
  // fp16 normal range whatever the magnitude of V.  vexp (an integer, wave
  // wide) is re-chosen when a tile's largest |f| leaves
  // [2^(vexp-12), 2^(vexp+4)]; l and O share the reference, so O / l and the
  // split merge are unaffected.
  float vexp;
  float vlo, vhi;         // that window as thresholds on |f|
};

// Largest |f| of the wave (every lane gets it).
__device__ inline float wave_max(float v) {
  v = row16_max(v);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Q operands of S^T, in registers: rows (query row, block) with separate hi
// and lo operands for 4 query rows per wave; rows (query, hi/lo part) for 8;
// query rows with separate hi and lo operands for 16.
template <int NT>
struct QOperands {
  half8 h[NT][4], l[NT][4];
};
template <>
struct QOperands<2> {
  half8 w[4];  // MFMA b: row n16 = 2 q + part of query q, chunk qg of block b
};
template <>
struct QOperands<4> {
  // MFMA b: row n16 = query n16, chunk qg of block b, fp16 hi and lo parts.
  // They are the same in every wave, so they live in LDS (one copy per
  // workgroup, 8 KB) and are read per tile: held in registers they pushed
  // the 16-row kernels past 256 VGPRs.  ops[(part * 4 + b) * 64 + lane].
  const half8* ops;
};

// K factors of the lane's tile row 16h + n16 for blocks 0..3: the fp16 block
// scale (rot4: times the row norm); 1 for f16 planes.
template <int KC, class Regs>
__device__ __forceinline__ void k_block_factors(const Regs& cur, float (&kf)[2][4]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kf[h][i] = 1.0f;
    if constexpr (KC != F16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[h][i] = f16_to_float(cur.ks[h][i >> 1] >> ((i & 1) * 16));
      if constexpr (KC == ROT4) {
        const float nrm = f16_to_float(cur.kn[h]);
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[h][i] *= nrm;
      }
    }
  }
}

// One 32-row tile for one wave with 4 query rows: S^T = Q K^T, online
// softmax, O += P V.
//   L:    rows of the stream that hold data (the last query row's length);
//   lmin: the shortest query row's length; lim: this lane's query row length.
template <int KC, int VC, int NT>
__device__ __forceinline__ void process_tile(const TileRegs<KC, VC, NT>& cur, int t, int L, int lmin,
                                             const int (&lim)[NT], int lane, const QOperands<NT>& aq,
                                             WaveState<NT>& st, float (*s_p)[4][kTile], const Lut& lut) {
  static_assert(NT == 1, "4 query rows per wave");
  const int n16 = lane & 15, qg = lane >> 4;
  const bool partial = (t + 1) * kTile > lmin;
  // ---- V block factors of the lane's P.V operand rows (block n16 & 3, tile
  //      rows 8qg .. 8qg+7) and the wave's V exponent check, first so that
  //      they overlap the S^T products ----
  float vf[8];
  float vexp_new = st.vexp;
  bool v_rescale = false;
  if constexpr (VC != F16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float f = f16_to_float(cur.vs[0][j >> 1] >> ((j & 1) * 16));
      if constexpr (VC == ROT4) f *= f16_to_float(cur.vn[j >> 1] >> ((j & 1) * 16));
      vf[j] = f;
    }
    if (partial) {
      // rows past L may hold any bits: their factor is 0 (their p is 0 too)
#pragma unroll
      for (int j = 0; j < 8; ++j) vf[j] = t * kTile + 8 * qg + j < L ? vf[j] : 0.0f;
    }
    float vm = fabsf(vf[0]);  // largest |factor| among this lane's rows
#pragma unroll
    for (int j = 1; j < 8; ++j) vm = fmaxf(vm, fabsf(vf[j]));
    if (__builtin_amdgcn_ballot_w64(vm > st.vhi) || !__builtin_amdgcn_ballot_w64(vm >= st.vlo)) {
      int e;
      (void)__builtin_frexpf(wave_max(vm), &e);  // wave max in [2^(e-1), 2^e)
      vexp_new = static_cast<float>(e);
      st.vlo = __builtin_ldexpf(1.0f, e - 12);
      st.vhi = __builtin_ldexpf(1.0f, e + 4);
      v_rescale = true;
    }
  }

  // ---- S^T: lane (n16, qg) gets the 4 block partials of query row 4*nt + qg
  //      at tile row 16h + n16, for both halves h ----
  float kf[2][4];
  k_block_factors<KC>(cur, kf);
  float s[NT][2];
  half8 bk[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int m = 0; m < 4; ++m) bk[h][m] = unpack_k<KC>(cur.kd[h], m, lut);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float4v acc_h[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    float4v acc_l[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const half8 qh = aq.h[nt][m], ql = aq.l[nt][m];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        acc_h[h] = mfma16(qh, bk[h][m], acc_h[h]);
        acc_l[h] = mfma16(ql, bk[h][m], acc_l[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4v acc = acc_h[h] + acc_l[h];
      float v;
      if constexpr (KC == F16) v = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      else v = (acc[0] * kf[h][0] + acc[1] * kf[h][1]) + (acc[2] * kf[h][2] + acc[3] * kf[h][3]);
      const bool dead = partial && t * kTile + 16 * h + n16 >= lim[nt];
      s[nt][h] = dead ? -INFINITY : v;
    }
  }

  // ---- online softmax (base 2); all lanes of a 16-lane row share the row
  //      state; the reference is m_run + vexp ----
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float tmax = row16_max(fmaxf(s[nt][0], s[nt][1]));
    const float mnew = fmaxf(st.m_run[nt], tmax);
    if (__builtin_amdgcn_ballot_w64(mnew > st.m_run[nt]) || v_rescale) {
      const float alpha = __builtin_amdgcn_exp2f((st.m_run[nt] + st.vexp) - (mnew + vexp_new));
      st.l_run[nt] *= alpha;
#pragma unroll
      for (int c = 0; c < 8; ++c) st.oacc[c] *= alpha;
      st.m_run[nt] = mnew;
    }
    const float mref = st.m_run[nt] + vexp_new;
    const float p0 = __builtin_amdgcn_exp2f(s[nt][0] - mref);
    const float p1 = __builtin_amdgcn_exp2f(s[nt][1] - mref);
    st.l_run[nt] += p0 + p1;
    s_p[nt][qg][n16] = p0;
    s_p[nt][qg][16 + n16] = p1;
  }
  st.vexp = vexp_new;
  wave_lds_fence();
  float pv[NT][8];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float4v p_lo = *reinterpret_cast<const float4v*>(&s_p[nt][n16 >> 2][8 * qg]);
    const float4v p_hi = *reinterpret_cast<const float4v*>(&s_p[nt][n16 >> 2][8 * qg + 4]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pv[nt][j] = p_lo[j];
      pv[nt][4 + j] = p_hi[j];
    }
  }
  wave_lds_fence();

  // ---- O += P V: A row n16 = 4*(query row) + block b carries P times the
  //      block-b factor of V over tile rows 8qg .. 8qg+7 ----

  half8 aph[NT], apl[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if constexpr (VC != F16) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[nt][j] *= vf[j];
    }
    split8(pv[nt], aph[nt], apl[nt]);
  }
  const int row8 = t * kTile + 8 * qg;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    half8 bv = unpack_v<VC>(cur.vd, c, lut);
    if constexpr (VC == F16) {
      if (partial) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (row8 + j >= L) bv[j] = static_cast<_Float16>(0.0f);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      st.oacc[c] = mfma16(aph[nt], bv, st.oacc[c]);
      st.oacc[c] = mfma16(apl[nt], bv, st.oacc[c]);
    }
  }
}

// V factors of (tile row 8qg + j, block b) for all four blocks, as the 8-
// and 16-row layouts use them, with the rows past L zeroed, and the wave's V
// exponent check.  The fp16 block scales stay in fp16 (fw[b][i]: rows
// 8qg + 2i and 2i + 1; the largest magnitude is an integer max over the bit
// patterns, and the products take the fp16 operand directly); rot4's row
// norms come back in fp32 (nrm[j]), and its factor norm x scale is formed
// where it is used.
template <int KC, int VC, int NT>
__device__ __forceinline__ void v_block_factors(const TileRegs<KC, VC, NT>& cur, int t, int L, int qg, bool partial,
                                                WaveState<NT>& st, float (&nrm)[8], uint32_t (&fw)[4][4],
                                                float& vexp_new, bool& v_rescale) {
  vexp_new = st.vexp;
  v_rescale = false;
  if constexpr (VC != F16) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) fw[b][i] = cur.vs[b][i];
    if constexpr (VC == ROT4) {
#pragma unroll
      for (int j = 0; j < 8; ++j) nrm[j] = f16_to_float(cur.vn[j >> 1] >> ((j & 1) * 16));
    }
    if (partial) {
      // rows past L may hold any bits: their scale (and rot4 norm) is 0, so
      // their factor is 0 (their p is 0 too).  (The empty asm keeps this a
      // branch: only a tile cut by L pays.)
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = t * kTile + 8 * qg + 2 * i;
        const uint32_t keep = (r0 < L ? 0x0000FFFFu : 0u) | (r0 + 1 < L ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int b = 0; b < 4; ++b) fw[b][i] = fw[b][i] & keep;
        if constexpr (VC == ROT4) {
          nrm[2 * i] = r0 < L ? nrm[2 * i] : 0.0f;
          nrm[2 * i + 1] = r0 + 1 < L ? nrm[2 * i + 1] : 0.0f;
        }
      }
    }
    // largest |scale| among this lane's rows (fp16 magnitudes order like
    // their bit patterns); for rot4 times the largest norm, a bound on the
    // largest |norm x scale| within the scale spread of one row
    u16x2 mx = {0, 0};
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, fw[b][i] & 0x7FFF7FFFu));
    float vm = f16_to_float(mx[0] > mx[1] ? mx[0] : mx[1]);
    if constexpr (VC == ROT4) {
      float nm = nrm[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) nm = fmaxf(nm, nrm[j]);
      vm *= nm;
    }
    if (__builtin_amdgcn_ballot_w64(vm > st.vhi) || !__builtin_amdgcn_ballot_w64(vm >= st.vlo)) {
      int e;
      (void)__builtin_frexpf(wave_max(vm), &e);  // wave max in [2^(e-1), 2^e)
      vexp_new = static_cast<float>(e);
      st.vlo = __builtin_ldexpf(1.0f, e - 12);
      st.vhi = __builtin_ldexpf(1.0f, e + 4);
      v_rescale = true;
    }
  }
}

// One 32-row tile for one wave with 8 query rows.  Both products use rows
// r = 2 q + p: query q of the wave's 8, part p of its fp16 hi/lo split
// (0 = hi, 1 = lo), so no operand row is zero when 8 rows are live.
//   S^T: MFMA b covers block b; output lane (n16, qg) holds, for cached row
//        16h + n16, block b's partial dots of queries 2qg and 2qg+1 (hi and
//        lo rows), which are summed, scaled by the K block scale and summed
//        over the blocks.
//   P.V: for block b the A rows carry part p of P(q, row) times the V factor
//        of (row, block b) over the tile rows 8qg .. 8qg+7, and N-tile c uses
//        the operand of its block c / 2; the output rows are (query, part)
//        again, and the two parts are added at the end.
template <int KC, int VC>
__device__ __forceinline__ void process_tile_wide(const TileRegs<KC, VC, 2>& cur, int t, int L, int lmin,
                                                  const int (&lim)[2], int lane, const QOperands<2>& aq,
                                                  WaveState<2>& st, float* s_p, const Lut& lut) {
  const int n16 = lane & 15, qg = lane >> 4;
  const bool partial = (t + 1) * kTile > lmin;
  // ---- V factors of (tile row 8qg + j, block b) and the wave's V exponent
  //      check, first so that they overlap the S^T products ----
  [[maybe_unused]] float nrm[8];
  [[maybe_unused]] uint32_t fw[4][4];
  float vexp_new;
  bool v_rescale;
  v_block_factors(cur, t, L, qg, partial, st, nrm, fw, vexp_new, v_rescale);

  // ---- S^T: lane (n16, qg) gets queries 2qg + jj at tile row 16h + n16 ----
  float kf[2][4];
  k_block_factors<KC>(cur, kf);
  float s[2][2];  // [query 2qg + jj][half]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float4v acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      acc[b] = mfma16(aq.w[b], unpack_k<KC>(cur.kd[h], b, lut), float4v{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      float d[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) d[b] = acc[b][2 * jj] + acc[b][2 * jj + 1];
      if constexpr (KC == F16) s[jj][h] = (d[0] + d[1]) + (d[2] + d[3]);
      else s[jj][h] = (d[0] * kf[h][0] + d[1] * kf[h][1]) + (d[2] * kf[h][2] + d[3] * kf[h][3]);
    }
  }
  if (partial) {  // rows at or past a query's length
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        if (t * kTile + 16 * h + n16 >= lim[jj]) s[jj][h] = -INFINITY;
  }

  // ---- online softmax (base 2); the 16 lanes of a lane group share the
  //      state of its two queries; the reference is m_run + vexp.  One
  //      decision rescales both queries, so the accumulators are scaled as
  //      whole vectors {a0, a0, a1, a1} ----
  float mnew[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) mnew[jj] = fmaxf(st.m_run[jj], row16_max(fmaxf(s[jj][0], s[jj][1])));
  if (__builtin_amdgcn_ballot_w64(mnew[0] > st.m_run[0]) || __builtin_amdgcn_ballot_w64(mnew[1] > st.m_run[1]) ||
      v_rescale) {
    float alpha[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      alpha[jj] = __builtin_amdgcn_exp2f((st.m_run[jj] + st.vexp) - (mnew[jj] + vexp_new));
      st.l_run[jj] *= alpha[jj];
      st.m_run[jj] = mnew[jj];
    }
    const float4v av = {alpha[0], alpha[0], alpha[1], alpha[1]};
#pragma unroll
    for (int c = 0; c < 8; ++c) st.oacc[c] *= av;
  }
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const float mref = st.m_run[jj] + vexp_new;
    const float p0 = __builtin_amdgcn_exp2f(s[jj][0] - mref);
    const float p1 = __builtin_amdgcn_exp2f(s[jj][1] - mref);
    st.l_run[jj] += p0 + p1;
    s_p[(2 * qg + jj) * kTile + n16] = p0;
    s_p[(2 * qg + jj) * kTile + 16 + n16] = p1;
  }
  st.vexp = vexp_new;
  wave_lds_fence();
  // P of this lane's A row: query n16 >> 1 over tile rows 8qg .. 8qg+7
  float pv[8];
  {
    const float4v p_lo = *reinterpret_cast<const float4v*>(&s_p[(n16 >> 1) * kTile + 8 * qg]);
    const float4v p_hi = *reinterpret_cast<const float4v*>(&s_p[(n16 >> 1) * kTile + 8 * qg + 4]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pv[j] = p_lo[j];
      pv[4 + j] = p_hi[j];
    }
  }
  wave_lds_fence();

  // ---- O += P V ----
  // Part p of x: hi rows take fp16(x) toward zero, lo rows fp16(x - hi), the
  // same split as split8, chosen per lane by the row's parity.
  const float nb = (n16 & 1) ? -1.0f : 0.0f;
  auto part = [&](const float x[8]) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = split_part(x[2 * i], x[2 * i + 1], nb);
    return __builtin_bit_cast(half8, r);
  };
  half8 ap[4];
  if constexpr (VC == F16) {
    ap[0] = part(pv);
  } else {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float x[8];
      if constexpr (VC == ROT4) {
        // norm x scale is exact in fp32 (two fp16 values); then times P
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = pv[2 * i] * mul_f16<0>(nrm[2 * i], fw[b][i]);
          x[2 * i + 1] = pv[2 * i + 1] * mul_f16<1>(nrm[2 * i + 1], fw[b][i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = mul_f16<0>(pv[2 * i], fw[b][i]);
          x[2 * i + 1] = mul_f16<1>(pv[2 * i + 1], fw[b][i]);
        }
      }
      ap[b] = part(x);
    }
  }
  const int row8 = t * kTile + 8 * qg;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    half8 bv = unpack_v<VC>(cur.vd, c, lut);
    if constexpr (VC == F16) {
      if (partial) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (row8 + j >= L) bv[j] = static_cast<_Float16>(0.0f);
      }
    }
    st.oacc[c] = mfma16(VC == F16 ? ap[0] : ap[c >> 1], bv, st.oacc[c]);
  }
}

// One 32-row tile for one wave with 16 query rows (9 .. 16 per KV head: the
// tile is read and unpacked once for all of them).  The MFMA rows are the
// 16 queries in both products; the fp16 hi and lo parts of Q and of P go
// to two chained MFMAs.
//   S^T: for half h and block b, lane (n16, qg) gets block b's partial dots
//        of queries 4qg .. 4qg+3 at tile row 16h + n16, which are scaled by
//        the K block scale and summed over the blocks.
//   P.V: the A operand of block b is P(query n16, tile rows 8qg .. 8qg+7)
//        times the V factor of (row, block b); N-tile c uses the operands
//        of its block c / 2, and output lane (n16, qg) holds channel
//        16c + n16 of queries 4qg .. 4qg+3.
template <int KC, int VC>
__device__ __forceinline__ void process_tile_16(const TileRegs<KC, VC, 4>& cur, int t, int L, int lmin,
                                                const int (&lim)[4], int lane, const QOperands<4>& aq,
                                                WaveState<4>& st, float* s_p, const Lut& lut) {
  const int n16 = lane & 15, qg = lane >> 4;
  const bool partial = (t + 1) * kTile > lmin;
  [[maybe_unused]] float nrm[8];
  [[maybe_unused]] uint32_t fw[4][4];
  float vexp_new;
  bool v_rescale;
  v_block_factors(cur, t, L, qg, partial, st, nrm, fw, vexp_new, v_rescale);

  // ---- S^T ----
  float kf[2][4];
  k_block_factors<KC>(cur, kf);
  float s[4][2];  // [query 4qg + i][half]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float4v acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const half8 kb = unpack_k<KC>(cur.kd[h], b, lut);
      acc[b] = mfma16(aq.ops[b * 64 + lane], kb, float4v{0.0f, 0.0f, 0.0f, 0.0f});
      acc[b] = mfma16(aq.ops[(4 + b) * 64 + lane], kb, acc[b]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (KC == F16) s[i][h] = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
      else s[i][h] = (acc[0][i] * kf[h][0] + acc[1][i] * kf[h][1]) + (acc[2][i] * kf[h][2] + acc[3][i] * kf[h][3]);
    }
  }
  if (partial) {  // rows at or past a query's length
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t * kTile + 16 * h + n16 >= lim[i]) s[i][h] = -INFINITY;
  }

  // ---- online softmax (base 2); the 16 lanes of a lane group share the
  //      state of its four queries.  One decision rescales all four ----
  float mnew[4];
  bool grow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mnew[i] = fmaxf(st.m_run[i], row16_max(fmaxf(s[i][0], s[i][1])));
    grow = grow || mnew[i] > st.m_run[i];
  }
  if (__builtin_amdgcn_ballot_w64(grow) || v_rescale) {
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      alpha[i] = __builtin_amdgcn_exp2f((st.m_run[i] + st.vexp) - (mnew[i] + vexp_new));
      st.l_run[i] *= alpha[i];
      st.m_run[i] = mnew[i];
    }
    const float4v av = {alpha[0], alpha[1], alpha[2], alpha[3]};
#pragma unroll
    for (int c = 0; c < 8; ++c) st.oacc[c] *= av;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float mref = st.m_run[i] + vexp_new;
    const float p0 = __builtin_amdgcn_exp2f(s[i][0] - mref);
    const float p1 = __builtin_amdgcn_exp2f(s[i][1] - mref);
    st.l_run[i] += p0 + p1;
    s_p[(4 * qg + i) * kTile + n16] = p0;
    s_p[(4 * qg + i) * kTile + 16 + n16] = p1;
  }
  st.vexp = vexp_new;
  wave_lds_fence();
  // P of this lane's A row: query n16 over tile rows 8qg .. 8qg+7
  float pv[8];
  {
    const float4v p_lo = *reinterpret_cast<const float4v*>(&s_p[n16 * kTile + 8 * qg]);
    const float4v p_hi = *reinterpret_cast<const float4v*>(&s_p[n16 * kTile + 8 * qg + 4]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pv[j] = p_lo[j];
      pv[4 + j] = p_hi[j];
    }
  }
  wave_lds_fence();

  // ---- O += P V: block b's hi and lo operands are built just before its
  //      two N-tiles, so only one pair is live at a time ----
  const int row8 = t * kTile + 8 * qg;
  [[maybe_unused]] half8 fh, fl;  // f16 planes: one P operand pair for all N-tiles
  if constexpr (VC == F16) split8(pv, fh, fl);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    half8 ah, al;
    if constexpr (VC == F16) {
      ah = fh;
      al = fl;
    } else {
      float x[8];
      if constexpr (VC == ROT4) {
        // norm x scale is exact in fp32 (two fp16 values); then times P
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = pv[2 * i] * mul_f16<0>(nrm[2 * i], fw[b][i]);
          x[2 * i + 1] = pv[2 * i + 1] * mul_f16<1>(nrm[2 * i + 1], fw[b][i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = mul_f16<0>(pv[2 * i], fw[b][i]);
          x[2 * i + 1] = mul_f16<1>(pv[2 * i + 1], fw[b][i]);
        }
      }
      split8(x, ah, al);
    }
#pragma unroll
    for (int c = 2 * b; c < 2 * b + 2; ++c) {
      half8 bv = unpack_v<VC>(cur.vd, c, lut);
      if constexpr (VC == F16) {
        if (partial) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (row8 + j >= L) bv[j] = static_cast<_Float16>(0.0f);
        }
      }
      st.oacc[c] = mfma16(ah, bv, st.oacc[c]);
      st.oacc[c] = mfma16(al, bv, st.oacc[c]);
    }
  }
}

// Decode kernel: one workgroup of kDecodeWaves waves per (split, KV head,
// sequence), sized to be the only workgroup on its compute unit (two waves
// per SIMD).  Every wave handles all query rows of its KV head (RW = 4*NT
// >= G rows, padded with zero rows).  The split's tiles are dealt to the
// waves statically (tile slot k to wave k mod 8); with one workgroup per
// compute unit this measured within 1.5 % of waves taking tiles from an LDS
// counter as they free up, and it fixes the summation order.
template <int KC, int VC, int NT>
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_kernel(DecodeArgs a) {
  constexpr int RW = 4 * NT;
  constexpr int GMAX = 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n16 = lane & 15;
  const int qg = lane >> 4;
  const int split = blockIdx.x;
  const int head = blockIdx.y;
  const int seq = blockIdx.z;
  // Query rows of this KV head: r = t * gqa + g for new token t < q_len and
  // q-head g < gqa; row r attends rows 0 .. lmin - 1 + t of the stream.
  const int L = a.seq_len[seq];  // rows attended by the last new token
  const int QL = a.q_len;
  // Fetch every scalar argument the prologue uses in one round trip: read
  // one by one where they are first needed, the compiler waited for each
  // fetch in turn (four serial trips, about 1.3 us before the query loads
  // could be issued).
  const uint32_t ks0 = rotated(KC) ? a.ksigns[0] : 0u, ks1 = rotated(KC) ? a.ksigns[1] : 0u;
  const uint32_t ks2 = rotated(KC) ? a.ksigns[2] : 0u, ks3 = rotated(KC) ? a.ksigns[3] : 0u;
  __asm__ volatile("" ::"s"(L), "s"(QL), "s"(a.gqa), "s"(a.n_splits), "s"(a.n_kv_heads), "s"(a.n_q_heads),
                   "s"(a.capacity), "s"(a.q), "s"(a.k_new), "s"(a.kcodes), "s"(a.vcodes), "s"(a.qscale), "s"(ks0),
                   "s"(ks1), "s"(ks2), "s"(ks3));
  const int lmin = L - QL + 1;    // rows attended by the first new token
  const int G = a.gqa * QL;       // query rows
  constexpr int kThreads = 64 * kDecodeWaves;
  static_assert(RW <= GMAX, "query rows per wave");
  const int n_tiles = (L + kTile - 1) / kTile;
  // contiguous tile ranges per split (the last ones may be short or empty)
  const int tiles_per_split = (n_tiles + a.n_splits - 1) / a.n_splits;

  __shared__ __align__(16) float sq[GMAX][kD];
  constexpr bool kRot4 = KC == ROT4 || VC == ROT4;
  constexpr bool kRot3 = KC == ROT3 || VC == ROT3;
  __shared__ uint32_t lut[kRot4 ? 256 * 64 : 1];
  __shared__ uint32_t lut3[kRot3 ? 64 * 64 : 1];
  __shared__ float s_p[kDecodeWaves][NT][4][kTile];
  // the waves' outputs for the merge; with both tables (rot4 and rot3) they
  // reuse the 64 KB rot4 table once every wave is past its tiles
  constexpr bool kOutInLut = kRot4 && kRot3;
  static_assert(!kOutInLut || kDecodeWaves * RW * kD <= 256 * 64, "outputs fit the rot4 table");
  __shared__ float s_o_own[kOutInLut ? 1 : kDecodeWaves * RW * kD];
  float (*const s_o)[RW][kD] = reinterpret_cast<float (*)[RW][kD]>(kOutInLut ? static_cast<void*>(lut) : s_o_own);
  __shared__ float s_m[kDecodeWaves][RW];
  __shared__ float s_l[kDecodeWaves][RW];
  __shared__ uint8_t s_row[5][256];

  const int64_t ph = static_cast<int64_t>(seq) * a.n_kv_heads + head;
  const uint8_t* kbase = a.kcodes + ph * a.capacity * row_code_bytes(KC);
  const uint8_t* vbase = a.vcodes + ph * a.capacity * row_code_bytes(VC);
  const uint16_t* ksb = has_scales(KC) ? a.kscales + ph * a.capacity * 4 : nullptr;
  const uint16_t* vsb = has_scales(VC) ? a.vscales + ph * a.capacity * 4 : nullptr;
  const uint16_t* knb = has_norms(KC) ? a.knorms + ph * a.capacity : nullptr;
  const uint16_t* vnb = has_norms(VC) ? a.vnorms + ph * a.capacity : nullptr;

  // Tiles each wave has in flight from the start (its first D slots).
  constexpr int D = prefetch_depth<KC, VC, NT>() + 1;

  // ---- fused append: the new rows p = lmin - 1 + i (i < q_len) are stored
  //      by the workgroup owning their tile, before it reads that tile (no
  //      other workgroup reads it).  K row i goes on wave 2i; the V rows go
  //      in order on wave 1, because 4-bit V rows of one 8-row group share
  //      32-bit words that each store rewrites ----
  if (a.k_new != nullptr) {
    auto owned = [&](int i) { return ((lmin - 1 + i) / kTile) / tiles_per_split == split; };
    bool mine = false;
    int first_slot = n_tiles;  // the lowest slot of this split that gets a new row
    for (int i = 0; i < QL; ++i) {
      if (owned(i)) {
        mine = true;
        first_slot = min(first_slot, (lmin - 1 + i) / kTile - split * tiles_per_split);
      }
    }
    if (mine) {
      auto src = [&](int i) { return ((static_cast<int64_t>(seq) * QL + i) * a.n_kv_heads + head) * kD; };
      for (int i = 0; i < QL; ++i) {
        if (owned(i) && wave == 2 * i)
          append_one_row<KC, 0>(const_cast<uint8_t*>(kbase), const_cast<uint16_t*>(ksb), const_cast<uint16_t*>(knb),
                                lmin - 1 + i, a.k_new + src(i), lane, a.ksigns, s_row[i]);
      }
      if (wave == 1) {
        for (int i = 0; i < QL; ++i)
          if (owned(i))
            append_one_row<VC, 1>(const_cast<uint8_t*>(vbase), const_cast<uint16_t*>(vsb),
                                  const_cast<uint16_t*>(vnb), lmin - 1 + i, a.v_new + src(i), lane, a.vsigns,
                                  s_row[4]);
      }
      // Only waves of this workgroup read the rows back, and they share its
      // L1: a barrier's workgroup-scope release/acquire is enough.  (A
      // device-scope fence here writes back and invalidates the L2 and costs
      // tens of us.)  When no wave prefetches the tile of a new row (it is
      // past every wave's first D slots), the query staging barrier below
      // orders the stores before its first read, and the other waves go on
      // to issue their prefetch while the rows are encoded.
      if (first_slot < D * kDecodeWaves) __syncthreads();
    }
  }

  // Every global load below is unconditional: a load under a branch makes
  // the compiler wait for all outstanding loads where the paths merge, which
  // would serialise the prefetch.  Out-of-range indices are clamped instead.
  // index (into [S][q_len][Hq]) of query row r; also the output row
  auto qrow_index = [&](int r) {
    return (static_cast<int64_t>(seq) * QL + r / a.gqa) * a.n_q_heads + static_cast<int64_t>(head) * a.gqa + r % a.gqa;
  };
  // The query rows are staged through LDS: thread tid < 256 holds floats
  // 8*tid .. 8*tid+7 of the padded [16][128] rows (two registers per thread,
  // so nothing needs the query before the tile prefetch is issued).
  const int qs_row = min((8 * tid) >> 7, GMAX - 1);
  float4v q0, q1;
  [[maybe_unused]] uint32_t ksw = 0;
  {
    const float* qsrc = a.q + qrow_index(min(qs_row, G - 1)) * kD + ((8 * tid) & 127);
    q0 = *reinterpret_cast<const float4v*>(qsrc);
    q1 = *reinterpret_cast<const float4v*>(qsrc + 4);
    if constexpr (rotated(KC)) {
      // sign bits of those 8 channels (selected, not indexed: an indexed
      // read of the arguments is a vector load that the staging would wait on)
      const int si = ((8 * tid) & 127) >> 5;
      ksw = si == 0 ? ks0 : si == 1 ? ks1 : si == 2 ? ks2 : ks3;
    }
  }
  // rot4 levels: lane l (< 16) fetches level l; issued before the tile loads
  // so that building the table below does not wait for them
  [[maybe_unused]] uint32_t lv = 0, lv3 = 0;
  if constexpr (kRot4) lv = kLevelBits[lane & 15];
  if constexpr (kRot3) lv3 = kLevelBits3[lane & 7];
  // Keep those loads ahead of the tile prefetch: loads complete in issue
  // order, so the staging below then waits only for them, and the query
  // rotation overlaps the tiles' latency (left to itself the compiler
  // issues them after the tiles and waits for everything).
  __asm__ volatile("" ::: "memory");

  // Split s owns the contiguous tiles s * tiles_per_split .. (s + 1) *
  // tiles_per_split - 1 of the stream (slot k is tile first + k), so each
  // workgroup streams one run of memory.  Wave w owns the slots k = w,
  // w + kDecodeWaves, w + 2 kDecodeWaves, ..., in that order, so every
  // wave's summation order (and the result) is fixed.  It starts with its first D = prefetch_depth
  // + 1 slots in flight and loads its next slot into a buffer as soon as the
  // buffer is consumed.  Loads of slots past the last tile are clamped to
  // it; a split without tiles re-reads tile 0 (always there).
  const int first = split * tiles_per_split;
  const int n_mine = max(0, min(n_tiles - first, tiles_per_split));  // this split's tiles
  const int t_last = n_mine > 0 ? first + n_mine - 1 : 0;
  auto tile_of = [&](int k) { return first + k; };
  auto load_slot = [&](TileRegs<KC, VC, NT>& r, int k) {
    load_tile<KC, VC>(r, min(tile_of(k), t_last), lane, kbase, vbase, ksb, knb, vsb, vnb);
  };
  TileRegs<KC, VC, NT> ta, tb;
  [[maybe_unused]] TileRegs<KC, VC, NT> tc;
  // the first tile now; the second after the query staging barrier, so that
  // the waves reach the barrier without waiting for the whole compute unit's
  // prefetch to be issued (each 1 KB load takes the vector memory unit ~16
  // cycles: 8 waves x 2 tiles are ~1.2 us of issue)
  load_slot(ta, wave);
  // f16 keys at 8 query rows: the second tile now too (issued later, it is
  // live across the query operand build and the kernel spills)
  constexpr bool kSecondEarly = KC == F16 && NT == 2;
  if constexpr (kSecondEarly) load_slot(tb, wave + kDecodeWaves);

  if constexpr (kRot4) fill_rot4_lut<kThreads>(lut, tid, lv);
  if constexpr (kRot3) fill_rot3_lut<kThreads>(lut3, tid, lv3);
  const Lut lutr{lut, lut3, 4u * static_cast<uint32_t>(lane)};
  QOperands<NT> aq;
  // ---- A operands of S^T = Q K^T for this wave's rows: row n16 = 4*(query
  //      row) + block slot; MFMA m covers block m (lane group qg its chunk
  //      qg), so a row's operand is zero except in MFMA m = its slot ----
  if (tid < 256) {
    const int c0 = (8 * tid) & 127;
    const bool live = qs_row < G;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = live ? (j < 4 ? q0[j] : q1[j - 4]) : 0.0f;
      if constexpr (rotated(KC)) v = ((ksw >> ((c0 + j) & 31)) & 1u) ? -v : v;  // the keys' sign flip
      sq[qs_row][c0 + j] = v;
    }
  }
  __syncthreads();
  // (rotated keys: after the query rotation, whose barriers would otherwise
  // wait for every wave's issue of it)
  if constexpr (!rotated(KC) && !kSecondEarly) load_slot(tb, wave + kDecodeWaves);
  float qs = a.qscale;
  if constexpr (rotated(KC)) {
    // rotate the query rows like the keys (WHT); the keys reconstruct as
    // N*S*level/sqrt(128) (rot3: S*level/sqrt(128)) against q~ = H(s.q)/sqrt(128)
    wht128_lds<kThreads>(&sq[0][0], RW, tid);
    qs *= 1.0f / 128.0f;
    load_slot(tb, wave + kDecodeWaves);
  }
  // the lane's row is block slot = n16 & 3 of its query row (rows past G
  // are zero in sq); its operand is that block's chunk qg in MFMA m = slot
  if constexpr (NT == 1) {
    // row n16 = 4 * (query row) + block slot: the operand of the lane's row
    // is its slot's chunk qg, in MFMA m = slot, zero in the others
    const int slot = n16 & 3;
    const int g = n16 >> 2;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = sq[g][k_chan<KC>(qg, slot, j)] * qs;
    half8 h, l;
    split8(v, h, l);
    const half8 z = {};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      aq.h[0][m] = m == slot ? h : z;
      aq.l[0][m] = m == slot ? l : z;
    }
  } else if constexpr (NT == 4) {
    // row n16 = query row: in MFMA b the lane holds chunk qg of block b,
    // hi and lo parts in separate operands.  Wave 0 builds them and stores
    // them over the staged query rows (which every wave has read by the
    // barrier), where they stay until the tile loop ends.
    half8 oh[4], ol[4];
    if (wave == 0) {
      const int g = n16;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = sq[g][k_chan<KC>(qg, b, j)] * qs;
        split8(v, oh[b], ol[b]);
      }
    }
    __syncthreads();
    half8* ops = reinterpret_cast<half8*>(&sq[0][0]);
    static_assert(sizeof(half8) * 8 * 64 <= sizeof(sq), "operands fit the staging rows");
    if (wave == 0) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        ops[b * 64 + lane] = oh[b];
        ops[(4 + b) * 64 + lane] = ol[b];
      }
    }
    __syncthreads();
    aq.ops = ops;
  } else {
    // row n16 = 2 * (query row) + part: in MFMA b the lane holds part
    // n16 & 1 of chunk qg of block b of its query row
    const int g = n16 >> 1;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = sq[g][k_chan<KC>(qg, b, j)] * qs;
      half8 h, l;
      split8(v, h, l);
      aq.w[b] = (n16 & 1) ? l : h;
    }
  }
  // (the LUT was written before the staging barrier)

  WaveState<NT> st;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    // finite, so that a row whose tiles so far were all masked (an early new
    // token on a tile past its last row) gets p = 2^(-inf) = 0 and alpha
    // stays finite; no real score lies below it
    st.m_run[nt] = -__FLT_MAX__;
    st.l_run[nt] = 0.0f;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) st.oacc[c] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  st.vexp = 0.0f;
  st.vlo = INFINITY;  // the first tile sets the exponent
  st.vhi = INFINITY;

  // the lane's query row of state nt within the wave's RW rows
  auto state_row = [&](int nt) { return NT == 1 ? qg : NT * qg + nt; };
  // length of that row; padding rows past G stop at L like the last live row
  int lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) lim[nt] = min(lmin + state_row(nt) / a.gqa, L);

  // slot k is live while its tile exists; a wave's slots increase, so it
  // stops at its first dead slot
  auto live_slot = [&](int k) { return k < n_mine; };
  int next_slot = wave + D * kDecodeWaves;
  auto take = [&]() {  // the wave's next slot
    const int k = next_slot;
    next_slot += kDecodeWaves;
    return k;
  };
  auto proc = [&](const TileRegs<KC, VC, NT>& r, int t) {
    if constexpr (NT == 1) process_tile<KC, VC, NT>(r, t, L, lmin, lim, lane, aq, st, s_p[wave], lutr);
    else if constexpr (NT == 2) process_tile_wide<KC, VC>(r, t, L, lmin, lim, lane, aq, st, &s_p[wave][0][0][0], lutr);
    else process_tile_16<KC, VC>(r, t, L, lmin, lim, lane, aq, st, &s_p[wave][0][0][0], lutr);
  };
  int ka = wave, kb = wave + kDecodeWaves;
  if constexpr (D == 3) {
    // three register buffers in rotation: two tiles in flight while one is used
    int kc = wave + 2 * kDecodeWaves;
    load_slot(tc, kc);
    while (live_slot(ka)) {
      proc(ta, tile_of(ka));
      ka = take();
      load_slot(ta, ka);
      if (!live_slot(kb)) break;
      proc(tb, tile_of(kb));
      kb = take();
      load_slot(tb, kb);
      if (!live_slot(kc)) break;
      proc(tc, tile_of(kc));
      kc = take();
      load_slot(tc, kc);
    }
  } else {
    // two buffers: the next tile is in flight while one is used
    while (live_slot(ka)) {
      proc(ta, tile_of(ka));
      ka = take();
      load_slot(ta, ka);
      if (!live_slot(kb)) break;
      proc(tb, tile_of(kb));
      kb = take();
      load_slot(tb, kb);
    }
  }

  // ---- per-wave state to LDS: row r of the wave's RW query rows ----
  if constexpr (kOutInLut) __syncthreads();  // no wave reads the rot4 table any more
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = state_row(nt);
    const float l = row16_sum(st.l_run[nt]);
    if (n16 == 0) {
      s_m[wave][r] = st.m_run[nt] + st.vexp;  // the reference of l and O
      s_l[wave][r] = l;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // 4 rows: the output row of (query, block of N-tile c); 8 rows: hi + lo;
      // 16 rows: the query's own row
      const float o = NT == 1   ? st.oacc[c][c >> 1]
                      : NT == 2 ? st.oacc[c][2 * nt] + st.oacc[c][2 * nt + 1]
                                : st.oacc[c][nt];
      s_o[wave][r][16 * c + n16] = o;
    }
  }
  __syncthreads();

  // ---- merge the waves; write the partial or final row ----
  const bool final_out = a.n_splits == 1;
  for (int i = tid; i < RW * kD; i += kThreads) {
    const int g = i >> 7, c = i & 127;
    // all reads first, then no branch: a wave without rows (l = 0) gets
    // weight 0 by a select
    float mw[kDecodeWaves], lw[kDecodeWaves], ow[kDecodeWaves];
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      mw[w] = s_m[w][g];
      lw[w] = s_l[w][g];
      ow[w] = s_o[w][g][c];
    }
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mw[w]);
    float O = 0.0f, Ls = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = lw[w] > 0.0f ? __builtin_amdgcn_exp2f(mw[w] - M) : 0.0f;
      O += ow[w] * f;
      Ls += lw[w] * f;
    }
    if (final_out) {
      sq[g][c] = Ls > 0.0f ? O / Ls : 0.0f;
    } else if (g < G) {
      // agent-scope stores: coherent across the GPU's L2 caches without a
      // cache write-back, so a workgroup anywhere can merge them in-kernel
      const int64_t row = qrow_index(g) * a.n_splits + split;
      __hip_atomic_store(&a.ws_o[row * kD + c], O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (c == 0) {
        __hip_atomic_store(&a.ws_ml[row * 2], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.ws_ml[row * 2 + 1], Ls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  bool write_final = final_out;
  if (!final_out && a.arrive != nullptr) {
    // ---- in-kernel split merge: the last of the n_splits workgroups of this
    //      (sequence, KV head) to get here merges the partials of its rows.
    //      Each thread waits until its partial stores have completed; after
    //      the barrier one thread counts the workgroup in.  The count and the
    //      merge's loads are agent-scope atomics too, issued after those
    //      stores completed, so the last arrival reads every split's
    //      partial.  It also puts the count back to 0 for the next call ----
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&a.arrive[ph], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = prev == static_cast<uint32_t>(a.n_splits - 1);
      if (last) __hip_atomic_store(&a.arrive[ph], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last ? 1 : 0;
    }
    __syncthreads();
    if (s_last == 0) return;
    // thread (row r, channel group cg) merges every split of its row's 4
    // channels with the reduce kernel's arithmetic: split s goes to lane
    // s mod 8, each lane in split order, then the lanes in order; 16 splits'
    // loads are in flight at a time
    const int r = tid >> 5, cg = tid & 31;
    if (r < G) {
      constexpr int SL = kMergeLanesFew;
      const int64_t row0 = qrow_index(r) * a.n_splits;
      const float* ml = a.ws_ml + row0 * 2;
      const float* po = a.ws_o + row0 * kD + 4 * cg;
      // two floats in one agent-scope 8-byte load, split with scalar shifts
      // (a bit cast of an ext-vector element such as v[1] compiles to a
      // read of element 0 on this toolchain, so none is used)
      struct F2 {
        float x, y;
      };
      auto ld2 = [](const float* p) {
        const uint64_t w = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        return F2{__builtin_bit_cast(float, static_cast<uint32_t>(w)),
                  __builtin_bit_cast(float, static_cast<uint32_t>(w >> 32))};
      };
      float lm[SL], ll[SL];
      float4v lo[SL];
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        lm[i] = -INFINITY;
        ll[i] = 0.0f;
        lo[i] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
      }
      for (int s0 = 0; s0 < a.n_splits; s0 += 2 * SL) {
        F2 w_ml[2 * SL], w_o0[2 * SL], w_o1[2 * SL];
#pragma unroll
        for (int j = 0; j < 2 * SL; ++j) {
          const int s = min(s0 + j, a.n_splits - 1);
          w_ml[j] = ld2(ml + 2 * s);
          w_o0[j] = ld2(po + static_cast<int64_t>(s) * kD);
          w_o1[j] = ld2(po + static_cast<int64_t>(s) * kD + 2);
        }
#pragma unroll
        for (int j = 0; j < 2 * SL; ++j) {
          if (s0 + j < a.n_splits) {
            const float4v pv = {w_o0[j].x, w_o0[j].y, w_o1[j].x, w_o1[j].y};
            merge_into(lm[j % SL], ll[j % SL], lo[j % SL], w_ml[j].x, w_ml[j].y, pv);
          }
        }
      }
      const float4v v = combine_lanes<SL>([&](int i) { return lm[i]; }, [&](int i) { return ll[i]; },
                                          [&](int i) { return lo[i]; });
#pragma unroll
      for (int c = 0; c < 4; ++c) sq[r][4 * cg + c] = v[c];
    }
    write_final = true;
  }
  if (write_final) {
    __syncthreads();
    if constexpr (rotated(VC)) wht128_lds<kThreads>(&sq[0][0], RW, tid);
    for (int i = tid; i < G * kD; i += kThreads) {
      const int g = i >> 7, c = i & 127;
      float v = sq[g][c];
      if constexpr (rotated(VC)) {
        v *= (1.0f / 128.0f);
        v = ((a.vsigns[c >> 5] >> (c & 31)) & 1u) ? -v : v;
      }
      a.out[qrow_index(g) * kD + c] = v;
    }
  }
}

#define VIT_DECODE_NT(KC, VC)                                                                   \
  if (nt == 1)                                                                                  \
    hipExtLaunchKernelGGL((decode_kernel<KC, VC, 1>), grid, dim3(64 * kDecodeWaves), 0, stream, ev.start, ev.stop, 0, args); \
  else if (nt == 2)                                                                             \
    hipExtLaunchKernelGGL((decode_kernel<KC, VC, 2>), grid, dim3(64 * kDecodeWaves), 0, stream, ev.start, ev.stop, 0, args); \
  else                                                                                          \
    hipExtLaunchKernelGGL((decode_kernel<KC, VC, 4>), grid, dim3(64 * kDecodeWaves), 0, stream, ev.start, ev.stop, 0, args);

#define VIT_DECODE_FOR_K(KC)                                                          \
  hipError_t launch_decode_k##KC(int vc, int nt, dim3 grid, hipStream_t stream,       \
                                 const DecodeArgs& args, const KernelEvents& ev) {    \
    switch (vc) {                                                                     \
      case F16: VIT_DECODE_NT(KC, F16) break;                                         \
      case Q8_0: VIT_DECODE_NT(KC, Q8_0) break;                                       \
      case Q4_0: VIT_DECODE_NT(KC, Q4_0) break;                                       \
      case ROT4: VIT_DECODE_NT(KC, ROT4) break;                                       \
      case ROT3: VIT_DECODE_NT(KC, ROT3) break;                                       \
      default: return hipErrorInvalidValue;                                           \
    }                                                                                 \
    return hipGetLastError();                                                         \
  }

}  // namespace vit
