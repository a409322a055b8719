// Flash-decode attention over a quantized KV plane pair, for gfx950.
//
// One workgroup (4 waves) per (split, KV head, sequence).  The split's 32-row
// tiles are dealt round-robin to the 4 waves; each wave keeps its own online
// softmax state and the waves are merged through LDS at the end.
//
// Both products run on MFMA 16x16x32 f16 with exact operands:
//   * K and V codes are exact in fp16 (f16 values, int8 / 4-bit integers,
//     fp16 rot4 levels), and every per-block scale is applied in fp32;
//   * the query and the probabilities are split into fp16 hi + lo parts
//     (two MFMAs), so operand rounding stays near 2^-22 relative.
// Query rows are packed four per 16-column MFMA tile, one column per
// (query row, 32-channel block) pair: lane group q (lanes 16q..16q+15) of the
// A operand always holds block q of its K row, and the B operand is zero
// except where column block == q.  One MFMA chain therefore yields per-block
// partial dot products for four query rows at once, which are scaled by the
// block scale in fp32 and summed across the four column lanes.  The same
// (row, block) pairing builds the P.V operand, with the V block scale folded
// into P per block, so no lane does dequantization work for padding rows.
#pragma once

#include "vit_device.h"
#include "vit_launch.h"

namespace vit {

__device__ inline float4v mfma16(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// --- exact fp16 conversions of packed codes ---------------------------------
__device__ inline half2v h2_bits(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ inline uint32_t bits_h2(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// four int8 codes -> fp16 pairs (b0,b2) and (b1,b3): (0x6400 | (c ^ 0x80)) is
// the fp16 value 1024 + c + 128, so subtracting 1152 is exact.
__device__ inline u32x2 q8_pairs(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const half2v k = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  u32x2 r;
  r[0] = bits_h2(h2_bits((u & 0x00FF00FFu) | 0x64006400u) - k);
  r[1] = bits_h2(h2_bits(((u >> 8) & 0x00FF00FFu) | 0x64006400u) - k);
  return r;
}

__device__ inline half8 q8_unpack(uint32_t w0, uint32_t w1) {
  const u32x2 a = q8_pairs(w0), b = q8_pairs(w1);
  const u32x4 r = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(half8, r);
}

// eight 4-bit codes (offset 8) -> fp16 pairs, element order
// (lo b0, lo b2, lo b1, lo b3, hi b0, hi b2, hi b1, hi b3).
__device__ inline half8 q4_unpack(uint32_t w) {
  const half2v k_lo = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
  const half2v s_hi = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
  const half2v k_hi = {static_cast<_Float16>(-72.0f), static_cast<_Float16>(-72.0f)};
  const uint32_t w8 = w >> 8;
  const half2v a = h2_bits((w & 0x000F000Fu) | 0x64006400u) - k_lo;
  const half2v b = h2_bits((w8 & 0x000F000Fu) | 0x64006400u) - k_lo;
  const half2v c = h2_bits((w & 0x00F000F0u) | 0x64006400u) * s_hi + k_hi;
  const half2v d = h2_bits((w8 & 0x00F000F0u) | 0x64006400u) * s_hi + k_hi;
  half8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// eight rot4 indices -> fp16 levels through the byte LUT (LUT[b] = level[b&15]
// | level[b>>4] << 16), element order (lo b0, hi b0, lo b1, hi b1, ...).
__device__ inline half8 rot4_unpack(uint32_t w, const uint32_t* lut) {
  u32x4 r;
  r[0] = lut[w & 0xFFu];
  r[1] = lut[(w >> 8) & 0xFFu];
  r[2] = lut[(w >> 16) & 0xFFu];
  r[3] = lut[w >> 24];
  return __builtin_bit_cast(half8, r);
}

// Channel (within the row) of element j of lane group q's K operand in MFMA m.
template <int KC>
__device__ inline int k_chan(int q, int m, int j) {
  if constexpr (KC == F16) {
    return 32 * q + 8 * m + j;
  } else if constexpr (KC == Q8_0) {
    const int p8 = (j & 4) | ((j & 1) << 1) | ((j >> 1) & 1);
    return 32 * q + 16 * (m >> 1) + 8 * (m & 1) + p8;
  } else if constexpr (KC == Q4_0) {
    const int byte = 4 * m + (((j & 1) << 1) | ((j >> 1) & 1));
    return 32 * q + byte + ((j >> 2) << 4);
  } else {
    return 32 * q + 4 * m + (j >> 1) + ((j & 1) << 4);
  }
}

template <int KC>
__device__ inline half8 unpack_k(const u32x4* units, int m, const uint32_t* lut) {
  if constexpr (KC == F16) {
    return __builtin_bit_cast(half8, units[m]);
  } else if constexpr (KC == Q8_0) {
    const u32x4 u = units[m >> 1];
    return (m & 1) ? q8_unpack(u[2], u[3]) : q8_unpack(u[0], u[1]);
  } else if constexpr (KC == Q4_0) {
    return q4_unpack(units[0][m]);
  } else {
    return rot4_unpack(units[0][m], lut);
  }
}

// V operand of N-tile nt (channels 16nt..16nt+15): element j = row 8q + j.
template <int VC>
__device__ inline half8 unpack_v(const u32x4* vd, int nt, const uint32_t* lut) {
  if constexpr (VC == F16) {
    return __builtin_bit_cast(half8, vd[nt]);
  } else if constexpr (VC == Q8_0) {
    const u32x4 u = vd[nt >> 1];
    return (nt & 1) ? q8_unpack(u[2], u[3]) : q8_unpack(u[0], u[1]);
  } else if constexpr (VC == Q4_0) {
    return q4_unpack(vd[nt >> 2][nt & 3]);
  } else {
    return rot4_unpack(vd[nt >> 2][nt & 3], lut);
  }
}

template <int C>
constexpr int v_loads() {
  return C == F16 ? 8 : (C == Q8_0 ? 4 : 2);
}

__device__ inline float quad_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ inline float quad_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}

// Per-row factors (fp32) of the 8 rows 8q..8q+7 for one block: fp16 scale,
// times the fp16 norm for rot4.
template <int C>
__device__ inline void row_factors(u32x4 sc, u32x4 nm, float f[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v = f16_to_float(sc[j >> 1] >> ((j & 1) * 16));
    if constexpr (C == ROT4) v *= f16_to_float(nm[j >> 1] >> ((j & 1) * 16));
    f[j] = v;
  }
}

template <int KC, int VC, int NT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int GP = 4 * NT;
  constexpr int KCB = units_per_block(KC);
  constexpr int NVL = v_loads<VC>();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n16 = lane & 15;
  const int qg = lane >> 4;
  const int split = blockIdx.x;
  const int head = blockIdx.y;
  const int seq = blockIdx.z;
  const int L = a.seq_len[seq];
  const int G = a.gqa;
  const int n_tiles = (L + kTile - 1) / kTile;
  const int tps = (n_tiles + a.n_splits - 1) / a.n_splits;
  const int t_begin = min(n_tiles, split * tps);
  const int t_end = min(n_tiles, t_begin + tps);

  __shared__ float sq[GP][kD];
  __shared__ uint32_t lut[256];
  __shared__ float s_o[4][GP][kD];
  __shared__ float s_m[4][GP];
  __shared__ float s_l[4][GP];

  // ---- query rows (zero rows pad G up to GP); rot4 K: sign flip + WHT ----
  const float* qrow = a.q + (static_cast<int64_t>(seq) * a.n_q_heads + static_cast<int64_t>(head) * G) * kD;
  for (int i = tid; i < GP * kD; i += 256) {
    const int g = i >> 7, c = i & 127;
    float v = g < G ? qrow[g * kD + c] : 0.0f;
    if constexpr (KC == ROT4) v = ((a.ksigns[c >> 5] >> (c & 31)) & 1u) ? -v : v;
    sq[g][c] = v;
  }
  if constexpr (KC == ROT4 || VC == ROT4) {
    const int i = tid;
    lut[i] = static_cast<uint32_t>(kLevelBits[i & 15]) | (static_cast<uint32_t>(kLevelBits[i >> 4]) << 16);
  }
  __syncthreads();
  if constexpr (KC == ROT4) {
    for (int h = 1; h < kD; h <<= 1) {
      for (int i = tid; i < GP * 64; i += 256) {
        const int g = i >> 6, k = i & 63;
        const int lo = ((k & ~(h - 1)) << 1) | (k & (h - 1));
        const float x = sq[g][lo], y = sq[g][lo + h];
        sq[g][lo] = x + y;
        sq[g][lo + h] = x - y;
      }
      __syncthreads();
    }
  }
  // rot4 K rows reconstruct as N*S*level/sqrt(128) against q~ = H(s.q)/sqrt(128)
  const float qs = (KC == ROT4) ? a.qscale * (1.0f / 128.0f) : a.qscale;

  // ---- B operands of S = K Q^T: column n16 = 4*(row) + block slot ----------
  half8 bqh[NT][4], bql[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int g = 4 * nt + (n16 >> 2);
    const bool live = (n16 & 3) == qg;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = live ? sq[g][k_chan<KC>(qg, m, j)] * qs : 0.0f;
        const _Float16 hi = static_cast<_Float16>(v);
        bqh[nt][m][j] = hi;
        bql[nt][m][j] = static_cast<_Float16>(v - static_cast<float>(hi));
      }
    }
  }

  const int64_t ph = static_cast<int64_t>(seq) * a.n_kv_heads + head;
  const uint8_t* kbase = a.kcodes + ph * a.capacity * row_code_bytes(KC);
  const uint8_t* vbase = a.vcodes + ph * a.capacity * row_code_bytes(VC);
  const uint16_t* ksb = has_scales(KC) ? a.kscales + ph * a.capacity * 4 : nullptr;
  const uint16_t* vsb = has_scales(VC) ? a.vscales + ph * a.capacity * 4 : nullptr;
  const uint16_t* knb = has_norms(KC) ? a.knorms + ph * a.capacity : nullptr;
  const uint16_t* vnb = has_norms(VC) ? a.vnorms + ph * a.capacity : nullptr;

  float m_run[NT], l_run[NT];
  float4v oacc[NT][8];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) oacc[nt][c] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  }

  for (int t = t_begin + wave; t < t_end; t += 4) {
    // ---- loads: every wave-wide 16-byte load covers 1 KB of contiguous bytes
    const uint8_t* kt = kbase + static_cast<int64_t>(t) * tile_code_bytes(KC);
    const uint8_t* vt = vbase + static_cast<int64_t>(t) * tile_code_bytes(VC);
    u32x4 kd[2][KCB];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int c = 0; c < KCB; ++c)
        kd[hf][c] = *reinterpret_cast<const u32x4*>(kt + ((hf * KCB + c) * 64 + lane) * 16);
    u32x4 vd[NVL];
#pragma unroll
    for (int i = 0; i < NVL; ++i) vd[i] = *reinterpret_cast<const u32x4*>(vt + (i * 64 + lane) * 16);
    const int blk = lane & 3;
    u32x4 kss{}, kns{}, vss{}, vns{};
    if constexpr (has_scales(KC)) kss = *reinterpret_cast<const u32x4*>(ksb + static_cast<int64_t>(t) * 128 + blk * 32 + 8 * qg);
    if constexpr (has_norms(KC)) kns = *reinterpret_cast<const u32x4*>(knb + static_cast<int64_t>(t) * 32 + 8 * qg);
    if constexpr (has_scales(VC)) vss = *reinterpret_cast<const u32x4*>(vsb + static_cast<int64_t>(t) * 128 + blk * 32 + 8 * qg);
    if constexpr (has_norms(VC)) vns = *reinterpret_cast<const u32x4*>(vnb + static_cast<int64_t>(t) * 32 + 8 * qg);

    // ---- S = K Q^T per (row, block) column, two 16-row halves ----
    float s[NT][8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      half8 ak[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) ak[m] = unpack_k<KC>(kd[hf], m, lut);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc = mfma16(ak[m], bqh[nt][m], acc);
          acc = mfma16(ak[m], bql[nt][m], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) s[nt][4 * hf + i] = acc[i];
      }
    }
    if constexpr (KC != F16) {
      float kf[8];
      row_factors<KC>(kss, kns, kf);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 8; ++j) s[nt][j] *= kf[j];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = s[nt][j];
        v += quad_xor1(v);
        v += quad_xor2(v);
        s[nt][j] = v;
      }
    const int row0 = t * kTile + 8 * qg;
    const bool partial = (t + 1) * kTile > L;
    if (partial) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (row0 + j >= L) s[nt][j] = -INFINITY;
    }

    // ---- online softmax (base 2) ----
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float tmax = s[nt][0];
#pragma unroll
      for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, s[nt][j]);
      tmax = fmaxf(tmax, shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      const float mnew = fmaxf(m_run[nt], tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - mnew);
      float psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(s[nt][j] - mnew);
        s[nt][j] = p;
        psum += p;
      }
      l_run[nt] = l_run[nt] * alpha + psum;
      m_run[nt] = mnew;
      // the accumulator rows of lane group qg belong to query row 4*nt + qg
      const float alpha_o = __shfl(alpha, 4 * qg, kWave);
#pragma unroll
      for (int c = 0; c < 8; ++c) oacc[nt][c] *= alpha_o;
    }

    // ---- O += P V: A rows (query row, block) carry P times the V block factor
    float vf[8];
    if constexpr (VC != F16) row_factors<VC>(vss, vns, vf);
    half8 aph[NT], apl[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = s[nt][j];
        if constexpr (VC != F16) v = (v != 0.0f) ? v * vf[j] : 0.0f;
        const _Float16 hi = static_cast<_Float16>(v);
        aph[nt][j] = hi;
        apl[nt][j] = static_cast<_Float16>(v - static_cast<float>(hi));
      }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      half8 bv = unpack_v<VC>(vd, c, lut);
      if constexpr (VC == F16) {
        if (partial) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (row0 + j >= L) bv[j] = static_cast<_Float16>(0.0f);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        oacc[nt][c] = mfma16(aph[nt], bv, oacc[nt][c]);
        oacc[nt][c] = mfma16(apl[nt], bv, oacc[nt][c]);
      }
    }
  }

  // ---- per-wave state to LDS ----
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = l_run[nt];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (qg == 0 && (n16 & 3) == 0) {
      s_m[wave][4 * nt + (n16 >> 2)] = m_run[nt];
      s_l[wave][4 * nt + (n16 >> 2)] = l;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) s_o[wave][4 * nt + qg][16 * c + n16] = oacc[nt][c][c >> 1];
  }
  __syncthreads();

  // ---- merge the 4 waves; write the partial or the final row ----
  const bool final_out = a.n_splits == 1;
  for (int i = tid; i < GP * kD; i += 256) {
    const int g = i >> 7, c = i & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][g]);
    float O = 0.0f, Ls = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lw = s_l[w][g];
      if (lw > 0.0f) {
        const float f = __builtin_amdgcn_exp2f(s_m[w][g] - M);
        O += s_o[w][g][c] * f;
        Ls += lw * f;
      }
    }
    if (final_out) {
      sq[g][c] = Ls > 0.0f ? O / Ls : 0.0f;
    } else if (g < G) {
      const int64_t row = (static_cast<int64_t>(seq) * a.n_q_heads + static_cast<int64_t>(head) * G + g) * a.n_splits + split;
      a.ws_o[row * kD + c] = O;
      if (c == 0) {
        a.ws_ml[row * 2] = M;
        a.ws_ml[row * 2 + 1] = Ls;
      }
    }
  }
  if (final_out) {
    __syncthreads();
    if constexpr (VC == ROT4) {
      for (int h = 1; h < kD; h <<= 1) {
        for (int i = tid; i < GP * 64; i += 256) {
          const int g = i >> 6, k = i & 63;
          const int lo = ((k & ~(h - 1)) << 1) | (k & (h - 1));
          const float x = sq[g][lo], y = sq[g][lo + h];
          sq[g][lo] = x + y;
          sq[g][lo + h] = x - y;
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < G * kD; i += 256) {
      const int g = i >> 7, c = i & 127;
      float v = sq[g][c];
      if constexpr (VC == ROT4) {
        v *= (1.0f / 128.0f);
        v = ((a.vsigns[c >> 5] >> (c & 31)) & 1u) ? -v : v;
      }
      a.out[(static_cast<int64_t>(seq) * a.n_q_heads + static_cast<int64_t>(head) * G + g) * kD + c] = v;
    }
  }
}

#define VIT_DECODE_NT(KC, VC)                                                                 \
  switch (nt) {                                                                               \
    case 1: hipLaunchKernelGGL((decode_kernel<KC, VC, 1>), grid, dim3(256), 0, stream, args); break; \
    case 2: hipLaunchKernelGGL((decode_kernel<KC, VC, 2>), grid, dim3(256), 0, stream, args); break; \
    case 4: hipLaunchKernelGGL((decode_kernel<KC, VC, 4>), grid, dim3(256), 0, stream, args); break; \
    default: return hipErrorInvalidValue;                                                     \
  }

#define VIT_DECODE_FOR_K(KC)                                                          \
  hipError_t launch_decode_k##KC(int vc, int nt, dim3 grid, hipStream_t stream,       \
                                 const DecodeArgs& args) {                            \
    switch (vc) {                                                                     \
      case F16: VIT_DECODE_NT(KC, F16) break;                                         \
      case Q8_0: VIT_DECODE_NT(KC, Q8_0) break;                                       \
      case Q4_0: VIT_DECODE_NT(KC, Q4_0) break;                                       \
      case ROT4: VIT_DECODE_NT(KC, ROT4) break;                                       \
      default: return hipErrorInvalidValue;                                           \
    }                                                                                 \
    return hipGetLastError();                                                         \
  }

}  // namespace vit
