// Append: quantize new K or V rows and store them in a cache plane.
//
// Compiled with -ffp-contract=off: the encoders' fp32 operation order is part
// of the codec formats (codes and fp16 scales are bit-exact), so no multiply
// may fuse with an add.
//
// Work split: one wave per (8-row group, KV head, sequence).  The wave walks
// the group's rows that fall in [pos0, pos0 + n_tokens), encodes each row with
// the row encoder (lane l holds channels l and l + 64), writes the K-side
// units / scales / norms directly, and for the V side collects the group's
// codes in LDS so that each V column unit (8 rows of one channel, several rows
// sharing a byte for the 4-bit codecs) is read-modified-written by one lane.
#include "vit_device.h"
#include "vit_launch.h"

namespace vit {

template <int CODEC, int SIDE>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const int lane = threadIdx.x;
  const int grp_local = blockIdx.x;
  const int head = blockIdx.y;
  const int seq = blockIdx.z;
  const int64_t p_begin = a.pos0[seq];
  const int64_t p_end = p_begin + a.n_tokens;
  const int64_t g = (p_begin >> 3) + grp_local;  // 8-row group index in the stream
  const int64_t g_first_row = g * 8;
  if (g_first_row >= p_end) return;  // this sequence has fewer groups

  constexpr int RB = row_code_bytes(CODEC);
  const int64_t ph = static_cast<int64_t>(seq) * a.n_kv_heads + head;
  uint8_t* codes = static_cast<uint8_t*>(a.codes) + ph * a.capacity * RB;
  uint16_t* scales = a.scales ? a.scales + ph * a.capacity * 4 : nullptr;
  uint16_t* norms = a.norms ? a.norms + ph * a.capacity : nullptr;
  const uint32_t signs[4] = {a.signs[0], a.signs[1], a.signs[2], a.signs[3]};

  __shared__ uint8_t row_bytes[256];        // canonical bytes of one K row
  __shared__ uint32_t vcodes[8][128];       // V codes of the group's 8 rows
  __shared__ uint32_t in_range[8];

  if (lane < 8) {
    const int64_t p = g_first_row + lane;
    in_range[lane] = (p >= p_begin && p < p_end) ? 1u : 0u;
  }
  __syncthreads();

  for (int j = 0; j < 8; ++j) {
    const int64_t p = g_first_row + j;
    if (!in_range[j]) continue;
    const int64_t t = p - p_begin;
    const float* src = a.src + ((static_cast<int64_t>(seq) * a.n_tokens + t) * a.n_kv_heads + head) * kD;
    const float x0 = src[lane];
    const float x1 = src[lane + 64];
    const RowCodes rc = encode_row<CODEC>(x0, x1, lane, signs);

    const int64_t tile = p >> 5;
    const int pt = static_cast<int>(p & 31);
    if (scales && (lane & 31) == 0) {
      const int b0 = lane >> 5;  // block of x0; x1 is in block 2 + b0
      if constexpr (SIDE == 0) {
        scales[k_scale_index(p, b0)] = rc.s0;
        scales[k_scale_index(p, 2 + b0)] = rc.s1;
      } else {
        scales[v_scale_index(tile, b0, pt)] = rc.s0;
        scales[v_scale_index(tile, 2 + b0, pt)] = rc.s1;
      }
    }
    if (norms && lane == 0) norms[p] = rc.norm;

    if constexpr (SIDE == 0) {
      // canonical row bytes in LDS, then 16-byte units to their tile slots
      if constexpr (CODEC == F16) {
        reinterpret_cast<uint16_t*>(row_bytes)[lane] = static_cast<uint16_t>(rc.c0);
        reinterpret_cast<uint16_t*>(row_bytes)[lane + 64] = static_cast<uint16_t>(rc.c1);
        __syncthreads();
      } else if constexpr (CODEC == Q8_0) {
        row_bytes[lane] = static_cast<uint8_t>(rc.c0);
        row_bytes[lane + 64] = static_cast<uint8_t>(rc.c1);
        __syncthreads();
      } else {
        // nibble codes: byte 16b + j = code[32b + j] | code[32b + j + 16] << 4
        __shared__ uint8_t nib[128];
        nib[lane] = static_cast<uint8_t>(rc.c0);
        nib[lane + 64] = static_cast<uint8_t>(rc.c1);
        __syncthreads();
        const int b = lane >> 4, jj = lane & 15;
        row_bytes[lane] = static_cast<uint8_t>(nib[32 * b + jj] | (nib[32 * b + jj + 16] << 4));
        __syncthreads();
      }
      constexpr int CB = units_per_block(CODEC);
      if (lane < 4 * CB) {
        const int b = lane / CB, c = lane % CB;
        const u32x4 v = *reinterpret_cast<const u32x4*>(row_bytes + b * 16 * CB + 16 * c);
        *reinterpret_cast<u32x4*>(codes + tile * tile_code_bytes(CODEC) + k_unit_offset(CODEC, pt, b, c)) = v;
      }
      __syncthreads();
    } else {
      vcodes[j][lane] = rc.c0;
      vcodes[j][lane + 64] = rc.c1;
    }
  }

  if constexpr (SIDE == 1) {
    __syncthreads();
    // one lane per channel (two channels per lane): merge the group's rows
    // into the channel's column unit, keeping rows outside the range.
    const int64_t tile = g_first_row >> 5;
    const int pbase = static_cast<int>(g_first_row & 31);  // 8-aligned
    uint8_t* tbase = codes + tile * tile_code_bytes(CODEC);
    for (int half = 0; half < 2; ++half) {
      const int ch = lane + 64 * half;
      int sh;
      if constexpr (CODEC == F16) {
        uint16_t* u = reinterpret_cast<uint16_t*>(tbase + v_code_offset(CODEC, pbase, ch, &sh));
        for (int j = 0; j < 8; ++j)
          if (in_range[j]) u[j] = static_cast<uint16_t>(vcodes[j][ch]);
      } else if constexpr (CODEC == Q8_0) {
        for (int j = 0; j < 8; ++j)
          if (in_range[j]) tbase[v_code_offset(CODEC, pbase + j, ch, &sh)] = static_cast<uint8_t>(vcodes[j][ch]);
      } else {
        // 4-bit: the channel's 8 rows live in one aligned 32-bit word
        const int off0 = v_code_offset(CODEC, pbase, ch, &sh);
        uint32_t* wp = reinterpret_cast<uint32_t*>(tbase + (off0 & ~3));
        uint32_t w = 0;
        bool all = true;
        for (int j = 0; j < 8; ++j) all = all && in_range[j];
        if (!all) w = *wp;
        for (int j = 0; j < 8; ++j) {
          if (!in_range[j]) continue;
          const int off = v_code_offset(CODEC, pbase + j, ch, &sh);
          const int bit = ((off & 3) << 3) + sh;
          w = (w & ~(0xFu << bit)) | ((vcodes[j][ch] & 0xFu) << bit);
        }
        *wp = w;
      }
    }
  }
}

#define VIT_APPEND_CASE(C, S)                                                   \
  case (C)*2 + (S):                                                             \
    hipLaunchKernelGGL((append_kernel<C, S>), grid, dim3(64), 0, stream, args); \
    break;

hipError_t launch_append(int codec, int side, dim3 grid, hipStream_t stream, const AppendArgs& args) {
  switch (codec * 2 + side) {
    VIT_APPEND_CASE(F16, 0)
    VIT_APPEND_CASE(F16, 1)
    VIT_APPEND_CASE(Q8_0, 0)
    VIT_APPEND_CASE(Q8_0, 1)
    VIT_APPEND_CASE(Q4_0, 0)
    VIT_APPEND_CASE(Q4_0, 1)
    VIT_APPEND_CASE(ROT4, 0)
    VIT_APPEND_CASE(ROT4, 1)
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vit
