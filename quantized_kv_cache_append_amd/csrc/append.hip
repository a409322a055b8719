// Append: quantize new K or V rows and store them in a cache plane.
//
// Compiled with -ffp-contract=off: the encoders' fp32 operation order is part
// of the codec formats (codes and fp16 scales are bit-exact), so no multiply
// may fuse with an add.
//
// Work split: one 8-wave workgroup per (8-row group, KV head, sequence);
// wave j encodes row 8g + j when it lies in [pos0, pos0 + n_tokens) (lane l
// holds channels l and l + 64).  K rows go straight to their tile units.  For
// the V side the group's codes are collected in LDS, and each V column word
// (8 rows of one channel; rows share bytes in the 4-bit codecs) is then
// read-modified-written by a single lane, keeping rows outside the range.
#include "decode_impl.h"

namespace vit {

template <int CODEC, int SIDE>
__global__ __launch_bounds__(512) void append_kernel(AppendArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = tid >> 6;  // row of the group handled by this wave
  const int grp_local = blockIdx.x;
  const int head = blockIdx.y;
  const int seq = blockIdx.z;
  const int64_t p_begin = a.pos0[seq];
  const int64_t p_end = p_begin + a.n_tokens;
  const int64_t g = (p_begin >> 3) + grp_local;  // 8-row group index in the stream
  const int64_t g_first_row = g * 8;
  if (g_first_row >= p_end) return;  // this sequence has fewer groups (uniform)

  constexpr int RB = row_code_bytes(CODEC);
  const int64_t ph = static_cast<int64_t>(seq) * a.n_kv_heads + head;
  uint8_t* codes = static_cast<uint8_t*>(a.codes) + ph * a.capacity * RB;
  uint16_t* scales = has_scales(CODEC) ? a.scales + ph * a.capacity * 4 : nullptr;
  uint16_t* norms = has_norms(CODEC) ? a.norms + ph * a.capacity : nullptr;
  const uint32_t signs[4] = {a.signs[0], a.signs[1], a.signs[2], a.signs[3]};

  __shared__ uint8_t rowbuf[8][256];
  __shared__ uint32_t vcodes[8][128];

  const int64_t p = g_first_row + j;
  const bool live = p >= p_begin && p < p_end;
  const float* src = a.src + ((static_cast<int64_t>(seq) * a.n_tokens + (p - p_begin)) * a.n_kv_heads + head) * kD;

  if constexpr (SIDE == 0) {
    if (live) append_one_row<CODEC, 0>(codes, scales, norms, p, src, lane, signs, rowbuf[j]);
  } else {
    if (live) {
      const RowCodes rc = encode_row<CODEC>(src[lane], src[lane + 64], lane, signs);
      vcodes[j][lane] = rc.c0;
      vcodes[j][lane + 64] = rc.c1;
      const int64_t tile = p >> 5;
      const int pt = static_cast<int>(p & 31);
      if constexpr (has_scales(CODEC)) {
        if ((lane & 31) == 0) {
          const int b0 = lane >> 5;
          scales[v_scale_index(tile, b0, pt)] = rc.s0;
          scales[v_scale_index(tile, 2 + b0, pt)] = rc.s1;
        }
      }
      if constexpr (has_norms(CODEC)) {
        if (lane == 0) norms[p] = rc.norm;
      }
    }
    __syncthreads();
    if (j == 0) {
      // one lane per channel (two channels per lane): merge the group's rows
      // into the channel's column unit, keeping rows outside the range.
      bool in_range[8];
      bool all = true;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        in_range[r] = g_first_row + r >= p_begin && g_first_row + r < p_end;
        all = all && in_range[r];
      }
      const int64_t tile = g_first_row >> 5;
      const int pbase = static_cast<int>(g_first_row & 31);  // 8-aligned
      uint8_t* tbase = codes + tile * tile_code_bytes(CODEC);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ch = lane + 64 * half;
        int sh;
        if constexpr (CODEC == F16) {
          uint16_t* u = reinterpret_cast<uint16_t*>(tbase + v_code_offset(CODEC, pbase, ch, &sh));
#pragma unroll
          for (int r = 0; r < 8; ++r)
            if (in_range[r]) u[r] = static_cast<uint16_t>(vcodes[r][ch]);
        } else if constexpr (CODEC == Q8_0) {
#pragma unroll
          for (int r = 0; r < 8; ++r)
            if (in_range[r]) tbase[v_code_offset(CODEC, pbase + r, ch, &sh)] = static_cast<uint8_t>(vcodes[r][ch]);
        } else {
          // 4-bit: the channel's 8 rows live in one aligned 32-bit word
          const int off0 = v_code_offset(CODEC, pbase, ch, &sh);
          uint32_t* wp = reinterpret_cast<uint32_t*>(tbase + (off0 & ~3));
          uint32_t w = all ? 0u : *wp;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            if (!in_range[r]) continue;
            const int off = v_code_offset(CODEC, pbase + r, ch, &sh);
            const int bit = ((off & 3) << 3) + sh;
            w = (w & ~(0xFu << bit)) | ((vcodes[r][ch] & 0xFu) << bit);
          }
          *wp = w;
        }
      }
    }
  }
}

#define VIT_APPEND_CASE(C, S)                                                   \
  case (C)*2 + (S):                                                             \
    hipLaunchKernelGGL((append_kernel<C, S>), grid, dim3(512), 0, stream, args); \
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
