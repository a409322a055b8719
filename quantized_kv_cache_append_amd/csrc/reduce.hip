// Split-K merge of decode partials, plus the decode dispatch over K codecs.
//
// One workgroup per (query head, sequence) of 32 x SL threads (SL = 8, or 32
// above 64 splits).  Thread t owns channels 4*(t & 31) .. +3 and the partials
// s = (t >> 5), (t >> 5) + SL, ... ; each thread merges its partials online,
// then the SL lane results are combined through LDS (the arithmetic of
// merge.h, which the decode kernel's in-kernel merge shares).  For a rotated
// V plane the merged row is in the rotated domain scaled by sqrt(128); it is
// mapped back with x = s .* (H o) / 128.
#include "merge.h"
#include "vit_device.h"
#include "vit_launch.h"

namespace vit {

// SL split lanes x 32 channel groups; SL = 8 for few splits, 32 for many.
template <int SL>
__global__ __launch_bounds__(32 * SL) void reduce_kernel(ReduceArgs a) {
  const int hq = blockIdx.x;
  const int seq = blockIdx.y;
  // every scalar argument in one round trip (fetched where each is first
  // used, they were waited for one after another)
  __asm__ volatile("" ::"s"(a.n_q_heads), "s"(a.n_splits), "s"(a.ws_ml), "s"(a.ws_o), "s"(a.out), "s"(a.rotate));
  const int t = threadIdx.x;
  const int cg = t & 31, sl = t >> 5;
  const int64_t row = static_cast<int64_t>(seq) * a.n_q_heads + hq;
  const float* ml = a.ws_ml + row * a.n_splits * 2;
  const float* o = a.ws_o + row * a.n_splits * kD + 4 * cg;

  __shared__ float s_m[SL], s_l[SL];
  __shared__ __align__(16) float s_o[SL][kD];
  __shared__ __align__(16) float v[kD];

  float M = -INFINITY, L = 0.0f;
  float4v O = {0.0f, 0.0f, 0.0f, 0.0f};
  // 4 partials per round, all loads issued first (indices clamped, not branched)
  for (int s0 = sl; s0 < a.n_splits; s0 += 4 * SL) {
    float pm[4], pl[4];
    float4v po[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = min(s0 + SL * i, a.n_splits - 1);
      pm[i] = ml[2 * s];
      pl[i] = ml[2 * s + 1];
      po[i] = *reinterpret_cast<const float4v*>(o + static_cast<int64_t>(s) * kD);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (s0 + SL * i < a.n_splits) merge_into(M, L, O, pm[i], pl[i], po[i]);
  }
  if (cg == 0) {
    s_m[sl] = M;
    s_l[sl] = L;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) s_o[sl][4 * cg + i] = O[i];
  __syncthreads();

  if (t < 32) {
    const float4v r = combine_lanes<SL>([&](int i) { return s_m[i]; }, [&](int i) { return s_l[i]; },
                                        [&](int i) { return *reinterpret_cast<const float4v*>(&s_o[i][4 * t]); });
#pragma unroll
    for (int c = 0; c < 4; ++c) v[4 * t + c] = r[c];
  }
  __syncthreads();  // v is written 4 channels per thread and read 1 per thread
  if (a.rotate) {
    wht128_lds<32 * SL>(v, 1, t);
    if (t < kD) {
      float r = v[t] * (1.0f / 128.0f);
      v[t] = ((a.vsigns[t >> 5] >> (t & 31)) & 1u) ? -r : r;
    }
  }
  if (t < kD) a.out[row * kD + t] = v[t];
}

// Measurement aid: read n16 16-byte units with nontemporal loads, the way
// a decode wave reads a tile: each wave takes contiguous 8 KB chunks (eight
// wave-wide 16-byte loads of 1 KB each), two chunks in flight, chunks dealt
// to the waves of the whole grid in turn; nothing else is done.  The xor of
// the data is stored only if it equals a constant, so the loads stay live.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* buf, int64_t n16, uint32_t* sink) {
  constexpr int kChunk = 512;  // 16-byte units per chunk (8 KB)
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * (blockDim.x / 64);
  const int64_t n_chunks = n16 / kChunk;
  uint32_t acc = 0;
  int64_t c = wave;
  for (; c + n_waves < n_chunks; c += 2 * n_waves) {
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = __builtin_nontemporal_load(buf + c * kChunk + i * 64 + lane);
      v[8 + i] = __builtin_nontemporal_load(buf + (c + n_waves) * kChunk + i * 64 + lane);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  }
  for (; c < n_chunks; c += n_waves) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 v = __builtin_nontemporal_load(buf + c * kChunk + i * 64 + lane);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  // the units past the last whole chunk, one per thread of the grid
  for (int64_t i = n_chunks * kChunk + wave * 64 + lane; i < n16; i += n_waves * 64) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* buf, int64_t n16, uint32_t* sink, hipStream_t stream,
                              const KernelEvents& ev) {
  hipExtLaunchKernelGGL(stream_read_kernel, dim3(1024), dim3(256), 0, stream, ev.start, ev.stop, 0,
                        static_cast<const u32x4*>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t launch_reduce(dim3 grid, hipStream_t stream, const ReduceArgs& args) {
  if (args.n_splits > kMergeFewMaxSplits) hipLaunchKernelGGL(reduce_kernel<kMergeLanesMany>, grid, dim3(1024), 0, stream, args);
  else hipLaunchKernelGGL(reduce_kernel<kMergeLanesFew>, grid, dim3(256), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_decode(int kc, int vc, int nt, dim3 grid, hipStream_t stream, const DecodeArgs& args,
                         const KernelEvents& ev) {
  switch (kc) {
    case F16: return launch_decode_k0(vc, nt, grid, stream, args, ev);
    case Q8_0: return launch_decode_k1(vc, nt, grid, stream, args, ev);
    case Q4_0: return launch_decode_k2(vc, nt, grid, stream, args, ev);
    case ROT4: return launch_decode_k3(vc, nt, grid, stream, args, ev);
    case ROT3: return launch_decode_k4(vc, nt, grid, stream, args, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vit
