// Split-K merge of decode partials, plus the decode dispatch over K codecs.
//
// One workgroup per (query head, sequence) of 32 x SL threads (SL = 8, or 32
// above 64 splits).  Thread t owns channels 4*(t & 31) .. +3 and the partials
// s = (t >> 5), (t >> 5) + SL, ... ; each thread merges its partials online,
// then the SL partial merges per channel are combined through LDS.  Partial s
// of a row is (o_s[128] unnormalised, m_s in base-2 units, l_s):
// M = max m_s, L = sum l_s 2^(m_s - M), O = sum o_s 2^(m_s - M) / L.  Empty partials (l_s = 0, m_s = -inf) are
// skipped.  For a rot4 V plane the merged row is in the rotated domain scaled
// by sqrt(128); it is mapped back with x = s .* (H o) / 128.
#include "vit_device.h"
#include "vit_launch.h"

namespace vit {

__device__ inline void merge_into(float& M, float& L, float4v& O, float pm, float pl, float4v po) {
  if (pl > 0.0f) {
    if (pm > M) {
      const float sc = __builtin_amdgcn_exp2f(M - pm);
      O *= sc;
      L *= sc;
      M = pm;
    }
    const float f = __builtin_amdgcn_exp2f(pm - M);
    O += po * f;
    L += pl * f;
  }
}

// SL split lanes x 32 channel groups; SL = 8 for few splits, 32 for many.
template <int SL>
__global__ __launch_bounds__(32 * SL) void reduce_kernel(ReduceArgs a) {
  const int hq = blockIdx.x;
  const int seq = blockIdx.y;
  const int t = threadIdx.x;
  const int cg = t & 31, sl = t >> 5;
  const int64_t row = static_cast<int64_t>(seq) * a.n_q_heads + hq;
  const float* ml = a.ws_ml + row * a.n_splits * 2;
  const float* o = a.ws_o + row * a.n_splits * kD + 4 * cg;

  __shared__ float s_m[SL], s_l[SL];
  __shared__ float s_o[SL][kD];
  __shared__ float v[kD];

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

  if (t < kD) {
    float Mf = -INFINITY, Lf = 0.0f, Of = 0.0f;
#pragma unroll
    for (int i = 0; i < SL; ++i) Mf = fmaxf(Mf, s_m[i]);
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      if (s_l[i] > 0.0f) {
        const float f = __builtin_amdgcn_exp2f(s_m[i] - Mf);
        Of += s_o[i][t] * f;
        Lf += s_l[i] * f;
      }
    }
    v[t] = Lf > 0.0f ? Of / Lf : 0.0f;
  }
  if (a.rotate) {
    __syncthreads();
    for (int h = 1; h < kD; h <<= 1) {
      if (t < 64) {
        const int lo = ((t & ~(h - 1)) << 1) | (t & (h - 1));
        const float x = v[lo], y = v[lo + h];
        v[lo] = x + y;
        v[lo + h] = x - y;
      }
      __syncthreads();
    }
    if (t < kD) {
      float r = v[t] * (1.0f / 128.0f);
      v[t] = ((a.vsigns[t >> 5] >> (t & 31)) & 1u) ? -r : r;
    }
  }
  if (t < kD) a.out[row * kD + t] = v[t];
}

hipError_t launch_reduce(dim3 grid, hipStream_t stream, const ReduceArgs& args) {
  if (args.n_splits > 64) hipLaunchKernelGGL(reduce_kernel<32>, grid, dim3(1024), 0, stream, args);
  else hipLaunchKernelGGL(reduce_kernel<8>, grid, dim3(256), 0, stream, args);
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
