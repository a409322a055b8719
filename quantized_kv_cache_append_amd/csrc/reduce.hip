// Split-K merge of decode partials, plus the decode dispatch over K codecs.
//
// One 128-thread workgroup per (query head, sequence); thread c owns channel c.
// Partial s of a row is (o_s[128] unnormalised, m_s in base-2 units, l_s):
// M = max m_s, L = sum l_s 2^(m_s - M), O = sum o_s 2^(m_s - M) / L.  Empty
// splits (l_s = 0, m_s = -inf) are skipped.  For a rot4 V plane the merged
// row is in the rotated domain scaled by sqrt(128); it is mapped back with
// x = s .* (H o) / 128.
#include "vit_device.h"
#include "vit_launch.h"

namespace vit {

__global__ __launch_bounds__(128) void reduce_kernel(ReduceArgs a) {
  const int hq = blockIdx.x;
  const int seq = blockIdx.y;
  const int c = threadIdx.x;
  const int64_t row = static_cast<int64_t>(seq) * a.n_q_heads + hq;
  const float* ml = a.ws_ml + row * a.n_splits * 2;
  const float* o = a.ws_o + row * a.n_splits * kD;

  float M = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, ml[2 * s]);
  float O = 0.0f, L = 0.0f;
  for (int s = 0; s < a.n_splits; ++s) {
    const float l = ml[2 * s + 1];
    if (l > 0.0f) {
      const float f = __builtin_amdgcn_exp2f(ml[2 * s] - M);
      O += o[static_cast<int64_t>(s) * kD + c] * f;
      L += l * f;
    }
  }
  float r = L > 0.0f ? O / L : 0.0f;
  if (a.rotate) {
    __shared__ float v[kD];
    v[c] = r;
    __syncthreads();
    for (int h = 1; h < kD; h <<= 1) {
      if (c < 64) {
        const int lo = ((c & ~(h - 1)) << 1) | (c & (h - 1));
        const float x = v[lo], y = v[lo + h];
        v[lo] = x + y;
        v[lo + h] = x - y;
      }
      __syncthreads();
    }
    r = v[c] * (1.0f / 128.0f);
    r = ((a.vsigns[c >> 5] >> (c & 31)) & 1u) ? -r : r;
  }
  a.out[row * kD + c] = r;
}

hipError_t launch_reduce(dim3 grid, hipStream_t stream, const ReduceArgs& args) {
  hipLaunchKernelGGL(reduce_kernel, grid, dim3(kD), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_decode(int kc, int vc, dim3 grid, hipStream_t stream, const DecodeArgs& args) {
  switch (kc) {
    case F16: return launch_decode_k0(vc, grid, stream, args);
    case Q8_0: return launch_decode_k1(vc, grid, stream, args);
    case Q4_0: return launch_decode_k2(vc, grid, stream, args);
    case ROT4: return launch_decode_k3(vc, grid, stream, args);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vit
