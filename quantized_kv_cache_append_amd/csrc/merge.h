// Split-K merge arithmetic, shared by the reduce kernel and the decode
// kernel's in-kernel merge so that both give the same bits.
//
// Partial s of a query row is (o_s[128] unnormalised, m_s in base-2 units,
// l_s).  Lane i of SL merges the partials s = i, i + SL, i + 2 SL, ... in
// that order, online; the SL lane results are then combined in lane order:
// M = max m, L = sum l 2^(m - M), O = sum o 2^(m - M), and the row is O / L.
// Empty partials and lanes (l = 0) are skipped.
#pragma once

#include "vit_device.h"

namespace vit {

// Merge lanes: 8 for up to 64 splits, 32 above.
constexpr int kMergeLanesFew = 8;
constexpr int kMergeLanesMany = 32;
constexpr int kMergeFewMaxSplits = 64;

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

// The lanes' (M, L, O) of 4 channels combined in lane order; the normalised
// channels (0 when every lane is empty).  m(i), l(i), o(i) read lane i.
template <int SL, class GetM, class GetL, class GetO>
__device__ inline float4v combine_lanes(GetM m, GetL l, GetO o) {
  float Mf = -INFINITY;
#pragma unroll
  for (int i = 0; i < SL; ++i) Mf = fmaxf(Mf, m(i));
  float Lf = 0.0f;
  float4v Of = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const float li = l(i);
    if (li > 0.0f) {
      const float f = __builtin_amdgcn_exp2f(m(i) - Mf);
      Of += o(i) * f;
      Lf += li * f;
    }
  }
  float4v r = {0.0f, 0.0f, 0.0f, 0.0f};
  if (Lf > 0.0f) {
#pragma unroll
    for (int c = 0; c < 4; ++c) r[c] = Of[c] / Lf;
  }
  return r;
}

}  // namespace vit
