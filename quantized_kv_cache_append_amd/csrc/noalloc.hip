// vit_attn_decode_noalloc: decode attention (+ split-K merge) for callers
// that cannot allocate device memory.  The split partials live in `scratch`,
// a file-scope device array of this translation unit.  Host code never uses
// the array's name as an address: on the first call made with a GPU current,
// hipGetSymbolAddress gives that GPU's copy of the array, and that pointer is
// what the decode and reduce kernels receive.
#include <mutex>

#include "vit_launch.h"

namespace {

constexpr size_t kScratchBytes = VIT_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // per device; null until looked up

// The current device's copy of `scratch` (looked up once per device).
int scratch_for_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return VIT_E_HIP;
  if (dev >= kMaxDevices) return VIT_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return VIT_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return VIT_OK;
}

}  // namespace

extern "C" int vit_attn_decode_noalloc(const vit_kv_plane* k, const vit_kv_plane* v, const float* q,
                                       int32_t n_q_heads, int32_t q_len, const int64_t* seq_len,
                                       const float* k_new, const float* v_new, float scale, int32_t n_splits,
                                       float* out, void* stream) {
  const vit::KernelEvents ev = vit::take_armed_events();  // one-shot, whatever the outcome
  // validated as the decode with a workspace (which also covers every check
  // of the merge: shapes, split count, V codec and signs, alignment), then
  // the partials' size against the static array
  int st = vit::check_decode(k, v, q, n_q_heads, q_len, seq_len, k_new, v_new, scale, n_splits, true, nullptr, out);
  if (st != VIT_OK) return st;
  const int32_t rows = n_q_heads * q_len;
  if (n_splits > 1 && vit_attn_workspace_bytes(k->n_seqs, rows, VIT_HEAD_DIM, n_splits) > kScratchBytes)
    return VIT_E_SCRATCH;
  float* ws = nullptr;
  if (n_splits > 1) {
    st = scratch_for_current_device(&ws);
    if (st != VIT_OK) return st;
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  st = vit::enqueue_decode(k, v, q, n_q_heads, q_len, seq_len, k_new, v_new, scale, n_splits, ws, out, nullptr, hs, ev);
  if (st != VIT_OK || n_splits == 1) return st;
  return vit::enqueue_reduce(ws, k->n_seqs, rows, n_splits, v, out, hs);
}
