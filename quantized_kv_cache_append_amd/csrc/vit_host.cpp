// C ABI of the library: host-side validation, argument packing and launches.
// Every check runs before anything is enqueued; a failed check returns a
// negative vit_status and touches no device state.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/vit.h"
#include "vit_launch.h"

namespace {

constexpr int kRowBytes[4] = {256, 128, 64, 64};

// events armed by vit_arm_kernel_events for this host thread's next decode
thread_local vit::KernelEvents g_armed;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_plane(const vit_kv_plane* p) {
  if (!p) return VIT_E_ARG;
  if (p->codec < VIT_CODEC_F16 || p->codec > VIT_CODEC_ROT4) return VIT_E_UNSUPPORTED;
  if (p->side != VIT_SIDE_K && p->side != VIT_SIDE_V) return VIT_E_ARG;
  if (p->head_dim != VIT_HEAD_DIM) return VIT_E_UNSUPPORTED;
  if (p->reserved != 0) return VIT_E_ARG;
  if (p->n_seqs < 1 || p->n_kv_heads < 1 || p->capacity <= 0) return VIT_E_ARG;
  if (p->n_seqs > VIT_MAX_SEQS) return VIT_E_UNSUPPORTED;
  if (p->capacity > VIT_MAX_CAPACITY) return VIT_E_UNSUPPORTED;
  if (p->capacity % VIT_CAPACITY_ALIGN != 0) return VIT_E_CAPACITY;
  if (!p->codes) return VIT_E_ARG;
  if (p->codec != VIT_CODEC_F16 && !p->scales) return VIT_E_ARG;
  if (p->codec == VIT_CODEC_ROT4 && (!p->norms || !p->signs)) return VIT_E_ARG;
  if (!aligned(p->codes, 256) || (p->scales && !aligned(p->scales, 256)) ||
      (p->norms && !aligned(p->norms, 256)))
    return VIT_E_ALIGN;
  return VIT_OK;
}

void load_signs(const vit_kv_plane* p, uint32_t out[4]) {
  memset(out, 0, 4 * sizeof(uint32_t));
  if (p->codec == VIT_CODEC_ROT4 && p->signs) {
    for (int j = 0; j < 16; ++j) out[j >> 2] |= static_cast<uint32_t>(p->signs[j]) << (8 * (j & 3));
  }
}

size_t ws_o_bytes(int32_t s, int32_t hq, int32_t ns) {
  const size_t b = static_cast<size_t>(s) * hq * ns * VIT_HEAD_DIM * sizeof(float);
  return (b + 255) & ~size_t{255};
}

int enqueue_append(const vit_kv_plane* dst, const float* src, const int64_t* pos0, int32_t n_tokens,
                   hipStream_t stream) {
  vit::AppendArgs a{};
  a.codes = dst->codes;
  a.scales = dst->scales;
  a.norms = dst->norms;
  a.src = src;
  a.capacity = dst->capacity;
  a.n_kv_heads = dst->n_kv_heads;
  a.n_tokens = n_tokens;
  load_signs(dst, a.signs);
  int64_t groups = 0;
  for (int s = 0; s < dst->n_seqs; ++s) {
    a.pos0[s] = pos0[s];
    const int64_t g = ((pos0[s] + n_tokens - 1) >> 3) - (pos0[s] >> 3) + 1;
    if (g > groups) groups = g;
  }
  const dim3 grid(static_cast<unsigned>((groups + vit::kAppendWaves - 1) / vit::kAppendWaves),
                  static_cast<unsigned>(dst->n_kv_heads),
                  static_cast<unsigned>(dst->n_seqs));
  return vit::launch_append(dst->codec, dst->side, grid, stream, a) == hipSuccess ? VIT_OK : VIT_E_HIP;
}

}  // namespace

extern "C" {

const char* vit_status_string(int status) {
  switch (status) {
    case VIT_OK: return "ok";
    case VIT_E_ARG: return "invalid argument";
    case VIT_E_UNSUPPORTED: return "unsupported shape or codec";
    case VIT_E_CAPACITY: return "row outside the plane capacity (or capacity not a multiple of 256)";
    case VIT_E_ALIGN: return "misaligned pointer";
    case VIT_E_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int vit_kv_plane_sizes(int32_t codec, int32_t n_seqs, int32_t n_kv_heads, int32_t head_dim,
                       int64_t capacity, size_t* codes_bytes, size_t* scales_bytes,
                       size_t* norms_bytes) {
  if (codec < VIT_CODEC_F16 || codec > VIT_CODEC_ROT4) return VIT_E_UNSUPPORTED;
  if (head_dim != VIT_HEAD_DIM) return VIT_E_UNSUPPORTED;
  if (n_seqs < 1 || n_kv_heads < 1 || capacity <= 0) return VIT_E_ARG;
  if (n_seqs > VIT_MAX_SEQS) return VIT_E_UNSUPPORTED;
  if (capacity > VIT_MAX_CAPACITY) return VIT_E_UNSUPPORTED;
  if (capacity % VIT_CAPACITY_ALIGN != 0) return VIT_E_CAPACITY;
  const size_t rows = static_cast<size_t>(n_seqs) * n_kv_heads * capacity;
  if (codes_bytes) *codes_bytes = rows * kRowBytes[codec];
  if (scales_bytes) *scales_bytes = codec == VIT_CODEC_F16 ? 0 : rows * 4 * sizeof(uint16_t);
  if (norms_bytes) *norms_bytes = codec == VIT_CODEC_ROT4 ? rows * sizeof(uint16_t) : 0;
  return VIT_OK;
}

int vit_kv_append_quant(const vit_kv_plane* dst, const float* src, const int64_t* pos0,
                        int32_t n_tokens, void* stream) {
  int st = check_plane(dst);
  if (st != VIT_OK) return st;
  if (n_tokens < 0 || !pos0) return VIT_E_ARG;
  if (n_tokens == 0) return VIT_OK;
  if (!src) return VIT_E_ARG;
  if (!aligned(src, 16)) return VIT_E_ALIGN;
  for (int s = 0; s < dst->n_seqs; ++s)
    if (pos0[s] < 0 || pos0[s] + n_tokens > dst->capacity) return VIT_E_CAPACITY;
  return enqueue_append(dst, src, pos0, n_tokens, static_cast<hipStream_t>(stream));
}

size_t vit_attn_workspace_bytes(int32_t n_seqs, int32_t n_q_heads, int32_t head_dim, int32_t n_splits) {
  if (head_dim != VIT_HEAD_DIM || n_seqs < 1 || n_q_heads < 1 || n_splits < 1 || n_splits > VIT_MAX_SPLITS)
    return 0;
  return ws_o_bytes(n_seqs, n_q_heads, n_splits) + static_cast<size_t>(n_seqs) * n_q_heads * n_splits * 2 * sizeof(float);
}

int32_t vit_attn_default_splits(int32_t n_seqs, int32_t n_kv_heads, int32_t n_q_heads, int64_t max_seq_len) {
  (void)n_q_heads;
  if (n_seqs < 1 || n_kv_heads < 1 || max_seq_len < 1) return 1;
  const int64_t units = static_cast<int64_t>(n_seqs) * n_kv_heads;
  const int64_t tiles = (max_seq_len + 31) / 32;
  int64_t s = (256 + units - 1) / units;        // ~one (8-wave) workgroup per compute unit
  const int64_t by_work = tiles / 4 > 0 ? tiles / 4 : 1;  // >= 4 tiles per split
  if (s > by_work) s = by_work;
  if (s > VIT_MAX_SPLITS) s = VIT_MAX_SPLITS;
  if (s < 1) s = 1;
  return static_cast<int32_t>(s);
}

int vit_attn_decode(const vit_kv_plane* k, const vit_kv_plane* v, const float* q, int32_t n_q_heads,
                    const int64_t* seq_len, const float* k_new, const float* v_new, float scale,
                    int32_t n_splits, float* workspace, float* out, void* stream) {
  return vit_attn_decode_mq(k, v, q, n_q_heads, 1, seq_len, k_new, v_new, scale, n_splits, workspace, out, stream);
}

int vit_attn_decode_mq(const vit_kv_plane* k, const vit_kv_plane* v, const float* q, int32_t n_q_heads,
                       int32_t q_len, const int64_t* seq_len, const float* k_new, const float* v_new, float scale,
                       int32_t n_splits, float* workspace, float* out, void* stream) {
  const vit::KernelEvents ev = g_armed;  // one-shot: consumed by this call whatever its outcome
  g_armed = vit::KernelEvents{};
  int st = check_plane(k);
  if (st != VIT_OK) return st;
  st = check_plane(v);
  if (st != VIT_OK) return st;
  if (k->side != VIT_SIDE_K || v->side != VIT_SIDE_V) return VIT_E_ARG;
  if (k->n_seqs != v->n_seqs || k->n_kv_heads != v->n_kv_heads || k->capacity != v->capacity) return VIT_E_ARG;
  if (!q || !out || !seq_len) return VIT_E_ARG;
  if (n_q_heads < 1 || n_q_heads % k->n_kv_heads != 0) return VIT_E_ARG;
  if (q_len < 1) return VIT_E_ARG;
  const int32_t gqa = n_q_heads / k->n_kv_heads;
  if (q_len > VIT_MAX_QLEN || gqa * q_len > VIT_MAX_GQA) return VIT_E_UNSUPPORTED;
  if ((k_new == nullptr) != (v_new == nullptr)) return VIT_E_ARG;
  if (n_splits < 1 || n_splits > VIT_MAX_SPLITS) return VIT_E_ARG;
  if (n_splits > 1 && !workspace) return VIT_E_ARG;
  if (!isfinite(scale)) return VIT_E_ARG;
  for (int s = 0; s < k->n_seqs; ++s) {
    if (seq_len[s] < q_len) return VIT_E_ARG;
    if (seq_len[s] > k->capacity) return VIT_E_CAPACITY;
  }
  if (!aligned(q, 16) || !aligned(out, 16) || (workspace && !aligned(workspace, 16)) ||
      (k_new && !aligned(k_new, 16)) || (v_new && !aligned(v_new, 16)))
    return VIT_E_ALIGN;

  hipStream_t hs = static_cast<hipStream_t>(stream);

  vit::DecodeArgs a{};
  a.kcodes = static_cast<const uint8_t*>(k->codes);
  a.kscales = k->scales;
  a.knorms = k->norms;
  a.vcodes = static_cast<const uint8_t*>(v->codes);
  a.vscales = v->scales;
  a.vnorms = v->norms;
  a.q = q;
  a.k_new = k_new;  // quantized and stored in-kernel by the owning workgroup
  a.v_new = v_new;
  a.ws_o = workspace;
  a.ws_ml = workspace ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                                 ws_o_bytes(k->n_seqs, n_q_heads * q_len, n_splits))
                      : nullptr;
  a.out = out;
  a.capacity = k->capacity;
  a.n_kv_heads = k->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.gqa = gqa;
  a.q_len = q_len;
  a.n_splits = n_splits;
  a.qscale = scale * 1.4426950408889634f;
  load_signs(k, a.ksigns);
  load_signs(v, a.vsigns);
  for (int s = 0; s < k->n_seqs; ++s) a.seq_len[s] = static_cast<int32_t>(seq_len[s]);
  const dim3 grid(static_cast<unsigned>(n_splits), static_cast<unsigned>(k->n_kv_heads),
                  static_cast<unsigned>(k->n_seqs));
  const int rows = gqa * q_len;  // query rows per KV head, all in every wave
  const int nt = rows <= 4 ? 1 : rows <= 8 ? 2 : 4;  // query rows per wave: 4, 8 or 16
  return vit::launch_decode(k->codec, v->codec, nt, grid, hs, a, ev) == hipSuccess ? VIT_OK : VIT_E_HIP;
}

int vit_arm_kernel_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return VIT_E_ARG;
  g_armed.start = static_cast<hipEvent_t>(start_event);
  g_armed.stop = static_cast<hipEvent_t>(stop_event);
  return VIT_OK;
}

int vit_attn_splitk_reduce(const float* workspace, int32_t n_seqs, int32_t n_q_heads, int32_t head_dim,
                           int32_t n_splits, const vit_kv_plane* v, float* out, void* stream) {
  if (head_dim != VIT_HEAD_DIM) return VIT_E_UNSUPPORTED;
  if (!workspace || !out || !v) return VIT_E_ARG;
  if (n_seqs < 1 || n_q_heads < 1 || n_splits < 2 || n_splits > VIT_MAX_SPLITS) return VIT_E_ARG;
  if (n_seqs > VIT_MAX_SEQS) return VIT_E_UNSUPPORTED;
  if (v->codec < VIT_CODEC_F16 || v->codec > VIT_CODEC_ROT4) return VIT_E_UNSUPPORTED;
  if (v->codec == VIT_CODEC_ROT4 && !v->signs) return VIT_E_ARG;
  if (!aligned(workspace, 16) || !aligned(out, 16)) return VIT_E_ALIGN;
  vit::ReduceArgs a{};
  a.ws_o = workspace;
  a.ws_ml = reinterpret_cast<const float*>(reinterpret_cast<const char*>(workspace) +
                                           ws_o_bytes(n_seqs, n_q_heads, n_splits));
  a.out = out;
  a.n_q_heads = n_q_heads;
  a.n_splits = n_splits;
  a.rotate = v->codec == VIT_CODEC_ROT4 ? 1 : 0;
  load_signs(v, a.vsigns);
  const dim3 grid(static_cast<unsigned>(n_q_heads), static_cast<unsigned>(n_seqs));
  return vit::launch_reduce(grid, static_cast<hipStream_t>(stream), a) == hipSuccess ? VIT_OK : VIT_E_HIP;
}

}  // extern "C"
