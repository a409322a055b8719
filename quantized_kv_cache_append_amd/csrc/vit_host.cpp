// C ABI of the library: host-side validation, argument packing and launches.
// Every check runs before anything is enqueued; a failed check returns a
// negative vit_status and touches no device state.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/vit.h"
#include "vit_launch.h"

namespace {

constexpr int kRowBytes[5] = {256, 128, 64, 64, 48};

bool is_rotated(int32_t codec) { return codec == VIT_CODEC_ROT4 || codec == VIT_CODEC_ROT3; }

// events armed by vit_arm_kernel_events for this host thread's next append, decode, transcode
// or probe call
thread_local vit::KernelEvents g_armed;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_plane(const vit_kv_plane* p) {
  if (!p) return VIT_E_ARG;
  if (p->codec < VIT_CODEC_F16 || p->codec > VIT_CODEC_ROT3) return VIT_E_UNSUPPORTED;
  if (p->side != VIT_SIDE_K && p->side != VIT_SIDE_V) return VIT_E_ARG;
  if (p->head_dim != VIT_HEAD_DIM) return VIT_E_UNSUPPORTED;
  if (p->reserved != 0) return VIT_E_ARG;
  if (p->n_seqs < 1 || p->n_kv_heads < 1 || p->capacity <= 0) return VIT_E_ARG;
  if (p->n_seqs > VIT_MAX_SEQS) return VIT_E_UNSUPPORTED;
  if (p->capacity > VIT_MAX_CAPACITY) return VIT_E_UNSUPPORTED;
  if (p->capacity % VIT_CAPACITY_ALIGN != 0) return VIT_E_CAPACITY;
  if (!p->codes) return VIT_E_ARG;
  if (p->codec != VIT_CODEC_F16 && !p->scales) return VIT_E_ARG;
  if (p->codec == VIT_CODEC_ROT4 && !p->norms) return VIT_E_ARG;
  if (is_rotated(p->codec) && !p->signs) return VIT_E_ARG;
  if (!aligned(p->codes, 256) || (p->scales && !aligned(p->scales, 256)) ||
      (p->norms && !aligned(p->norms, 256)))
    return VIT_E_ALIGN;
  return VIT_OK;
}

void load_signs(const vit_kv_plane* p, uint32_t out[4]) {
  memset(out, 0, 4 * sizeof(uint32_t));
  if (is_rotated(p->codec) && p->signs) {
    for (int j = 0; j < 16; ++j) out[j >> 2] |= static_cast<uint32_t>(p->signs[j]) << (8 * (j & 3));
  }
}

// True when an array of plane a shares a byte with an array of plane b.
bool planes_overlap(const vit_kv_plane* a, const vit_kv_plane* b) {
  const void* ap[3] = {a->codes, a->scales, a->norms};
  const void* bp[3] = {b->codes, b->scales, b->norms};
  size_t ab[3], bb[3];
  vit_kv_plane_sizes(a->codec, a->n_seqs, a->n_kv_heads, VIT_HEAD_DIM, a->capacity, &ab[0], &ab[1], &ab[2]);
  vit_kv_plane_sizes(b->codec, b->n_seqs, b->n_kv_heads, VIT_HEAD_DIM, b->capacity, &bb[0], &bb[1], &bb[2]);
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      if (!ap[i] || !bp[j] || ab[i] == 0 || bb[j] == 0) continue;
      const uintptr_t a0 = reinterpret_cast<uintptr_t>(ap[i]), b0 = reinterpret_cast<uintptr_t>(bp[j]);
      if (a0 < b0 + bb[j] && b0 < a0 + ab[i]) return true;
    }
  return false;
}

size_t ws_o_bytes(int32_t s, int32_t hq, int32_t ns) {
  const size_t b = static_cast<size_t>(s) * hq * ns * VIT_HEAD_DIM * sizeof(float);
  return (b + 255) & ~size_t{255};
}

int enqueue_append(const vit_kv_plane* dst, const float* src, const int64_t* pos0, int32_t n_tokens,
                   hipStream_t stream, const vit::KernelEvents& ev) {
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
  return vit::launch_append(dst->codec, dst->side, grid, stream, a, ev) == hipSuccess ? VIT_OK : VIT_E_HIP;
}

}  // namespace

namespace vit {

KernelEvents take_armed_events() {
  const KernelEvents ev = g_armed;
  g_armed = KernelEvents{};
  return ev;
}

int check_decode(const vit_kv_plane* k, const vit_kv_plane* v, const float* q, int32_t n_q_heads, int32_t q_len,
                 const int64_t* seq_len, const float* k_new, const float* v_new, float scale, int32_t n_splits,
                 bool have_workspace, const void* workspace, const float* out) {
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
  if (n_splits > 1 && !have_workspace) return VIT_E_ARG;
  if (!isfinite(scale)) return VIT_E_ARG;
  for (int s = 0; s < k->n_seqs; ++s) {
    if (seq_len[s] < q_len) return VIT_E_ARG;
    if (seq_len[s] > k->capacity) return VIT_E_CAPACITY;
  }
  if (!aligned(q, 16) || !aligned(out, 16) || (workspace && !aligned(workspace, 16)) ||
      (k_new && !aligned(k_new, 16)) || (v_new && !aligned(v_new, 16)))
    return VIT_E_ALIGN;
  return VIT_OK;
}

int enqueue_decode(const vit_kv_plane* k, const vit_kv_plane* v, const float* q, int32_t n_q_heads, int32_t q_len,
                   const int64_t* seq_len, const float* k_new, const float* v_new, float scale, int32_t n_splits,
                   float* workspace, float* out, uint32_t* arrive, hipStream_t stream, const KernelEvents& ev) {
  const int32_t gqa = n_q_heads / k->n_kv_heads;
  DecodeArgs a{};
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
  a.arrive = n_splits > 1 ? arrive : nullptr;
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
  return launch_decode(k->codec, v->codec, nt, grid, stream, a, ev) == hipSuccess ? VIT_OK : VIT_E_HIP;
}

int check_reduce(const float* workspace, int32_t n_seqs, int32_t n_q_heads, int32_t head_dim, int32_t n_splits,
                 const vit_kv_plane* v, const float* out) {
  if (head_dim != VIT_HEAD_DIM) return VIT_E_UNSUPPORTED;
  if (!workspace || !out || !v) return VIT_E_ARG;
  if (n_seqs < 1 || n_q_heads < 1 || n_splits < 2 || n_splits > VIT_MAX_SPLITS) return VIT_E_ARG;
  if (n_seqs > VIT_MAX_SEQS) return VIT_E_UNSUPPORTED;
  if (v->codec < VIT_CODEC_F16 || v->codec > VIT_CODEC_ROT3) return VIT_E_UNSUPPORTED;
  if (is_rotated(v->codec) && !v->signs) return VIT_E_ARG;
  if (!aligned(workspace, 16) || !aligned(out, 16)) return VIT_E_ALIGN;
  return VIT_OK;
}

int enqueue_reduce(const float* workspace, int32_t n_seqs, int32_t n_q_heads, int32_t n_splits,
                   const vit_kv_plane* v, float* out, hipStream_t stream) {
  ReduceArgs a{};
  a.ws_o = workspace;
  a.ws_ml = reinterpret_cast<const float*>(reinterpret_cast<const char*>(workspace) +
                                           ws_o_bytes(n_seqs, n_q_heads, n_splits));
  a.out = out;
  a.n_q_heads = n_q_heads;
  a.n_splits = n_splits;
  a.rotate = is_rotated(v->codec) ? 1 : 0;
  load_signs(v, a.vsigns);
  const dim3 grid(static_cast<unsigned>(n_q_heads), static_cast<unsigned>(n_seqs));
  return launch_reduce(grid, stream, a) == hipSuccess ? VIT_OK : VIT_E_HIP;
}

}  // namespace vit

extern "C" {

const char* vit_status_string(int status) {
  switch (status) {
    case VIT_OK: return "ok";
    case VIT_E_ARG: return "invalid argument";
    case VIT_E_UNSUPPORTED: return "unsupported shape or codec";
    case VIT_E_CAPACITY: return "row outside the plane capacity (or capacity not a multiple of 256)";
    case VIT_E_ALIGN: return "misaligned pointer";
    case VIT_E_HIP: return "HIP launch error";
    case VIT_E_SCRATCH: return "split partials larger than the static scratch (VIT_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int vit_kv_plane_sizes(int32_t codec, int32_t n_seqs, int32_t n_kv_heads, int32_t head_dim,
                       int64_t capacity, size_t* codes_bytes, size_t* scales_bytes,
                       size_t* norms_bytes) {
  if (codec < VIT_CODEC_F16 || codec > VIT_CODEC_ROT3) return VIT_E_UNSUPPORTED;
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
  const vit::KernelEvents ev = g_armed;  // one-shot: consumed by this call whatever its outcome
  g_armed = vit::KernelEvents{};
  int st = check_plane(dst);
  if (st != VIT_OK) return st;
  if (n_tokens < 0 || !pos0) return VIT_E_ARG;
  if (n_tokens == 0) return VIT_OK;
  if (!src) return VIT_E_ARG;
  if (!aligned(src, 16)) return VIT_E_ALIGN;
  for (int s = 0; s < dst->n_seqs; ++s)
    if (pos0[s] < 0 || pos0[s] + n_tokens > dst->capacity) return VIT_E_CAPACITY;
  return enqueue_append(dst, src, pos0, n_tokens, static_cast<hipStream_t>(stream), ev);
}

int vit_kv_append_quant_multi(const vit_kv_plane* planes, int32_t n_planes, const float* const* src,
                              const int64_t* pos0, int32_t n_tokens, void* stream) {
  const vit::KernelEvents ev = g_armed;  // one-shot: consumed by this call whatever its outcome
  g_armed = vit::KernelEvents{};
  if (!planes || !src || !pos0) return VIT_E_ARG;
  if (n_planes < 1 || n_planes > VIT_MAX_APPEND_PLANES) return VIT_E_UNSUPPORTED;
  if (n_tokens < 0) return VIT_E_ARG;
  for (int i = 0; i < n_planes; ++i) {
    const vit_kv_plane* p = &planes[i];
    const int st = check_plane(p);
    if (st != VIT_OK) return st;
    if (p->n_seqs != planes[0].n_seqs || p->n_kv_heads != planes[0].n_kv_heads) return VIT_E_ARG;
    for (int j = 0; j < i; ++j)
      if (planes_overlap(&planes[j], p)) return VIT_E_ARG;  // every plane's arrays disjoint from the others
    if (n_tokens > 0) {
      if (!src[i]) return VIT_E_ARG;
      if (!aligned(src[i], 16)) return VIT_E_ALIGN;
    }
    for (int s = 0; s < p->n_seqs; ++s)
      if (pos0[s] < 0 || pos0[s] + n_tokens > p->capacity) return VIT_E_CAPACITY;
  }
  if (n_tokens == 0) return VIT_OK;
  vit::AppendMultiArgs a{};
  const int32_t S = planes[0].n_seqs;
  for (int i = 0; i < n_planes; ++i) {
    vit::AppendPlane& d = a.planes[i];
    d.codes = planes[i].codes;
    d.scales = planes[i].scales;
    d.norms = planes[i].norms;
    d.src = src[i];
    d.capacity = planes[i].capacity;
    d.codec_side = planes[i].codec * 2 + planes[i].side;
    load_signs(&planes[i], d.signs);
  }
  a.n_kv_heads = planes[0].n_kv_heads;
  a.n_tokens = n_tokens;
  a.n_seqs = S;
  a.n_planes = n_planes;
  int64_t groups = 0;
  for (int s = 0; s < S; ++s) {
    a.pos0[s] = pos0[s];
    const int64_t g = ((pos0[s] + n_tokens - 1) >> 3) - (pos0[s] >> 3) + 1;
    if (g > groups) groups = g;
  }
  const dim3 grid(static_cast<unsigned>((groups + vit::kAppendWaves - 1) / vit::kAppendWaves),
                  static_cast<unsigned>(a.n_kv_heads), static_cast<unsigned>(S * n_planes));
  return vit::launch_append_multi(grid, static_cast<hipStream_t>(stream), a, ev) == hipSuccess ? VIT_OK : VIT_E_HIP;
}

int vit_kv_transcode(const vit_kv_plane* src, const vit_kv_plane* dst, const int64_t* n_rows, void* stream) {
  const vit::KernelEvents ev = g_armed;  // one-shot: consumed by this call whatever its outcome
  g_armed = vit::KernelEvents{};
  int st = check_plane(src);
  if (st != VIT_OK) return st;
  st = check_plane(dst);
  if (st != VIT_OK) return st;
  if (!n_rows) return VIT_E_ARG;
  if (src->side != dst->side || src->n_seqs != dst->n_seqs || src->n_kv_heads != dst->n_kv_heads ||
      src->capacity != dst->capacity)
    return VIT_E_ARG;
  // the degrade steps: f16 -> q8_0 / q4_0 / rot4 / rot3, q8_0 -> q4_0 / rot4
  // / rot3, q4_0 -> rot3 (sources whose values decode exactly to fp32)
  const bool step = (src->codec == VIT_CODEC_F16 && dst->codec != VIT_CODEC_F16) ||
                    (src->codec == VIT_CODEC_Q8_0 && (dst->codec == VIT_CODEC_Q4_0 || is_rotated(dst->codec))) ||
                    (src->codec == VIT_CODEC_Q4_0 && dst->codec == VIT_CODEC_ROT3);
  if (!step) return VIT_E_UNSUPPORTED;
  if (planes_overlap(src, dst)) return VIT_E_ARG;  // the two planes' arrays must be disjoint
  int64_t max_rows = 0;
  for (int s = 0; s < src->n_seqs; ++s) {
    if (n_rows[s] < 0 || n_rows[s] > src->capacity) return VIT_E_CAPACITY;
    if (n_rows[s] > max_rows) max_rows = n_rows[s];
  }
  if (max_rows == 0) return VIT_OK;

  vit::TranscodeArgs a{};
  a.src_codes = static_cast<const uint8_t*>(src->codes);
  a.src_scales = src->scales;
  a.codes = dst->codes;
  a.scales = dst->scales;
  a.norms = dst->norms;
  a.capacity = dst->capacity;
  a.n_kv_heads = dst->n_kv_heads;
  load_signs(dst, a.signs);
  for (int s = 0; s < src->n_seqs; ++s) a.n_rows[s] = n_rows[s];
  const dim3 grid(static_cast<unsigned>((max_rows + 31) / 32), static_cast<unsigned>(dst->n_kv_heads),
                  static_cast<unsigned>(dst->n_seqs));
  return vit::launch_transcode(src->codec, dst->codec, dst->side, grid, static_cast<hipStream_t>(stream), a, ev) ==
                 hipSuccess
             ? VIT_OK
             : VIT_E_HIP;
}

int vit_vbr_classic_next_step(int32_t n_tensors, const int32_t* codecs, const int32_t* price_order,
                              const uint8_t* movable, double floor_bpv, int32_t* tensor, int32_t* new_codec) {
  if (n_tensors < 1 || !codecs || !price_order || !tensor || !new_codec) return VIT_E_ARG;
  // rung of each tensor on the ladder f16 (0) -> q8_0 (1) -> q4_0 (2)
  auto rung_of = [](int32_t c) { return c == VIT_CODEC_F16 ? 0 : c == VIT_CODEC_Q8_0 ? 1 : c == VIT_CODEC_Q4_0 ? 2 : -1; };
  static const int32_t kLadder[3] = {VIT_CODEC_F16, VIT_CODEC_Q8_0, VIT_CODEC_Q4_0};
  static const double kBpv[3] = {16.0, 8.5, 4.5};
  // every tensor on the ladder, and the price order a permutation of 0 .. n-1
  int top = 3;  // least degraded rung held by a movable tensor that can still move
  for (int32_t i = 0; i < n_tensors; ++i) {
    const int r = rung_of(codecs[i]);
    if (r < 0) return VIT_E_ARG;
    if ((!movable || movable[i]) && r < 2 && r < top) top = r;
  }
  for (int32_t k = 0; k < n_tensors; ++k) {  // each index in range and named once
    const int32_t i = price_order[k];
    if (i < 0 || i >= n_tensors) return VIT_E_ARG;
    for (int32_t m = 0; m < k; ++m)
      if (price_order[m] == i) return VIT_E_ARG;
  }
  *tensor = -1;
  *new_codec = -1;
  if (top == 3) return VIT_OK;  // every movable tensor is at q4_0
  for (int32_t k = 0; k < n_tensors; ++k) {
    const int32_t i = price_order[k];
    if ((movable && !movable[i]) || rung_of(codecs[i]) != top) continue;
    if (floor_bpv > 0.0) {
      // aggregate bits/value after the step, summed in tensor order
      double total = 0.0;
      for (int32_t j = 0; j < n_tensors; ++j) total += j == i ? kBpv[top + 1] : kBpv[rung_of(codecs[j])];
      if (total / n_tensors < floor_bpv) return VIT_OK;
    }
    *tensor = i;
    *new_codec = kLadder[top + 1];
    return VIT_OK;
  }
  return VIT_OK;
}

size_t vit_attn_probe_workspace_bytes(int32_t n_seqs, int32_t n_q_heads, int64_t capacity) {
  if (n_seqs < 1 || n_seqs > VIT_MAX_SEQS || n_q_heads < 1 || n_q_heads > vit::kProbeMaxHeads || capacity < 1 ||
      capacity > VIT_MAX_CAPACITY)
    return 0;
  const size_t logits = (static_cast<size_t>(n_seqs) * n_q_heads * capacity * sizeof(float) + 255) & ~size_t{255};
  return logits + static_cast<size_t>(n_seqs) * n_q_heads * vit::kProbeMaxChunks * 2 * sizeof(float);
}

int vit_attn_probe_scores(const vit_kv_plane* k, const float* q, int32_t n_q_heads, const int64_t* seq_len,
                          float scale, float decay, float* workspace, float* scores, void* stream) {
  const vit::KernelEvents ev = g_armed;  // one-shot: consumed by this call whatever its outcome
  g_armed = vit::KernelEvents{};
  int st = check_plane(k);
  if (st != VIT_OK) return st;
  if (k->side != VIT_SIDE_K) return VIT_E_ARG;
  if (!q || !seq_len || !workspace || !scores) return VIT_E_ARG;
  if (n_q_heads < 1 || n_q_heads % k->n_kv_heads != 0) return VIT_E_ARG;
  const int32_t gqa = n_q_heads / k->n_kv_heads;
  if (gqa > VIT_MAX_GQA || n_q_heads > vit::kProbeMaxHeads) return VIT_E_UNSUPPORTED;
  if (!isfinite(scale) || !isfinite(decay)) return VIT_E_ARG;
  int64_t max_len = 0;
  for (int s = 0; s < k->n_seqs; ++s) {
    if (seq_len[s] < 1) return VIT_E_ARG;
    if (seq_len[s] > k->capacity) return VIT_E_CAPACITY;
    if (seq_len[s] > max_len) max_len = seq_len[s];
  }
  if (!aligned(q, 16) || !aligned(workspace, 256) || !aligned(scores, 16)) return VIT_E_ALIGN;

  vit::ProbeArgs a{};
  a.kcodes = static_cast<const uint8_t*>(k->codes);
  a.kscales = k->scales;
  a.knorms = k->norms;
  a.q = q;
  a.logits = workspace;
  a.part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                    ((static_cast<size_t>(k->n_seqs) * n_q_heads * k->capacity * sizeof(float) + 255) &
                                     ~size_t{255}));
  a.scores = scores;
  a.capacity = k->capacity;
  a.n_kv_heads = k->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.gqa = gqa;
  // chunks per (sequence, KV head): about two 8-wave workgroups per compute
  // unit in all, at most one per tile
  const int64_t units = static_cast<int64_t>(k->n_seqs) * k->n_kv_heads;
  int64_t chunks = (512 + units - 1) / units;
  const int64_t tiles = (max_len + 31) / 32;
  if (chunks > tiles) chunks = tiles;
  if (chunks > vit::kProbeMaxChunks) chunks = vit::kProbeMaxChunks;
  a.n_chunks = static_cast<int32_t>(chunks < 1 ? 1 : chunks);
  a.qscale = scale * 1.4426950408889634f;
  a.decay = decay;
  load_signs(k, a.ksigns);
  for (int s = 0; s < k->n_seqs; ++s) a.seq_len[s] = static_cast<int32_t>(seq_len[s]);
  return vit::launch_probe(k->codec, k->n_seqs, static_cast<int>(max_len), static_cast<hipStream_t>(stream), a, ev) ==
                 hipSuccess
             ? VIT_OK
             : VIT_E_HIP;
}

size_t vit_probe_select_workspace_bytes(int32_t n_seqs) {
  if (n_seqs < 1 || n_seqs > VIT_MAX_SEQS) return 0;
  return static_cast<size_t>(n_seqs) * (3 * vit::kSelectBins + vit::kSelectMaxBlocks * 2) * sizeof(int32_t);
}

int vit_probe_select_evictions(const float* scores, int32_t n_seqs, int64_t capacity, const int64_t* seq_len,
                               int64_t n_sink, int64_t n_recent, int32_t n_evict, int64_t* rows_out, int32_t* n_out,
                               void* workspace, void* stream) {
  if (!scores || !seq_len || !n_out || !workspace) return VIT_E_ARG;
  if (n_seqs < 1 || capacity < 1 || n_sink < 0 || n_recent < 0 || n_evict < 0) return VIT_E_ARG;
  if (n_evict > 0 && !rows_out) return VIT_E_ARG;
  if (n_seqs > VIT_MAX_SEQS) return VIT_E_UNSUPPORTED;
  if (capacity > VIT_MAX_CAPACITY) return VIT_E_UNSUPPORTED;
  for (int s = 0; s < n_seqs; ++s)
    if (seq_len[s] < 0 || seq_len[s] > capacity) return VIT_E_CAPACITY;
  if (!aligned(scores, 4) || (rows_out && !aligned(rows_out, 8)) || !aligned(n_out, 4) || !aligned(workspace, 256))
    return VIT_E_ALIGN;
  vit::SelectArgs a{};
  a.scores = scores;
  a.rows_out = rows_out;
  a.n_out = n_out;
  a.hist = static_cast<int32_t*>(workspace);
  a.counts = a.hist + static_cast<size_t>(n_seqs) * 3 * vit::kSelectBins;
  a.capacity = capacity;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  a.n_evict = n_evict;
  a.n_seqs = n_seqs;
  int64_t max_mid = 0;  // middle cells of the longest middle range
  for (int s = 0; s < n_seqs; ++s) {
    a.seq_len[s] = seq_len[s];
    const int64_t lo = n_sink < seq_len[s] ? n_sink : seq_len[s];
    const int64_t hi = seq_len[s] - n_recent > lo ? seq_len[s] - n_recent : lo;
    if (hi - lo > max_mid) max_mid = hi - lo;
  }
  // blocks of >= 1024 cells (4 rounds of the workgroup's 256 threads in the
  // ordered write), at most kSelectMaxBlocks per sequence
  int64_t cpb = 1024;
  while ((max_mid + cpb - 1) / cpb > vit::kSelectMaxBlocks) cpb *= 2;
  const int64_t nb = (max_mid + cpb - 1) / cpb;
  a.cells_per_block = static_cast<int32_t>(cpb);
  a.n_blocks = static_cast<int32_t>(nb < 1 ? 1 : nb);
  a.max_mid = max_mid;
  return vit::launch_select(n_seqs, static_cast<hipStream_t>(stream), a) == hipSuccess ? VIT_OK : VIT_E_HIP;
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
  const vit::KernelEvents ev = vit::take_armed_events();  // one-shot, whatever the outcome
  const int st = vit::check_decode(k, v, q, n_q_heads, q_len, seq_len, k_new, v_new, scale, n_splits,
                                   workspace != nullptr, workspace, out);
  if (st != VIT_OK) return st;
  return vit::enqueue_decode(k, v, q, n_q_heads, q_len, seq_len, k_new, v_new, scale, n_splits, workspace, out,
                             nullptr, static_cast<hipStream_t>(stream), ev);
}

int vit_attn_decode_merged(const vit_kv_plane* k, const vit_kv_plane* v, const float* q, int32_t n_q_heads,
                           int32_t q_len, const int64_t* seq_len, const float* k_new, const float* v_new,
                           float scale, int32_t n_splits, float* workspace, uint32_t* counters, float* out,
                           void* stream) {
  const vit::KernelEvents ev = vit::take_armed_events();  // one-shot, whatever the outcome
  int st = vit::check_decode(k, v, q, n_q_heads, q_len, seq_len, k_new, v_new, scale, n_splits,
                             workspace != nullptr, workspace, out);
  if (st != VIT_OK) return st;
  if (n_splits > 1) {
    if (!counters) return VIT_E_ARG;
    if (!aligned(counters, 8)) return VIT_E_ALIGN;
    if (is_rotated(v->codec) && !v->signs) return VIT_E_ARG;
    const int32_t rows = (n_q_heads / k->n_kv_heads) * q_len;  // query rows per KV head
    if (n_splits > VIT_MERGE_MAX_SPLITS || rows * n_splits > VIT_MERGE_MAX_PARTIALS) return VIT_E_UNSUPPORTED;
  }
  return vit::enqueue_decode(k, v, q, n_q_heads, q_len, seq_len, k_new, v_new, scale, n_splits, workspace, out,
                             counters, static_cast<hipStream_t>(stream), ev);
}

int vit_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  const vit::KernelEvents ev = vit::take_armed_events();  // one-shot, whatever the outcome
  if (!buf || !sink || bytes == 0) return VIT_E_ARG;
  if (!aligned(buf, 16) || !aligned(sink, 4) || bytes % 16 != 0) return VIT_E_ALIGN;
  return vit::launch_stream_read(buf, static_cast<int64_t>(bytes / 16), sink, static_cast<hipStream_t>(stream), ev) ==
                 hipSuccess
             ? VIT_OK
             : VIT_E_HIP;
}

int vit_arm_kernel_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return VIT_E_ARG;
  g_armed.start = static_cast<hipEvent_t>(start_event);
  g_armed.stop = static_cast<hipEvent_t>(stop_event);
  return VIT_OK;
}

int vit_attn_splitk_reduce(const float* workspace, int32_t n_seqs, int32_t n_q_heads, int32_t head_dim,
                           int32_t n_splits, const vit_kv_plane* v, float* out, void* stream) {
  const int st = vit::check_reduce(workspace, n_seqs, n_q_heads, head_dim, n_splits, v, out);
  if (st != VIT_OK) return st;
  return vit::enqueue_reduce(workspace, n_seqs, n_q_heads, n_splits, v, out, static_cast<hipStream_t>(stream));
}

}  // extern "C"
