// Kernel argument blocks and launch entry points (host <-> kernels).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vit.h"

namespace vit {

constexpr int kMaxSeqs = 64;
constexpr int kAppendWaves = 4;  // append workgroup: one wave per 8-row group
constexpr int kDecodeWaves = 8;  // decode workgroup: one per compute unit

struct AppendArgs {
  void* codes;
  uint16_t* scales;
  uint16_t* norms;
  const float* src;
  int64_t capacity;
  int32_t n_kv_heads;
  int32_t n_tokens;
  uint32_t signs[4];
  int64_t pos0[kMaxSeqs];
};

// Several planes of one geometry appended in one launch (the same token
// range of each plane's own fp32 rows); each workgroup handles one plane.
constexpr int kMaxAppendPlanes = 32;
struct AppendPlane {
  void* codes;
  uint16_t* scales;
  uint16_t* norms;
  const float* src;   // [S][n_tokens][Hkv][128]
  int64_t capacity;
  int32_t codec_side;  // codec * 2 + side
  int32_t reserved;
  uint32_t signs[4];
};
struct AppendMultiArgs {
  AppendPlane planes[kMaxAppendPlanes];
  int64_t pos0[kMaxSeqs];
  int32_t n_kv_heads;
  int32_t n_tokens;
  int32_t n_seqs;
  int32_t n_planes;
};

// Re-encoding the rows a plane holds into a plane of another codec (same
// geometry and side).
struct TranscodeArgs {
  const uint8_t* src_codes;
  const uint16_t* src_scales;  // null for an f16 source
  void* codes;                 // destination plane
  uint16_t* scales;
  uint16_t* norms;
  int64_t capacity;
  int32_t n_kv_heads;
  uint32_t signs[4];           // destination signs (rot4)
  int64_t n_rows[kMaxSeqs];    // rows 0 .. n_rows[s]-1 of sequence s
};

// Attention-probe cell scores: per-cell logits of the current token's query
// rows and per-chunk softmax partials (probe_logits_kernel), then the per-cell
// mass with exponential decay (probe_mass_kernel).
constexpr int kProbeWaves = 8;
constexpr int kProbeMaxChunks = 64;
constexpr int kProbeMaxHeads = 256;  // n_q_heads
struct ProbeArgs {
  const uint8_t* kcodes;
  const uint16_t* kscales;
  const uint16_t* knorms;
  const float* q;        // [S][Hq][128]
  float* logits;         // [S][Hq][capacity], base-2 scaled
  float* part;           // [S][Hq][n_chunks][2]: (max, sum of 2^(logit - max))
  float* scores;         // [S][capacity]
  int64_t capacity;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t gqa;
  int32_t n_chunks;
  float qscale;          // softmax scale * log2(e)
  float decay;
  uint32_t ksigns[4];
  int32_t seq_len[kMaxSeqs];
};

// The cells to evict: a 3-pass radix select (11, 11, 10 bits) of the n_evict
// lowest (score, cell) keys among each sequence's middle cells, by blocks of
// cells_per_block cells, then their compaction in cell order.
// A longest middle range of at most kSelectSmallCells cells takes the
// one-workgroup-per-sequence form (keys in LDS, one launch).
constexpr int kSelectMaxBlocks = 256;     // blocks per sequence
constexpr int kSelectBins = 2048;         // bins of an 11-bit digit
constexpr int kSelectSmallCells = 8192;
struct SelectArgs {
  const float* scores;   // [S][capacity]
  int64_t* rows_out;     // [S][n_evict]
  int32_t* n_out;        // [S]
  int32_t* hist;         // [3][S][kSelectBins], zeroed by the first kernel
  int32_t* counts;       // [S][kSelectMaxBlocks][2]: block's cells below T, equal to T
  int64_t capacity;
  int64_t n_sink;
  int64_t n_recent;
  int32_t n_evict;
  int32_t n_seqs;
  int32_t cells_per_block;
  int32_t n_blocks;
  int64_t max_mid;       // middle cells of the longest middle range
  int64_t seq_len[kMaxSeqs];
};

struct DecodeArgs {
  const uint8_t* kcodes;
  const uint16_t* kscales;
  const uint16_t* knorms;
  const uint8_t* vcodes;
  const uint16_t* vscales;
  const uint16_t* vnorms;
  const float* q;
  const float* k_new;  // fused append: new K rows [S][q_len][Hkv][128] or null
  const float* v_new;
  float* ws_o;     // [S][q_len][Hq][n_splits][128]
  float* ws_ml;    // [S][q_len][Hq][n_splits][2]
  float* out;      // [S][q_len][Hq][128]
  uint32_t* arrive;  // in-kernel split merge: arrival counts [S][Hkv] (0 between calls), or null
  int64_t capacity;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t gqa;
  int32_t q_len;   // new query tokens per sequence (causal among themselves)
  int32_t n_splits;
  float qscale;    // softmax scale * log2(e)
  uint32_t ksigns[4];
  uint32_t vsigns[4];
  int32_t seq_len[kMaxSeqs];
};

struct ReduceArgs {
  const float* ws_o;
  const float* ws_ml;
  float* out;
  int32_t n_q_heads;
  int32_t n_splits;
  int32_t rotate;  // 1: V codec is rot4, rotate the merged row back
  uint32_t vsigns[4];
};

// Optional events recorded by a kernel's dispatch itself (kernel start and
// end, via hipExtLaunchKernel); null members record nothing.
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

hipError_t launch_append(int codec, int side, dim3 grid, hipStream_t stream, const AppendArgs& args,
                         const KernelEvents& ev);
hipError_t launch_transcode(int src_codec, int dst_codec, int side, dim3 grid, hipStream_t stream,
                            const TranscodeArgs& args, const KernelEvents& ev);
hipError_t launch_decode(int kc, int vc, int nt, dim3 grid, hipStream_t stream, const DecodeArgs& args,
                         const KernelEvents& ev);
hipError_t launch_decode_k0(int vc, int nt, dim3 grid, hipStream_t stream, const DecodeArgs& args, const KernelEvents& ev);
hipError_t launch_decode_k1(int vc, int nt, dim3 grid, hipStream_t stream, const DecodeArgs& args, const KernelEvents& ev);
hipError_t launch_decode_k2(int vc, int nt, dim3 grid, hipStream_t stream, const DecodeArgs& args, const KernelEvents& ev);
hipError_t launch_decode_k3(int vc, int nt, dim3 grid, hipStream_t stream, const DecodeArgs& args, const KernelEvents& ev);
hipError_t launch_decode_k4(int vc, int nt, dim3 grid, hipStream_t stream, const DecodeArgs& args, const KernelEvents& ev);
hipError_t launch_reduce(dim3 grid, hipStream_t stream, const ReduceArgs& args);
hipError_t launch_append_multi(dim3 grid, hipStream_t stream, const AppendMultiArgs& args, const KernelEvents& ev);
hipError_t launch_stream_read(const void* buf, int64_t n16, uint32_t* sink, hipStream_t stream,
                              const KernelEvents& ev);
// both probe kernels (logits over grid (n_chunks, Hkv, S), then the mass);
// ev brackets the logits kernel
hipError_t launch_probe(int kc, int n_seqs, int max_seq_len, hipStream_t stream, const ProbeArgs& args,
                        const KernelEvents& ev);
hipError_t launch_select(int n_seqs, hipStream_t stream, const SelectArgs& args);

// Host-side pieces of the decode and reduce entry points (vit_host.cpp),
// shared with the entry point that keeps the split partials in static device
// memory (noalloc.hip).
KernelEvents take_armed_events();  // this thread's armed events, disarming them
int check_decode(const vit_kv_plane* k, const vit_kv_plane* v, const float* q, int32_t n_q_heads, int32_t q_len,
                 const int64_t* seq_len, const float* k_new, const float* v_new, float scale, int32_t n_splits,
                 bool have_workspace, const void* workspace, const float* out);
int enqueue_decode(const vit_kv_plane* k, const vit_kv_plane* v, const float* q, int32_t n_q_heads, int32_t q_len,
                   const int64_t* seq_len, const float* k_new, const float* v_new, float scale, int32_t n_splits,
                   float* workspace, float* out, uint32_t* arrive, hipStream_t stream, const KernelEvents& ev);
int check_reduce(const float* workspace, int32_t n_seqs, int32_t n_q_heads, int32_t head_dim, int32_t n_splits,
                 const vit_kv_plane* v, const float* out);
int enqueue_reduce(const float* workspace, int32_t n_seqs, int32_t n_q_heads, int32_t n_splits,
                   const vit_kv_plane* v, float* out, hipStream_t stream);

}  // namespace vit
