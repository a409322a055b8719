/*
 * vit.h -- quantized KV-cache append and flash-decode attention for MI355X
 * (gfx950).  C ABI: plain pointers and sizes, no C++ or torch types.
 *
 * What the calls compute.  A decoder layer keeps, per (layer, side), one KV
 * cache tensor whose codec is chosen per side and per layer: the per-side
 * cache types (--cache-type-k / --cache-type-v) of the Randozart/VITRIOL page
 * ("Configuration" flag table) and the per-(layer, side) degrade ladder of
 * the buun-llama-cpp page ("VBR -- Variable Bit-Rate KV Cache").  Codecs:
 * f16, q8_0 and q4_0 with 32-value blocks (buun-llama-cpp page, "Codecs"
 * table), rot4, a Walsh-Hadamard-rotated 4-bit scalar codec (same table's
 * rotated "turbo4" row; step 1 of its "How it works" list), and rot3, its
 * 3-bit, 3.5 bits/value sibling (the "tq3_0" class of the Randozart/VITRIOL
 * page's "What sets VITRIOL apart" table, the buun-llama-cpp page's "turbo3").  Decode is
 * flash attention only (buun-llama-cpp page, "Requirements" paragraph), for
 * grouped-query heads, over a context whose per-sequence capacity is a
 * multiple of 256 (serverAppConfigs commit log, tests/frank_small_unit.bats
 * page: the 200,704-token slots "256-aligned for the FA path").
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked [host].  The library never
 *    allocates or frees device memory; the caller owns every buffer.  (The
 *    one exception is the static scratch array of vit_attn_decode_noalloc,
 *    part of the library's code object on each GPU.)
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without synchronising.
 *  - Arguments are validated on the host before anything is enqueued.  On a
 *    failed validation the call returns a negative vit_status and enqueues
 *    nothing.  After a launch, a HIP launch error maps to VIT_E_HIP.  Faults
 *    inside kernels surface at the caller's next synchronisation.
 *  - The library keeps no state between calls and is re-entrant (except
 *    vit_attn_decode_noalloc's per-GPU scratch, see there).  Two calls that
 *    write the same cache rows must not run concurrently.
 *  - head_dim must be 128.  Capacity must be a multiple of 256.  At most 64
 *    sequences per call; query heads per KV head (G) at most 16.
 *
 * ------------------------------------------------------------------------
 * Codecs (per 128-value row x of one (token, KV head); blocks of 32).
 *  F16   code_j = fp16(x_j) (round to nearest even).
 *  Q8_0  d = max|x| / 127 (fp32);  c_j = clamp(round_half_away(x_j / d), +-127)
 *        computed as x_j * (1/d) in fp32;  scale = fp16(d).
 *  Q4_0  m = the first x_j of largest magnitude; d = m / -8 (+0.0 if m == 0);
 *        c_j = clamp(round_half_away(x_j * (1/d)) + 8, 0, 15);  scale = fp16(d).
 *  ROT4  y = WHT(s .* x) (signs from the 16-byte mask, unnormalised Sylvester
 *        transform, stages h = 1..64); n = ||x||_2 (stride-halving fp32 sum);
 *        u = y / n; per block b: r_b = sqrt(mean(u_j^2)); t_j = u_j / r_b;
 *        idx_j = number of the 15 thresholds below t_j (a value equal to a
 *        threshold goes to the level farther from zero; 0 -> 8);
 *        norm = fp16(n), scale_b = fp16(r_b).  Levels: the 16-level
 *        Lloyd-Max quantizer for N(0,1), stored as fp16; thresholds are the
 *        midpoints of adjacent levels.  Reconstruction in the rotated domain
 *        is norm * scale_b * level[idx_j] / sqrt(128); the model-domain row is
 *        s .* (WHT(that) / sqrt(128)).
 *  ROT3  y = WHT(s .* x) as ROT4; per block b: r_b = sqrt(mean(y_j^2))
 *        (stride-halving fp32 sum, then * (1/32)); t_j = y_j * (1 / r_b);
 *        idx_j = number of the 7 thresholds below t_j (ties go to the level
 *        farther from zero; 0 -> 4); scale_b = fp16(r_b); no norm.  Levels:
 *        the 8-level Lloyd-Max quantizer for N(0,1) as fp16.  Reconstruction
 *        in the rotated domain is scale_b * level[idx_j] / sqrt(128).
 *
 * ------------------------------------------------------------------------
 * Physical layout of one cache plane (one (layer, side) tensor).
 * Rows of a (sequence, KV head) form a stream of `capacity` rows stored as
 * tiles of 32 positions; plane index ph = seq * n_kv_heads + head.
 *
 *  codes   ph * capacity * RB bytes per stream, RB = 256 (F16), 128 (Q8_0),
 *          64 (Q4_0, ROT4), 48 (ROT3) bytes per row; a tile is 32 * RB bytes.
 *  scales  fp16, 4 per row (one per 32-value block); NULL for F16.
 *          K side: [S][H][capacity][4] (row-major);  V side:
 *          [S][H][capacity/32][4][32], scale of (tile t, block b, row p) at
 *          ((ph * capacity/32 + t) * 4 + b) * 32 + p.
 *  norms   fp16 [S][H][capacity] (ROT4 only; NULL otherwise).
 *
 *  A K-side tile ("row-major units") is two 16-row halves h = 0, 1; row r of
 *  half h is position p = 16*h + r.  The canonical bytes of block b of a row
 *  (RB/4 of them) are:  F16: fp16 of channels 32b .. 32b+31;  Q8_0: int8
 *  codes of channels 32b .. 32b+31;  Q4_0/ROT4: byte j (< 16) =
 *  code[32b+j] | code[32b+j+16] << 4.  Chunk g (0..3) of a block is its
 *  canonical bytes [g*CHB, (g+1)*CHB), CHB = RB/16.  Each half holds 16-byte
 *  units U[c][g][r] (c < CB = RB/64, r = row 0..15), unit byte offset
 *  (((h*CB + c)*4 + g)*16 + r)*16; unit U[c][g][r] holds chunk g of blocks
 *  c*BPU .. c*BPU+BPU-1 of row r in block order, BPU = 4/CB (F16: 1 block,
 *  16 B; Q8_0: 2 blocks, 8 B each; Q4_0/ROT4: 4 blocks, 4 B each).
 *  ROT3 K tiles use 12-byte units instead: unit (h, g, r) at byte
 *  ((h*4 + g)*16 + r)*12 holds, for b = 0..3 at bytes 3b .. 3b+2, the 24-bit
 *  group of channels 32b + 8g + j (j < 8), code j at bits 3j.
 *  A V-side tile ("column units") stores, for each channel ch (N-tile
 *  nt = ch>>4, n = ch&15) and each group of 8 positions g8 = p>>3, the 8
 *  codes of positions 8*g8 .. 8*g8+7 of that channel:
 *    F16 : 16 B at ((nt*4 + g8)*16 + n)*16, fp16 of position 8*g8+j at 2*j;
 *    Q8_0: 8 B at ((nt>>1)*4 + g8)*16 + n)*16 + 8*(nt&1), position j at byte
 *          P8[j], P8 = {0,2,1,3,4,6,5,7};
 *    Q4_0: 4 B at ((nt>>2)*4 + g8)*16 + n)*16 + 4*(nt&3), position j in byte
 *          Q4B[j] = {0,2,1,3,0,2,1,3}[j], low nibble for j < 4, high for j >= 4;
 *    ROT4: 4 B as Q4_0, position j in byte j>>1, low nibble for even j;
 *    ROT3: 24 bits at byte (((ch>>6)*4 + g8)*16 + n)*12 + 3*((ch>>4)&3)
 *          (12-byte units of 4 channels), position j at bits 3j.
 *  K and V planes of the same codec differ only in this code layout (the
 *  plane's side field); their sizes are equal.
 *
 * Input domain of the encoders: finite values; a nonzero 32-value block has
 * largest magnitude >= 2^-100 (so the fp32 reciprocal of its scale is finite);
 * stored fp16 scales and norms stay below 65504.  Outside it the codes are
 * deterministic but unspecified.
 *
 * Sign mask (ROT4, ROT3): 16 bytes, bit (j & 7) of byte (j >> 3) set =>
 * channel j is negated before the transform.  One mask per (layer, side).
 */
#ifndef VIT_H
#define VIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vit_codec {
  VIT_CODEC_F16 = 0,
  VIT_CODEC_Q8_0 = 1,
  VIT_CODEC_Q4_0 = 2,
  VIT_CODEC_ROT4 = 3,
  VIT_CODEC_ROT3 = 4
} vit_codec;

typedef enum vit_side { VIT_SIDE_K = 0, VIT_SIDE_V = 1 } vit_side;

typedef enum vit_status {
  VIT_OK = 0,
  VIT_E_ARG = -1,         /* bad value, NULL required pointer, k_new xor v_new */
  VIT_E_UNSUPPORTED = -2, /* head_dim != 128, G > 16, > 64 sequences, unknown codec,
                             capacity > VIT_MAX_CAPACITY */
  VIT_E_CAPACITY = -3,    /* rows outside 0..capacity-1, capacity % 256 != 0 */
  VIT_E_ALIGN = -4,       /* plane pointer not 256-B aligned, other pointer not 16-B aligned */
  VIT_E_HIP = -5,         /* a HIP launch failed */
  VIT_E_SCRATCH = -6      /* vit_attn_decode_noalloc: split partials larger than its static scratch */
} vit_status;

#define VIT_HEAD_DIM 128
#define VIT_CAPACITY_ALIGN 256
#define VIT_MAX_SEQS 64
#define VIT_MAX_GQA 16 /* query rows per KV head: G, or G * q_len for vit_attn_decode_mq */
#define VIT_MAX_QLEN 4 /* new tokens per sequence in one vit_attn_decode_mq call */
#define VIT_MAX_SPLITS 4096
#define VIT_MERGE_MAX_SPLITS 64    /* vit_attn_decode_merged: split count */
#define VIT_MAX_APPEND_PLANES 32   /* vit_kv_append_quant_multi: planes per call */
#define VIT_MERGE_MAX_PARTIALS 128 /* vit_attn_decode_merged: query rows per KV head x splits */
#define VIT_MAX_CAPACITY (1 << 30) /* rows per (sequence, KV head) */

/* One (layer, side) cache tensor: caller-owned device memory in the layout
 * above.  `signs` is a [host] pointer to 16 bytes (ROT4 and ROT3, else NULL),
 * read during the call. */
typedef struct vit_kv_plane {
  int32_t codec;       /* vit_codec */
  int32_t side;        /* vit_side: selects the K or V code layout */
  int32_t n_seqs;
  int32_t n_kv_heads;
  int32_t head_dim;    /* must be 128 */
  int32_t reserved;    /* must be 0 */
  int64_t capacity;    /* rows per (sequence, KV head); multiple of 256, <= VIT_MAX_CAPACITY */
  void *codes;
  uint16_t *scales;    /* fp16 bits; NULL for F16 */
  uint16_t *norms;     /* fp16 bits; ROT4 only, else NULL */
  const uint8_t *signs;/* [host] 16 bytes; ROT4 and ROT3 only, else NULL */
} vit_kv_plane;

/* Byte sizes of the three arrays of a plane (host only, no device work):
 * bits per value 16 (f16), 8.5 (q8_0), 4.5 (q4_0) as in the buun-llama-cpp
 * page's "Codecs" table, 4.625 (rot4: codes, block scales and a row norm) and
 * 3.5 (rot3, the Randozart/VITRIOL page's tq3_0 size in "What sets VITRIOL
 * apart"); capacity a multiple of 256 (serverAppConfigs commit log,
 * "CTX_SIZE 540672 -> 401408" commit: slots aligned to 256 for the FA path).
 * Returns VIT_OK or a negative status; any out pointer may be NULL. */
int vit_kv_plane_sizes(int32_t codec, int32_t n_seqs, int32_t n_kv_heads, int32_t head_dim,
                       int64_t capacity, size_t *codes_bytes, size_t *scales_bytes,
                       size_t *norms_bytes);

/* Quantize new K or V rows and store them in a plane (the append of a
 * ubatch of new tokens: buun-llama-cpp page, "Codecs" table for the codecs;
 * serverAppConfigs commit log for ubatch <= batch and the 2048-row ubatch).
 *  src     fp32 [n_seqs][n_tokens][n_kv_heads][128], 16-B aligned.
 *  pos0    [host] int64 [n_seqs]: row of token 0 of each sequence; rows
 *          pos0[s] .. pos0[s]+n_tokens-1 are written (VIT_E_CAPACITY if any
 *          lies outside 0..capacity-1).  n_tokens == 0 is a no-op.
 * Codes and fp16 scales are bit-exact with the codec definitions above.
 * Rows not in the range are left untouched. */
int vit_kv_append_quant(const vit_kv_plane *dst, const float *src, const int64_t *pos0,
                        int32_t n_tokens, void *stream);

/* The same append for several planes in one launch: rows pos0[s] ..
 * pos0[s]+n_tokens-1 of each sequence s of every plane i, from src[i] (the
 * ubatch appended to every (layer, side) tensor of a step: serverAppConfigs
 * commit log, "BATCH_SIZE 2048 -> 4096, UBATCH_SIZE 1024 -> 2048" commit;
 * the per-(layer, side) codecs of the buun-llama-cpp page's "VBR" section).
 * Each plane is written exactly as vit_kv_append_quant(&planes[i], src[i],
 * pos0, n_tokens) would write it; one launch pays the fixed start cost once.
 *  planes   [host] n_planes planes (any codecs and sides) with equal n_seqs
 *           and n_kv_heads; the arrays of no two planes overlap.
 *  src      [host] n_planes device pointers, each fp32
 *           [n_seqs][n_tokens][n_kv_heads][128], 16-B aligned.
 *  n_planes 1 .. VIT_MAX_APPEND_PLANES.
 * Errors as vit_kv_append_quant (any plane); mismatched geometry or arrays
 * of two planes that overlap is VIT_E_ARG, n_planes outside 1..VIT_MAX_APPEND_PLANES is
 * VIT_E_UNSUPPORTED.  Kernel events armed by vit_arm_kernel_events bracket
 * its one kernel. */
int vit_kv_append_quant_multi(const vit_kv_plane *planes, int32_t n_planes, const float *const *src,
                              const int64_t *pos0, int32_t n_tokens, void *stream);

/* One degrade step of a variable bit-rate cache: re-encode the rows one
 * (layer, side) tensor holds into a plane of a codec with fewer bits per
 * value (buun-llama-cpp page, "VBR -- Variable Bit-Rate KV Cache": the cache
 * starts at f16 and moves one (layer, side) tensor at a time down a ladder;
 * the classic ladder is f16 -> q8_0 -> q4_0).  Each stored row of `src` is
 * decoded to its values, which are exact in fp32 for these sources (an fp16
 * value, or an int8 / 4-bit code times its fp16 scale), and encoded into the
 * same row of `dst` exactly as vit_kv_append_quant would encode those values
 * (so codes, scales and norms are bit-exact with the codec definitions).
 *  src, dst  planes with equal side, n_seqs, n_kv_heads and capacity, whose
 *            arrays do not overlap (VIT_E_ARG).  The codec pair is one of
 *            f16 -> q8_0, q4_0, rot4 or rot3; q8_0 -> q4_0, rot4 or rot3;
 *            q4_0 -> rot3 (rot4 and rot3 being the rotated 4-bit and 3-bit
 *            rungs); any other pair is VIT_E_UNSUPPORTED.
 *  n_rows    [host] int64 [n_seqs]: rows 0 .. n_rows[s]-1 of every KV head of
 *            sequence s are re-encoded, 0 <= n_rows[s] <= capacity
 *            (VIT_E_CAPACITY otherwise).  Rows of dst past them are left
 *            untouched; src is only read.
 * The caller then uses dst in place of src and may free src: the peak extra
 * memory of a step is one destination plane. */
int vit_kv_transcode(const vit_kv_plane *src, const vit_kv_plane *dst, const int64_t *n_rows,
                     void *stream);

/* Host only: the next step of the classic ladder f16 -> q8_0 -> q4_0 (same
 * page and section).  The classic order moves tensors band by band: no tensor
 * goes from q8_0 to q4_0 while a movable tensor is still at f16.  A side
 * pinned to a fixed type never moves, and no step is taken that would bring
 * the aggregate bits/value below the floor.
 *  codecs       [host] int32 [n_tensors]: each tensor's codec, f16, q8_0 or
 *               q4_0 (VIT_E_ARG otherwise); tensors are equally sized.
 *  price_order  [host] int32 [n_tensors]: tensor indices, cheapest to degrade
 *               first (a permutation of 0 .. n_tensors-1, else VIT_E_ARG).
 *  movable      [host] uint8 [n_tensors] or NULL (all movable): 0 = pinned.
 *  floor_bpv    minimum aggregate bits/value after the step (mean of 16, 8.5
 *               and 4.5 over the tensors); <= 0 means no floor.
 * On VIT_OK, *tensor / *new_codec name the step: among the movable tensors on
 * the least degraded rung that can still move, the first in price order moves
 * one rung down; *tensor = -1 when no step is left. */
int vit_vbr_classic_next_step(int32_t n_tensors, const int32_t *codecs, const int32_t *price_order,
                              const uint8_t *movable, double floor_bpv, int32_t *tensor,
                              int32_t *new_codec);

/* Workspace bytes vit_attn_decode needs for n_splits > 1 (the split-K
 * partials of the flash-decode path the buun-llama-cpp page's
 * "Requirements" paragraph requires): fp32 partial outputs
 * [S][Hq][n_splits][128] (256-byte padded) followed by (max, sum) pairs
 * [S][Hq][n_splits][2].  Returns 0 for invalid sizes. */
size_t vit_attn_workspace_bytes(int32_t n_seqs, int32_t n_q_heads, int32_t head_dim,
                                int32_t n_splits);

/* A split count that fills the GPU for this shape (host heuristic). */
int32_t vit_attn_default_splits(int32_t n_seqs, int32_t n_kv_heads, int32_t n_q_heads,
                                int64_t max_seq_len);

/* Decode attention for one new query token per sequence over rows
 * 0 .. seq_len[s]-1 of its KV head (grouped-query: kv_head = q_head / G,
 * G = n_q_heads / n_kv_heads), dequantizing K and V on the fly: flash
 * attention over a quantized KV cache (buun-llama-cpp page, "Requirements"
 * paragraph: quantized KV needs the flash-attention path; "Codecs" table for
 * the per-side codecs; Randozart/VITRIOL page, "Configuration" table for
 * separate K and V cache types).
 *  k, v      planes with equal n_seqs, n_kv_heads, capacity; sides K and V.
 *  q         fp32 [n_seqs][n_q_heads][128] in the model domain.
 *  seq_len   [host] int64 [n_seqs], 1 .. capacity, counting the new row.
 *  k_new, v_new  optional fp32 [n_seqs][n_kv_heads][128]: when given (both or
 *            neither), the new token's K and V rows are quantized and stored
 *            at row seq_len[s]-1 first, exactly as vit_kv_append_quant would.
 *  scale     softmax scale (typically 1/sqrt(128)).
 *  n_splits  1 .. VIT_MAX_SPLITS.  The 32-row tiles of each sequence's
 *            context are dealt to n_splits partial results in contiguous
 *            runs of ceil(tiles / n_splits) tiles (the last splits may get
 *            fewer or none).  With n_splits == 1 the
 *            normalised output is written to
 *            `out` and `workspace` may be NULL; otherwise partials go to
 *            `workspace` and vit_attn_splitk_reduce produces `out`.
 *  out       fp32 [n_seqs][n_q_heads][128], model domain.
 * The result equals softmax(scale * q K^T) V over the dequantized rows to
 * fp32 accumulation accuracy.  It is bitwise repeatable for the same inputs
 * and split count (the summation order is fixed); it is not bitwise across
 * split counts. */
int vit_attn_decode(const vit_kv_plane *k, const vit_kv_plane *v, const float *q,
                    int32_t n_q_heads, const int64_t *seq_len, const float *k_new,
                    const float *v_new, float scale, int32_t n_splits, float *workspace,
                    float *out, void *stream);

/* Decode attention for q_len new query tokens per sequence at once, causal
 * among themselves, as when a run of drafted tokens is verified in one pass
 * (Randozart/VITRIOL page: "How It Works -- Resident mode" drafts ahead with
 * parallel verification; "Configuration" runs up to 3 drafted tokens).
 * Token t (0 .. q_len-1) of sequence s attends rows
 * 0 .. seq_len[s] - q_len + t, i.e. the cached rows and the new rows up to
 * and including its own.  vit_attn_decode is the q_len == 1 case.
 *  q         fp32 [n_seqs][q_len][n_q_heads][128], model domain.
 *  q_len     1 .. VIT_MAX_QLEN, with G * q_len <= VIT_MAX_GQA.
 *  seq_len   [host] int64 [n_seqs], q_len .. capacity: rows attended by the
 *            last new token (the q_len new rows are its last rows).
 *  k_new, v_new  optional fp32 [n_seqs][q_len][n_kv_heads][128], stored at
 *            rows seq_len[s] - q_len + t first (both or neither).
 *  workspace vit_attn_workspace_bytes(n_seqs, n_q_heads * q_len, 128,
 *            n_splits) bytes; merge with vit_attn_splitk_reduce(workspace,
 *            n_seqs, n_q_heads * q_len, 128, n_splits, v, out).
 *  out       fp32 [n_seqs][q_len][n_q_heads][128].
 * Other arguments, errors and accuracy as vit_attn_decode; seq_len[s] <
 * q_len is VIT_E_ARG, q_len > VIT_MAX_QLEN or G * q_len > VIT_MAX_GQA is
 * VIT_E_UNSUPPORTED. */
int vit_attn_decode_mq(const vit_kv_plane *k, const vit_kv_plane *v, const float *q,
                       int32_t n_q_heads, int32_t q_len, const int64_t *seq_len,
                       const float *k_new, const float *v_new, float scale, int32_t n_splits,
                       float *workspace, float *out, void *stream);

/* Merge the split partials of vit_attn_decode (the second pass of the
 * split-K flash decode): M = max m_s, L = sum l_s 2^(m_s - M),
 * O = sum o_s 2^(m_s - M) / L (max values are kept in base-2 units); for a
 * ROT4 or ROT3 V plane the merged row is rotated back to the model domain
 * with v's sign mask (x = s .* WHT(o) / 128; buun-llama-cpp page, "How it
 * works", step 1: the rotation is an orthogonal transform after sign flips).
 * `v` is read only for its codec and signs.  Empty partials (l_s = 0) are
 * skipped.
 *  out  fp32 [n_seqs][n_q_heads][128]. */
int vit_attn_splitk_reduce(const float *workspace, int32_t n_seqs, int32_t n_q_heads,
                           int32_t head_dim, int32_t n_splits, const vit_kv_plane *v,
                           float *out, void *stream);

/* Decode attention (vit_attn_decode_mq) and its split merge
 * (vit_attn_splitk_reduce) in one launch: the flash decode over the quantized
 * cache (buun-llama-cpp page, "Requirements" paragraph; per-side codecs of
 * its "Codecs" table) without the second pass's launch.  Each split's
 * workgroup writes its partial as before; the last of a (sequence, KV head)'s
 * workgroups to finish merges that head's partials with the arithmetic of
 * vit_attn_splitk_reduce, so `out` equals the two-call result bit for bit.
 *  workspace  as vit_attn_decode_mq: vit_attn_workspace_bytes(n_seqs,
 *             n_q_heads * q_len, 128, n_splits) bytes.  The partials stay in
 *             it (vit_attn_splitk_reduce may still be called on them).
 *  counters   device uint32 [n_seqs][n_kv_heads], 8-B aligned: arrival
 *             counts, which must all be zero before the first call (one
 *             hipMemset when they are allocated); every call leaves them 0.
 *  Limits: n_splits <= VIT_MERGE_MAX_SPLITS and (n_q_heads / n_kv_heads) *
 *  q_len * n_splits <= VIT_MERGE_MAX_PARTIALS (the partial rows the merging
 *  workgroup reads); beyond them VIT_E_UNSUPPORTED: use the two calls.  With
 *  n_splits == 1 this is vit_attn_decode_mq (workspace, counters may be NULL).
 * Calls that share counters or a workspace and may run at the same time race.
 * Other arguments, errors and accuracy as vit_attn_decode_mq; NULL counters
 * with n_splits > 1 is VIT_E_ARG. */
int vit_attn_decode_merged(const vit_kv_plane *k, const vit_kv_plane *v, const float *q,
                           int32_t n_q_heads, int32_t q_len, const int64_t *seq_len,
                           const float *k_new, const float *v_new, float scale, int32_t n_splits,
                           float *workspace, uint32_t *counters, float *out, void *stream);

/* Workspace bytes of vit_attn_probe_scores: fp32 logits [n_seqs][n_q_heads]
 * [capacity] (256-byte padded) followed by softmax partials [n_seqs]
 * [n_q_heads][64][2].  Returns 0 for invalid sizes (n_q_heads up to 256). */
size_t vit_attn_probe_workspace_bytes(int32_t n_seqs, int32_t n_q_heads, int64_t capacity);

/* Attention-probe cell scores for sparse KV eviction (Randozart/VITRIOL page:
 * "What sets VITRIOL apart" -- an attention probe ranks the cache cells for
 * eviction, with the first and the latest cells kept; "How It Works --
 * Resident mode" -- a probe graph of a q.K softmax with exponential decay,
 * run every 16 steps; draft tokens are left out).  For every sequence s and every query head, the softmax of
 * scale * q . k over its KV head's cells 0 .. seq_len[s]-1 (keys dequantized
 * on the fly, as decode does) gives one probability per cell; a cell is a
 * token position holding every KV head, so its mass is the sum over all
 * n_q_heads query heads (a sequence's masses sum to n_q_heads).  Then
 *     scores[s][j] = decay * scores[s][j] + mass[s][j]   for j < seq_len[s];
 * cells at or past seq_len[s] are not touched.  The cadence of scoring events
 * is the caller's; for several layers in one event, pass the decay with the
 * first and 1 with the others.
 *  k          a K-side plane (any codec).
 *  q          fp32 [n_seqs][n_q_heads][128]: the current token's query rows,
 *             model domain, 16-B aligned; G = n_q_heads / n_kv_heads <= 16.
 *  seq_len    [host] int64 [n_seqs], 1 .. capacity.
 *  workspace  vit_attn_probe_workspace_bytes(n_seqs, n_q_heads, capacity)
 *             bytes, 256-B aligned.
 *  scores     fp32 [n_seqs][capacity], in/out, 16-B aligned.
 * The masses equal the fp64 definition to fp32 accumulation accuracy. */
int vit_attn_probe_scores(const vit_kv_plane *k, const float *q, int32_t n_q_heads, const int64_t *seq_len,
                          float scale, float decay, float *workspace, float *scores, void *stream);

/* The cells to evict (same page and sections: the middle cells with the
 * lowest scores are evicted first; the first (sink) and the latest cells are
 * never chosen).  For each sequence s, the
 * middle cells are n_sink <= j < seq_len[s] - n_recent; the n_evict lowest
 * (score, cell) pairs among them (equal scores: lower cell first, so the
 * choice is unique) are written in increasing cell order.
 *  scores     fp32 [n_seqs][capacity] (device), e.g. from vit_attn_probe_scores.
 *  seq_len    [host] int64 [n_seqs], 0 .. capacity.
 *  n_sink, n_recent, n_evict  >= 0.
 *  rows_out   int64 [n_seqs][n_evict] (device): the chosen cells, then -1.
 *  n_out      int32 [n_seqs] (device): how many were chosen,
 *             min(n_evict, middle cells).
 *  workspace  vit_probe_select_workspace_bytes(n_seqs) bytes (device).
 * Scores are finite (NaN is outside the domain); -0 and +0 are equal. */
int vit_probe_select_evictions(const float *scores, int32_t n_seqs, int64_t capacity, const int64_t *seq_len,
                               int64_t n_sink, int64_t n_recent, int32_t n_evict, int64_t *rows_out,
                               int32_t *n_out, void *workspace, void *stream);

/* Workspace bytes of vit_probe_select_evictions (radix histograms and block
 * counts; 256-B aligned; no state is kept between calls).  0 for invalid
 * n_seqs. */
size_t vit_probe_select_workspace_bytes(int32_t n_seqs);

/* Bytes of device memory vit_attn_decode_noalloc holds for split partials
 * on every GPU it runs on (a file-scope static array, kept until the process
 * ends). */
#define VIT_NOALLOC_SCRATCH_BYTES (4u << 20)

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * result as vit_attn_decode_mq followed, when n_splits > 1, by
 * vit_attn_splitk_reduce into `out`, with the split partials kept in a
 * static device array of VIT_NOALLOC_SCRATCH_BYTES bytes instead of a
 * caller's workspace.  The call allocates and frees nothing; the array is
 * the library's, one per GPU, held until the process ends.  Its device
 * address is looked up once per GPU, on the first call made with that GPU
 * current.
 *  Arguments as vit_attn_decode_mq (q, out fp32 [n_seqs][q_len][n_q_heads]
 *  [128]); there is no workspace argument.
 *  Errors: those of vit_attn_decode_mq; VIT_E_SCRATCH when
 *  vit_attn_workspace_bytes(n_seqs, n_q_heads * q_len, 128, n_splits) >
 *  VIT_NOALLOC_SCRATCH_BYTES (checked on the host before anything is
 *  enqueued); VIT_E_HIP if the array's address cannot be obtained.
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents: calls that may overlap on one GPU (different streams, or
 * host threads, without an order between them) race on it and may return
 * wrong results.  Nothing in it needs clearing: the decode writes every
 * partial the merge reads.  Kernel events armed by vit_arm_kernel_events
 * bracket the decode kernel of this call. */
int vit_attn_decode_noalloc(const vit_kv_plane *k, const vit_kv_plane *v, const float *q,
                            int32_t n_q_heads, int32_t q_len, const int64_t *seq_len,
                            const float *k_new, const float *v_new, float scale, int32_t n_splits,
                            float *out, void *stream);

/* Measurement aid (no operation of the method): arm two caller-created
 * hipEvent_t handles (timing enabled) so that the kernel of this host
 * thread's next vit_kv_append_quant, vit_kv_append_quant_multi, vit_attn_decode, vit_attn_decode_mq,
 * vit_attn_decode_merged, vit_attn_decode_noalloc, vit_kv_transcode, vit_stream_read or vit_attn_probe_scores call (for the latter: its
 * logits kernel)
 * records `start_event` when its dispatch begins and `stop_event` when it
 * ends (hipExtLaunchKernel), i.e. the pair brackets that one kernel and
 * nothing else.  One-shot: that next call consumes the arming whether or
 * not it launches.
 * Both NULL disarms; exactly one NULL returns VIT_E_ARG.  The events stay
 * owned by the caller. */
int vit_arm_kernel_events(void *start_event, void *stop_event);

/* Measurement aid (no operation of the method): read `bytes` bytes of `buf`
 * (device, 16-B aligned, a multiple of 16) with 16-byte nontemporal loads
 * spread over the whole GPU, each wave reading contiguous 8 KB chunks as a
 * decode wave reads its tiles, and do nothing else -- the read bandwidth this part reaches in practice, the
 * "measured stream-read peak" beside the 8 TB/s HBM figure.  `sink` (device,
 * 4 bytes) is written only if the xor of the data equals a fixed constant.
 * Kernel events armed by vit_arm_kernel_events bracket its kernel. */
int vit_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* A static string for a status code. */
const char *vit_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* VIT_H */
