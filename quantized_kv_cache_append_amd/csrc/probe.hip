// Attention-probe cell scoring for sparse KV eviction, and the eviction
// choice (Randozart/VITRIOL page: "How It Works -- Resident mode" runs a
// probe graph -- a q.K softmax with exponential decay -- every 16 steps and
// evicts the lowest-scored middle cells, sinks and recent cells protected).
//
// probe_logits_kernel: one 8-wave workgroup per (chunk, KV head, sequence).
// Chunk c owns tiles c, c + n_chunks, ...; wave w takes the chunk's tile
// slots w, w + 8, ..., prefetching the next one.  S^T = Q K^T runs on MFMA
// exactly as in decode's 16-row layout (query rows, fp16 hi and lo parts in
// two chained MFMAs, K codes exact in fp16, block scales in fp32); each
// lane writes its base-2 logits and keeps an online (max, sum of 2^(s - max))
// per query row; the waves merge into one partial per (query head, chunk).
// probe_mass_kernel: merges a sequence's partials per query head, then for
// every cell adds the query heads' probabilities and applies the decay.
// select_*_kernel: a 3-pass radix select over the middle cells' keys, by
// blocks of cells, finds the n_evict-th smallest (score, cell); then each
// block writes its chosen cells in cell order after those of the blocks
// before it.
#include "decode_impl.h"

namespace vit {

constexpr int kMassCells = 256;  // cells per probe_mass_kernel workgroup (one per thread)

// K registers of one 32-row tile for one lane (the K half of TileRegs).
template <int KC>
struct KTile {
  u32x4 kd[2][units_per_block(KC)];
  u32x2 ks[2];
  uint32_t kn[2];
};

template <int KC>
__device__ inline void load_k_tile(KTile<KC>& r, int t, int lane, const uint8_t* kbase, const uint16_t* ksb,
                                   const uint16_t* knb) {
  constexpr int KCB = units_per_block(KC);
  const uint8_t* kt = kbase + static_cast<int64_t>(t) * tile_code_bytes(KC);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (KC == ROT3) {
      r.kd[h][0] = load_unit12(kt + (h * 64 + lane) * 12);
    } else {
#pragma unroll
      for (int c = 0; c < KCB; ++c)
        r.kd[h][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kt + ((h * KCB + c) * 64 + lane) * 16));
    }
  }
  const int64_t row0 = static_cast<int64_t>(t) * kTile + (lane & 15);
  if constexpr (has_scales(KC)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) r.ks[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(ksb + (row0 + 16 * h) * 4));
  }
  if constexpr (has_norms(KC)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) r.kn[h] = __builtin_nontemporal_load(knb + row0 + 16 * h);
  }
}

template <int KC>
__global__ __launch_bounds__(64 * kProbeWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void probe_logits_kernel(
    ProbeArgs a) {
  constexpr int kThreads = 64 * kProbeWaves;
  constexpr bool kRot4 = KC == ROT4;
  constexpr bool kRot3 = KC == ROT3;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n16 = lane & 15;
  const int qg = lane >> 4;
  const int chunk = blockIdx.x;
  const int head = blockIdx.y;
  const int seq = blockIdx.z;
  const int L = a.seq_len[seq];
  // every scalar argument in one round trip (fetched where each is first
  // used, they were waited for one after another)
  __asm__ volatile("" ::"s"(L), "s"(a.gqa), "s"(a.n_chunks), "s"(a.n_kv_heads), "s"(a.n_q_heads), "s"(a.capacity),
                   "s"(a.kcodes), "s"(a.kscales), "s"(a.knorms), "s"(a.q), "s"(a.logits), "s"(a.part), "s"(a.qscale));
  const int G = a.gqa;
  const int n_tiles = (L + kTile - 1) / kTile;

  __shared__ __align__(16) float sq[16][kD];
  __shared__ uint32_t lut[kRot4 ? 256 * 64 : 1];
  __shared__ uint32_t lut3[kRot3 ? 64 * 64 : 1];
  __shared__ float s_m[kProbeWaves][16], s_l[kProbeWaves][16];

  const int64_t ph = static_cast<int64_t>(seq) * a.n_kv_heads + head;
  const uint8_t* kbase = a.kcodes + ph * a.capacity * row_code_bytes(KC);
  const uint16_t* ksb = has_scales(KC) ? a.kscales + ph * a.capacity * 4 : nullptr;
  const uint16_t* knb = has_norms(KC) ? a.knorms + ph * a.capacity : nullptr;

  // this chunk's tiles; loads past the last are clamped to it (a chunk
  // without tiles re-reads tile 0, which always exists, and processes none)
  const int n_mine = chunk < n_tiles ? (n_tiles - 1 - chunk) / a.n_chunks + 1 : 0;
  const int t_last = chunk < n_tiles ? chunk + a.n_chunks * (n_mine - 1) : 0;
  auto tile_of = [&](int k) { return chunk + a.n_chunks * k; };
  KTile<KC> ta, tb;
  load_k_tile<KC>(ta, min(tile_of(wave), t_last), lane, kbase, ksb, knb);
  load_k_tile<KC>(tb, min(tile_of(wave + kProbeWaves), t_last), lane, kbase, ksb, knb);

  // ---- query rows of this KV head (G <= 16, zero rows past G) in LDS ----
  [[maybe_unused]] uint32_t lv = 0, lv3 = 0;
  if constexpr (kRot4) lv = kLevelBits[lane & 15];
  if constexpr (kRot3) lv3 = kLevelBits3[lane & 7];
  const float* qhead = a.q + (static_cast<int64_t>(seq) * a.n_q_heads + static_cast<int64_t>(head) * G) * kD;
  if (tid < 256) {
    const int r = (8 * tid) >> 7, c0 = (8 * tid) & 127;
    const float* src = qhead + static_cast<int64_t>(min(r, G - 1)) * kD + c0;
    const float4v v0 = *reinterpret_cast<const float4v*>(src);
    const float4v v1 = *reinterpret_cast<const float4v*>(src + 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = r < G ? (j < 4 ? v0[j] : v1[j - 4]) : 0.0f;
      if constexpr (rotated(KC)) v = ((a.ksigns[(c0 + j) >> 5] >> ((c0 + j) & 31)) & 1u) ? -v : v;  // the keys' sign flip
      sq[r][c0 + j] = v;
    }
  }
  if constexpr (kRot4) fill_rot4_lut<kThreads>(lut, tid, lv);
  if constexpr (kRot3) fill_rot3_lut<kThreads>(lut3, tid, lv3);
  __syncthreads();
  float qs = a.qscale;
  if constexpr (rotated(KC)) {
    // rotate the query rows like the keys (unnormalised WHT; 1/128 folded in)
    wht128_lds<kThreads>(&sq[0][0], 16, tid);
    qs *= 1.0f / 128.0f;
  }
  // A operand of MFMA b: row n16 = query n16, chunk qg of block b, hi and lo
  half8 aqh[4], aql[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = sq[n16][k_chan<KC>(qg, b, j)] * qs;
    split8(v, aqh[b], aql[b]);
  }
  const Lut lutr{lut, lut3, 4u * static_cast<uint32_t>(lane)};

  float m_run[4], l_run[4];  // queries 4qg + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -__FLT_MAX__;  // finite: a fully masked first tile leaves l = 0, no NaN
    l_run[i] = 0.0f;
  }
  float* lg = a.logits + (static_cast<int64_t>(seq) * a.n_q_heads + static_cast<int64_t>(head) * G) * a.capacity;
  auto proc = [&](const KTile<KC>& cur, int t) {
    float kf[2][4];
    k_block_factors<KC>(cur, kf);
    float s[4][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float4v acc[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const half8 kb = unpack_k<KC>(cur.kd[h], b, lutr);
        acc[b] = mfma16(aqh[b], kb, float4v{0.0f, 0.0f, 0.0f, 0.0f});
        acc[b] = mfma16(aql[b], kb, acc[b]);
      }
      const int row = t * kTile + 16 * h + n16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v;
        if constexpr (KC == F16) v = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
        else v = (acc[0][i] * kf[h][0] + acc[1][i] * kf[h][1]) + (acc[2][i] * kf[h][2] + acc[3][i] * kf[h][3]);
        s[i][h] = row < L ? v : -INFINITY;
        if (row < L && 4 * qg + i < G) lg[static_cast<int64_t>(4 * qg + i) * a.capacity + row] = v;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mnew = fmaxf(m_run[i], row16_max(fmaxf(s[i][0], s[i][1])));
      l_run[i] = l_run[i] * __builtin_amdgcn_exp2f(m_run[i] - mnew) + __builtin_amdgcn_exp2f(s[i][0] - mnew) +
                 __builtin_amdgcn_exp2f(s[i][1] - mnew);
      m_run[i] = mnew;
    }
  };
  // two buffers: wave slots w + 16 j in ta, w + 8 + 16 j in tb
  for (int k = wave; k < n_mine; k += 2 * kProbeWaves) {
    proc(ta, tile_of(k));
    load_k_tile<KC>(ta, min(tile_of(k + 2 * kProbeWaves), t_last), lane, kbase, ksb, knb);
    if (k + kProbeWaves >= n_mine) break;
    proc(tb, tile_of(k + kProbeWaves));
    load_k_tile<KC>(tb, min(tile_of(k + 3 * kProbeWaves), t_last), lane, kbase, ksb, knb);
  }

  // ---- merge the waves: one (max, sum) per query head of this chunk ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float l = row16_sum(l_run[i]);
    if (n16 == 0) {
      s_m[wave][4 * qg + i] = m_run[i];
      s_l[wave][4 * qg + i] = l;
    }
  }
  __syncthreads();
  if (tid < G) {
    float M = -__FLT_MAX__;
    for (int w = 0; w < kProbeWaves; ++w) M = fmaxf(M, s_m[w][tid]);
    float Ls = 0.0f;
    for (int w = 0; w < kProbeWaves; ++w)
      if (s_l[w][tid] > 0.0f) Ls += s_l[w][tid] * __builtin_amdgcn_exp2f(s_m[w][tid] - M);
    float* p = a.part + ((static_cast<int64_t>(seq) * a.n_q_heads + static_cast<int64_t>(head) * G + tid) * a.n_chunks + chunk) * 2;
    p[0] = M;
    p[1] = Ls;
  }
}

// One workgroup per (256-cell block, sequence): merge every query head's
// chunk partials into (max, 1 / sum), then score <- decay * score + the sum
// over the query heads (in head order) of 2^(logit - max) / sum for each
// cell below L, one cell per thread.
__global__ __launch_bounds__(256) void probe_mass_kernel(ProbeArgs a) {
  const int tid = threadIdx.x;
  const int seq = blockIdx.y;
  const int L = a.seq_len[seq];
  __asm__ volatile("" ::"s"(L), "s"(a.n_chunks), "s"(a.n_q_heads), "s"(a.capacity), "s"(a.logits), "s"(a.part),
                   "s"(a.scores), "s"(a.decay));  // one round trip, as in probe_logits_kernel
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kMassCells;
  if (j0 >= L) return;  // uniform per workgroup
  __shared__ float s_max[kProbeMaxHeads], s_inv[kProbeMaxHeads];
  // a group of W lanes (W = n_chunks rounded up to a power of two, <= 64)
  // per query head, one lane per chunk partial: 256 / W heads per round
  int W = 1;
  while (W < a.n_chunks) W <<= 1;
  const int sub = tid & (W - 1);
  for (int h = tid / W; h < a.n_q_heads; h += kMassCells / W) {  // uniform per W-lane group
    const float* p = a.part + (static_cast<int64_t>(seq) * a.n_q_heads + h) * a.n_chunks * 2;
    float m = -__FLT_MAX__, l = 0.0f;
    if (sub < a.n_chunks) {
      m = p[2 * sub];
      l = p[2 * sub + 1];
    }
    float M = l > 0.0f ? m : -__FLT_MAX__;
    for (int d = W >> 1; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d, 64));
    float Ls = l > 0.0f ? l * __builtin_amdgcn_exp2f(m - M) : 0.0f;
    for (int d = W >> 1; d >= 1; d >>= 1) Ls += __shfl_xor(Ls, d, 64);
    if (sub == 0) {
      s_max[h] = M;
      s_inv[h] = 1.0f / Ls;  // every head sees L >= 1 cells: Ls >= 1
    }
  }
  __syncthreads();
  const float* lg = a.logits + static_cast<int64_t>(seq) * a.n_q_heads * a.capacity;
  float* sc = a.scores + static_cast<int64_t>(seq) * a.capacity;
  const int64_t j = j0 + tid;
  if (j < L) {
    const float prev = sc[j];
    float mass = 0.0f;
    int h = 0;
    // eight heads' logits in flight at a time, summed in head order
    for (; h + 8 <= a.n_q_heads; h += 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = lg[static_cast<int64_t>(h + i) * a.capacity + j];
#pragma unroll
      for (int i = 0; i < 8; ++i) mass += __builtin_amdgcn_exp2f(v[i] - s_max[h + i]) * s_inv[h + i];
    }
    for (; h < a.n_q_heads; ++h)
      mass += __builtin_amdgcn_exp2f(lg[static_cast<int64_t>(h) * a.capacity + j] - s_max[h]) * s_inv[h];
    sc[j] = a.decay * prev + mass;
  }
}

// ------------------------------------------------------------------ select
constexpr int kSelectThreads = 256;

// order-preserving key of an fp32 score (larger key = larger score; -0 and
// +0 are one key; NaN is outside the domain)
__device__ inline uint32_t score_key(float f) {
  const uint32_t u = f == 0.0f ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// inclusive sum over the workgroup's threads of v (every thread gets its
// prefix); `tot` receives the workgroup total
template <int NT = kSelectThreads>
__device__ inline int block_scan(int v, int tid, int* s_wave, int& tot) {
  const int lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = s_wave[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();  // s_wave is reused by the next call
  tot = all;
  return before + x;
}

// digit p of a key: bits 31..21, 20..10, 9..0
__device__ constexpr int kDigitShift[3] = {21, 10, 0};
__device__ constexpr uint32_t kDigitMask[3] = {0x7FFu, 0x7FFu, 0x3FFu};

// A sequence's middle cells and the number to choose.
struct SelectRange {
  int64_t lo, hi, k;
};
__device__ inline SelectRange select_range(const SelectArgs& a, int seq) {
  const int64_t L = a.seq_len[seq];
  SelectRange r;
  r.lo = a.n_sink < L ? a.n_sink : L;
  r.hi = L - a.n_recent > r.lo ? L - a.n_recent : r.lo;
  r.k = (r.hi - r.lo) < a.n_evict ? (r.hi - r.lo) : a.n_evict;
  return r;
}

// The key prefix after `passes` finished passes and the 1-based rank of the
// target among the keys carrying it (the same in every workgroup).
__device__ inline void select_state(const SelectArgs& a, int seq, int passes, int64_t k, int tid, uint32_t& prefix,
                                    uint32_t& mask, int64_t& rank, int* s_wave, int* s_pick) {
  prefix = 0;
  mask = 0;
  rank = k;
  for (int p = 0; p < passes; ++p) {
    const int* h = a.hist + (static_cast<int64_t>(p) * a.n_seqs + seq) * kSelectBins;
    constexpr int per = kSelectBins / kSelectThreads;  // 8 bins per thread
    int c[per], sum = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      c[i] = h[tid * per + i];
      sum += c[i];
    }
    int tot;
    const int incl = block_scan(sum, tid, s_wave, tot);
    int64_t before = incl - sum;
    if (before < rank && rank <= before + sum) {  // exactly one thread holds the target's bin
      int d = 0;
      while (d < per - 1 && before + c[d] < rank) before += c[d++];
      s_pick[0] = tid * per + d;
      s_pick[1] = static_cast<int>(rank - before);
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(s_pick[0]) << kDigitShift[p];
    mask |= kDigitMask[p] << kDigitShift[p];
    rank = s_pick[1];
    __syncthreads();
  }
}

// Every scalar argument of a select kernel in one round trip (fetched where
// each is first used, they were waited for one after another).
__device__ inline void fetch_select_args(const SelectArgs& a, int seq) {
  __asm__ volatile("" ::"s"(a.seq_len[seq]), "s"(a.capacity), "s"(a.n_sink), "s"(a.n_recent), "s"(a.n_evict),
                   "s"(a.n_seqs), "s"(a.cells_per_block), "s"(a.n_blocks), "s"(a.max_mid), "s"(a.scores),
                   "s"(a.rows_out), "s"(a.n_out), "s"(a.hist), "s"(a.counts));
}

__global__ __launch_bounds__(kSelectThreads) void select_zero_kernel(SelectArgs a) {
  const int seq = blockIdx.x;
  for (int p = 0; p < 3; ++p)
    for (int i = threadIdx.x; i < kSelectBins; i += kSelectThreads)
      a.hist[(static_cast<int64_t>(p) * a.n_seqs + seq) * kSelectBins + i] = 0;
}

// Pass P: histogram of digit P over the block's keys that carry the prefix
// of passes 0 .. P-1.  Lanes of a wave that share a bin are counted with one
// LDS add by a leader (scores cluster, so most keys share the top digits).
template <int P>
__global__ __launch_bounds__(kSelectThreads) void select_hist_kernel(SelectArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int seq = blockIdx.y;
  fetch_select_args(a, seq);
  const SelectRange r = select_range(a, seq);
  const int64_t b0 = r.lo + static_cast<int64_t>(blockIdx.x) * a.cells_per_block;
  if (r.k == 0 || b0 >= r.hi) return;  // uniform per workgroup
  const int64_t b1 = b0 + a.cells_per_block < r.hi ? b0 + a.cells_per_block : r.hi;
  __shared__ int hist[kSelectBins];
  __shared__ int s_wave[kSelectThreads / 64];
  __shared__ int s_pick[2];
  uint32_t prefix, mask;
  int64_t rank;
  select_state(a, seq, P, r.k, tid, prefix, mask, rank, s_wave, s_pick);
  for (int i = tid; i < kSelectBins; i += kSelectThreads) hist[i] = 0;
  __syncthreads();
  const float* sc = a.scores + static_cast<int64_t>(seq) * a.capacity;
  for (int64_t base = b0; base < b1; base += kSelectThreads) {  // uniform trip count
    const int64_t j = base + tid;
    const uint32_t key = j < b1 ? score_key(sc[j]) : 0u;
    bool pending = j < b1 && (key & mask) == prefix;
    const uint32_t bin = (key >> kDigitShift[P]) & kDigitMask[P];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const uint64_t act = __builtin_amdgcn_ballot_w64(pending);
      if (act == 0) break;
      const int leader = __builtin_ctzll(act);
      const uint32_t lb = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), leader));
      const uint64_t same = __builtin_amdgcn_ballot_w64(pending && bin == lb);
      if (lane == leader) atomicAdd(&hist[lb], __builtin_popcountll(same));
      pending = pending && bin != lb;
    }
    if (pending) atomicAdd(&hist[bin], 1);
  }
  __syncthreads();
  int* g = a.hist + (static_cast<int64_t>(P) * a.n_seqs + seq) * kSelectBins;
  for (int i = tid; i < kSelectBins; i += kSelectThreads)
    if (hist[i] != 0) atomicAdd(&g[i], hist[i]);
}

// Per block: its cells below the target key T and equal to it.
__global__ __launch_bounds__(kSelectThreads) void select_count_kernel(SelectArgs a) {
  const int tid = threadIdx.x;
  const int seq = blockIdx.y;
  fetch_select_args(a, seq);
  const SelectRange r = select_range(a, seq);
  const int64_t b0 = r.lo + static_cast<int64_t>(blockIdx.x) * a.cells_per_block;
  if (r.k == 0 || b0 >= r.hi) return;  // uniform per workgroup
  const int64_t b1 = b0 + a.cells_per_block < r.hi ? b0 + a.cells_per_block : r.hi;
  __shared__ int s_wave[kSelectThreads / 64];
  __shared__ int s_pick[2];
  uint32_t T, mask;
  int64_t rank;
  select_state(a, seq, 3, r.k, tid, T, mask, rank, s_wave, s_pick);
  const float* sc = a.scores + static_cast<int64_t>(seq) * a.capacity;
  int lt = 0, eq = 0;
  for (int64_t j = b0 + tid; j < b1; j += kSelectThreads) {
    const uint32_t key = score_key(sc[j]);
    lt += key < T ? 1 : 0;
    eq += key == T ? 1 : 0;
  }
  int n_lt, n_eq;
  block_scan(lt, tid, s_wave, n_lt);
  block_scan(eq, tid, s_wave, n_eq);
  if (tid == 0) {
    int* c = a.counts + (static_cast<int64_t>(seq) * kSelectMaxBlocks + blockIdx.x) * 2;
    c[0] = n_lt;
    c[1] = n_eq;
  }
}

// Per block, in cell order: every key below T and, of the keys equal to T,
// those whose rank among all of them (in cell order) is at most `rank`.
// The blocks before this one give the output offset.
__global__ __launch_bounds__(kSelectThreads) void select_write_kernel(SelectArgs a) {
  const int tid = threadIdx.x;
  const int seq = blockIdx.y;
  fetch_select_args(a, seq);
  const SelectRange r = select_range(a, seq);
  int64_t* out = a.rows_out + static_cast<int64_t>(seq) * a.n_evict;
  if (blockIdx.x == 0) {
    for (int64_t i = r.k + tid; i < a.n_evict; i += kSelectThreads) out[i] = -1;
    if (tid == 0) a.n_out[seq] = static_cast<int32_t>(r.k);
  }
  const int64_t b0 = r.lo + static_cast<int64_t>(blockIdx.x) * a.cells_per_block;
  if (r.k == 0 || b0 >= r.hi) return;  // uniform per workgroup
  const int64_t b1 = b0 + a.cells_per_block < r.hi ? b0 + a.cells_per_block : r.hi;
  __shared__ int s_wave[kSelectThreads / 64];
  __shared__ int s_pick[2];
  uint32_t T, mask;
  int64_t rank;
  select_state(a, seq, 3, r.k, tid, T, mask, rank, s_wave, s_pick);
  // cells chosen and keys equal to T in the blocks before this one
  const int* c = a.counts + static_cast<int64_t>(seq) * kSelectMaxBlocks * 2;
  int e_b = 0, l_b = 0;
  for (int b = tid; b < static_cast<int>(blockIdx.x); b += kSelectThreads) {
    l_b += c[2 * b];
    e_b += c[2 * b + 1];
  }
  int lt_before, eq_before;
  block_scan(l_b, tid, s_wave, lt_before);
  block_scan(e_b, tid, s_wave, eq_before);
  int64_t taken = lt_before + (eq_before < rank ? eq_before : rank);  // chosen before this block
  int64_t eq_seen = eq_before;
  const float* sc = a.scores + static_cast<int64_t>(seq) * a.capacity;
  for (int64_t base = b0; base < b1; base += kSelectThreads) {  // uniform trip count
    const int64_t j = base + tid;
    const uint32_t key = j < b1 ? score_key(sc[j]) : 0xFFFFFFFFu;
    const int is_eq = j < b1 && key == T ? 1 : 0;
    int n_eq;
    const int eq_incl = block_scan(is_eq, tid, s_wave, n_eq);
    const int sel = (j < b1 && key < T) || (is_eq && eq_seen + eq_incl <= rank) ? 1 : 0;
    int n_sel;
    const int pos = block_scan(sel, tid, s_wave, n_sel);
    if (sel && taken + pos - 1 < r.k) out[taken + pos - 1] = j;  // exactly k are chosen; the bound is a guard
    eq_seen += n_eq;
    taken += n_sel;
  }
}

#define VIT_PROBE_CASE(KC)                                                                                  \
  case KC:                                                                                                  \
    hipExtLaunchKernelGGL((probe_logits_kernel<KC>), grid, dim3(64 * kProbeWaves), 0, stream, ev.start,    \
                          ev.stop, 0, args);                                                                \
    break;

hipError_t launch_probe(int kc, int n_seqs, int max_seq_len, hipStream_t stream, const ProbeArgs& args,
                        const KernelEvents& ev) {
  const dim3 grid(static_cast<unsigned>(args.n_chunks), static_cast<unsigned>(args.n_kv_heads),
                  static_cast<unsigned>(n_seqs));
  switch (kc) {
    VIT_PROBE_CASE(F16)
    VIT_PROBE_CASE(Q8_0)
    VIT_PROBE_CASE(Q4_0)
    VIT_PROBE_CASE(ROT4)
    VIT_PROBE_CASE(ROT3)
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid(static_cast<unsigned>((max_seq_len + kMassCells - 1) / kMassCells), static_cast<unsigned>(n_seqs));
  hipLaunchKernelGGL(probe_mass_kernel, mgrid, dim3(256), 0, stream, args);
  return hipGetLastError();
}

// A sequence whose middle range fits in LDS: one workgroup does the three
// radix passes on an LDS histogram and the ordered write, in one launch.  In
// the write each thread owns a contiguous run of cells, so two block scans
// (keys below T, keys equal to T) give every thread its output offset.
constexpr int kSmallThreads = 1024;  // threads of the one-workgroup select

__global__ __launch_bounds__(kSmallThreads) void select_small_kernel(SelectArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int seq = blockIdx.x;
  fetch_select_args(a, seq);
  const SelectRange r = select_range(a, seq);
  int64_t* out = a.rows_out + static_cast<int64_t>(seq) * a.n_evict;
  for (int64_t i = r.k + tid; i < a.n_evict; i += kSmallThreads) out[i] = -1;
  if (tid == 0) a.n_out[seq] = static_cast<int32_t>(r.k);
  if (r.k == 0) return;  // uniform per workgroup
  const int n = static_cast<int>(r.hi - r.lo);  // <= kSelectSmallCells
  __shared__ uint32_t keys[kSelectSmallCells];
  __shared__ int hist[kSelectBins];
  __shared__ int s_wave[kSmallThreads / 64];
  __shared__ int s_pick[2];
  const float* sc = a.scores + static_cast<int64_t>(seq) * a.capacity + r.lo;
  for (int i = tid; i < n; i += kSmallThreads) keys[i] = score_key(sc[i]);
  uint32_t prefix = 0, mask = 0;
  int64_t rank = r.k;
  for (int p = 0; p < 3; ++p) {
    for (int i = tid; i < kSelectBins; i += kSmallThreads) hist[i] = 0;
    __syncthreads();  // (pass 0: also the key loads)
    for (int base = 0; base < n; base += kSmallThreads) {  // uniform trip count
      const int j = base + tid;
      const uint32_t key = j < n ? keys[j] : 0u;
      bool pending = j < n && (key & mask) == prefix;
      const uint32_t bin = (key >> kDigitShift[p]) & kDigitMask[p];
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const uint64_t act = __builtin_amdgcn_ballot_w64(pending);
        if (act == 0) break;
        const int leader = __builtin_ctzll(act);
        const uint32_t lb = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), leader));
        const uint64_t same = __builtin_amdgcn_ballot_w64(pending && bin == lb);
        if (lane == leader) atomicAdd(&hist[lb], __builtin_popcountll(same));
        pending = pending && bin != lb;
      }
      if (pending) atomicAdd(&hist[bin], 1);
    }
    __syncthreads();
    // the bin of the rank-th key and its rank among the keys in that bin
    constexpr int per = kSelectBins / kSmallThreads;
    int c[per], sum = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      c[i] = hist[tid * per + i];
      sum += c[i];
    }
    int tot;
    const int incl = block_scan<kSmallThreads>(sum, tid, s_wave, tot);
    int64_t before = incl - sum;
    if (before < rank && rank <= before + sum) {
      int d = 0;
      while (d < per - 1 && before + c[d] < rank) before += c[d++];
      s_pick[0] = tid * per + d;
      s_pick[1] = static_cast<int>(rank - before);
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(s_pick[0]) << kDigitShift[p];
    mask |= kDigitMask[p] << kDigitShift[p];
    rank = s_pick[1];
    __syncthreads();
  }
  // every key below T, and the first `rank` keys equal to T in cell order
  const uint32_t T = prefix;
  const int run = (n + kSmallThreads - 1) / kSmallThreads;
  const int c0 = min(tid * run, n), c1 = min(c0 + run, n);
  int lt = 0, eq = 0;
  for (int j = c0; j < c1; ++j) {
    lt += keys[j] < T ? 1 : 0;
    eq += keys[j] == T ? 1 : 0;
  }
  int n_lt, n_eq;
  const int lt_incl = block_scan<kSmallThreads>(lt, tid, s_wave, n_lt);
  const int eq_incl = block_scan<kSmallThreads>(eq, tid, s_wave, n_eq);
  int64_t eq_seen = eq_incl - eq;                                       // equal keys before this run
  int64_t pos = (lt_incl - lt) + (eq_seen < rank ? eq_seen : rank);     // chosen cells before this run
  for (int j = c0; j < c1; ++j) {
    const uint32_t key = keys[j];
    bool sel = key < T;
    if (key == T) sel = eq_seen++ < rank;
    if (sel) {
      if (pos < r.k) out[pos] = r.lo + j;  // exactly k are chosen; the bound is a guard
      ++pos;
    }
  }
}

hipError_t launch_select(int n_seqs, hipStream_t stream, const SelectArgs& args) {
  if (args.max_mid <= kSelectSmallCells) {
    hipLaunchKernelGGL(select_small_kernel, dim3(static_cast<unsigned>(n_seqs)), dim3(kSmallThreads), 0, stream,
                       args);
    return hipGetLastError();
  }
  const dim3 block(kSelectThreads), grid(static_cast<unsigned>(args.n_blocks), static_cast<unsigned>(n_seqs));
  hipLaunchKernelGGL(select_zero_kernel, dim3(static_cast<unsigned>(n_seqs)), block, 0, stream, args);
  hipLaunchKernelGGL(select_hist_kernel<0>, grid, block, 0, stream, args);
  hipLaunchKernelGGL(select_hist_kernel<1>, grid, block, 0, stream, args);
  hipLaunchKernelGGL(select_hist_kernel<2>, grid, block, 0, stream, args);
  hipLaunchKernelGGL(select_count_kernel, grid, block, 0, stream, args);
  hipLaunchKernelGGL(select_write_kernel, grid, block, 0, stream, args);
  return hipGetLastError();
}

}  // namespace vit
