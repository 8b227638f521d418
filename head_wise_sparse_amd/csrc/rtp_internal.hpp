// Internal declarations shared by the HIP sources of librtp (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstddef>

#include "rtp.h"

namespace rtp {

constexpr int kIdxDim = 16;       // the pages' indexer dimension (4, 8 and 32 are supported too)
constexpr int kMaxHeads = 64;     // KV heads a descriptor may hold

// ---------------------------------------------------------------- host-side helpers
// Record a failure message for rtp_last_error() and return the status.
rtp_status fail(rtp_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
rtp_status ok();
// Map a HIP error from a launch to RTP_EDEVICE (records the message).
rtp_status check_launch(const char* what);
// Called by every entry point where it would first touch the device, after its host
// checks: RTP_EDEVICE ("injected") when the environment sets RTP_FAULT_INJECT to a
// non-empty value, so that callers' device-error paths can be exercised without a GPU.
rtp_status enqueue_gate(const char* who);
// A roctx range around one C-ABI call, on when the environment sets RTP_ROCTX to a
// non-empty value at the library's first call (the roctx library is then opened with
// dlopen; the library does not link it).  Off, it costs one branch.
class TraceRange {
 public:
  explicit TraceRange(const char* name);
  ~TraceRange();
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;

 private:
  bool active_;
};

// Head bookkeeping derived from a validated descriptor.
struct Layer {
  int B, Hq, Hkv, D, G;
  int64_t n_cap;
  int n_ret, n_loc;               // retrieval / local KV heads
  int ret_kv[kMaxHeads];          // retrieval rank -> KV head
  int loc_kv[kMaxHeads];          // local rank -> KV head
  int n_sinks, window;
  int kv_layout;                  // RTP_KV_FULL / RTP_KV_COMPACT
  int idx;                        // indexer dimension
};

// Validate the descriptor (shared by every call).
rtp_status check_desc(const rtp_layer_desc* d, Layer* L);
bool aligned(const void* p, size_t a);

// Kernel-argument table mapping a rank to its KV head (passed by value).
struct HeadMap {
  int n;
  int kv[kMaxHeads];
};
HeadMap ret_map(const Layer& L);
HeadMap loc_map(const Layer& L);

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- per-call workspace layouts
// Indexer scoring: per-block (max, sum) partials.
constexpr int kScoreThreads = 256;
constexpr int kScoreItems = 8;                                  // tokens per thread (indexer dim <= 16)
constexpr int kScoreTile = kScoreThreads * kScoreItems;         // tokens per block (indexer dim <= 16)
constexpr int score_items(int idx) { return idx <= 16 ? kScoreItems : kScoreItems / 2; }
constexpr int score_tile(int idx) { return kScoreThreads * score_items(idx); }
size_t score_ws_bytes(const Layer& L, int64_t n_ctx);

// Top-p mass is summed in u64 fixed point with F fraction bits (the row max weighs 2^F):
// F = 42 up to 2^20 tokens, then one bit fewer per doubling of the context, so that a row
// of n_ctx weights (each <= 2^F) sums below 2^63.  Rounding moves each weight by at most
// 2^-(F+1) of the max weight, so the whole row's mass by at most n_ctx * 2^-(F+1) of it:
// 2^-23 at 2^20 tokens, 2^-15 at 2^24.  Top-p is refused above kTopPMaxCtx tokens, where
// that bound would pass 1e-4.
constexpr int64_t kTopPMaxCtx = int64_t(1) << 24;
__host__ __device__ inline int mass_frac_bits(int64_t n_ctx) {
  int c = 0;
  while ((int64_t(1) << c) < n_ctx) ++c;                        // ceil(log2(n_ctx))
  return 62 - c < 42 ? 62 - c : 42;
}
__host__ __device__ inline float mass_wscale(int64_t n_ctx) { return float(int64_t(1) << mass_frac_bits(n_ctx)); }

// Context length of a launch.  The calls take it from the host (live == null); the
// device-length step reads it from a device word written by an earlier launch (live),
// clamped to [1, n_max], where n_max is the host bound every stride and grid is sized
// for.  With live == null the length is n_max itself, so both paths share the kernels.
__device__ __forceinline__ int live_ctx(const int64_t* live, int n_max) {
  if (!live) return n_max;
  const int64_t v = *live;
  return int(v < 1 ? 1 : (v > n_max ? int64_t(n_max) : v));
}

// Top-p selection (four launches, or one for short rows; the workspace is zero before
// and after a call).
constexpr int kSelThreads = 256;
constexpr int kSelItems = 16;
constexpr int kSelTile = kSelThreads * kSelItems;               // tokens per block ...
constexpr int kSelItemsLong = 32;                                // ... or twice that when a pass would
                                                                 // otherwise take more than one round of blocks
constexpr int kSelSmallMax = kSelThreads * kSelItemsLong;       // rows up to this take one block each
constexpr int kBins = 2048;                                     // 11-bit digits (last level 10 bits)
constexpr int kTabDigits = 1024;                                // last-level digits (10 bits)
// The last radix pass leaves one record per kRecTok tokens (one decode range), so that
// the range index can be formed from the records alone.
constexpr int kRecTok = RTP_SEL_RANGE;
static_assert(kRecTok % kSelThreads == 0 && (kSelItems * kSelThreads) % (2 * kRecTok) == 0,
              "whole records per tile, an even number of them");
struct SelLevelState {           // what is known after resolving one level's digit
  uint32_t prefix;               // key bits resolved so far
  uint32_t cnt_above;            // tokens strictly above the prefix
  uint64_t above;                // their mass (fixed point)
  uint64_t target;               // mass the set must reach (fixed point)
};
struct SelRowState {             // one per score row, lives in the workspace
  float ref_max;                 // the row max every fixed-point weight is taken against
  uint32_t pad;
  SelLevelState lvl[2];          // after level 0, after level 1 (written by different launches)
};
static_assert(sizeof(SelRowState) == 56, "row state layout");
struct SelLayout {                // depends on the layer only (n_cap), not on n_ctx: the
  size_t hist_mass, hist_cnt, coarse_mass, coarse_cnt, state, ctr, tilerec, tiletab, total;
  int nrec_max;                   // zero-filled region stays in place while n_ctx grows
};
SelLayout sel_layout(const Layer& L);
struct SelRows {                 // device views of the selection workspace
  uint64_t* mass;                // [rows][3][kBins]
  uint32_t* cnt;                 // [rows][3][kBins]
  uint64_t* cmass;               // [rows][3][64]   coarse summaries (32 fine bins each)
  uint32_t* ccnt;                // [rows][3][64]
  SelRowState* state;            // [rows]
  uint32_t* ctr;                 // [rows][2]       compaction: [1] blocks done ([0] unused, kept zero)
  uint4* tilerec;                // [rows][nrec]    per kRecTok tokens: counts against the level-1 prefix (hist<2>)
  uint16_t* tiletab;             // [rows][nrec][kTabDigits] records that overflowed: candidates
                                 //                 with low digit >= d (hist<2>; written whole before
                                 //                 it is read, never cleared: the end of the region)
};
struct SelArgs {
  const float* scores;           // [rows][n_cap]
  const float* row_max;          // [rows], or null: then from score_part
  const float2* score_part;      // [rows][score_nblk] per-block (max, sum of exp) of the scoring, or null
  int score_nblk;
  float* row_max_out;            // with score_part: row statistics written by the first pass
  float* row_sum_out;
  float top_p;
  int by_count;                  // static top-k: bins weigh their token counts, the target is k_target
  int64_t k_target;
  int n_ctx;                     // the context (device-length step: its bound n_max)
  const int64_t* live;           // device-length step: the context's device word, else null
  int64_t n_cap;
  int nblk;                      // selection tiles per row (from n_ctx; set by launch_select)
  int items;                     // scores per thread per tile (kSelItems or kSelItemsLong; set by launch_select)
  int rec_stride;                // records per row (from n_cap)
  int32_t* sel_idx;
  int32_t* sel_count;
  int32_t* starts;               // [rows][nsplit + 1] range index of the selected lists, or null
  int nsplit;                    // ranges of n_ctx (row stride of starts: nsplit + 1)
  uint32_t* thr_out;             // decode step: [rows] threshold keys for the gather, which then
                                 // writes the lists itself (requires starts); null: the lists here
  SelRows R;
};
SelRows sel_rows(void* ws, const SelLayout& lay);
// Enqueue the selection launches for `rows` score rows (top_p < 1 uses the workspace).
rtp_status launch_select(const SelArgs& a, int rows, hipStream_t s);

// Decode attention (sparse and window share the layout).
constexpr int kDecThreads = 256;
constexpr int kDecRange = RTP_SEL_RANGE; // token-index range per block (sparse path)
constexpr int kWinRange = 256;           // list positions per block (window path) when no slice fits ...
constexpr int kWinRangeShort = 128;      // ... else the shortest multiple of 32 from 128 ...
constexpr int kWinRangeMax = 512;        // ... to 512 with which the launch fits one round
constexpr int kDecUnroll = 2;            // cached rows per pipeline stage per lane group (2 stages)
// Sparse path: blocks per index range (each takes one slice of the range's union list),
// chosen per call so that the grid is about one round of resident blocks
constexpr int kDecSubMax = 4;
constexpr int kDecBlocksTarget = 1024;
inline int dec_sub(int nsplit, int groups) {
  int n = kDecBlocksTarget / (nsplit * groups > 0 ? nsplit * groups : 1);
  return n < 1 ? 1 : (n > kDecSubMax ? kDecSubMax : n);
}
// window slice length for `len` list positions and `groups` (batch x local KV heads),
// sharing a launch with `other` blocks: a block walks its slice as a chain of dependent
// loads, so the shortest slice wins as long as every block still starts in the first
// round of resident blocks
inline int win_range(int64_t len, int groups, int other) {
  for (int wr = kWinRangeShort; wr <= kWinRangeMax; wr += 32)
    if (other + (len + wr - 1) / wr * groups <= kDecBlocksTarget) return wr;
  return kWinRange;
}
size_t dec_ws_bytes(const Layer& L, int64_t n_ctx, bool sparse);   // partials [rows][slots][D + 4]
// window slice length of a call (the same for the separate call and the fused step, which
// would run the scoring blocks beside the window blocks; equal results need equal slices)
int win_range_for(const Layer& L, int64_t n_ctx, int64_t len);
size_t dec_sparse_starts_offset(const Layer& L, int64_t n_ctx);   // int32 [rows][nsplit+1] after partials
// Rows with more than kMergeDirect splits are merged in two levels: first kMergeFan
// splits at a time into second-level partials (after the range index), then those.
constexpr int kMergeFan = 32;
constexpr int kMergeDirect = 128;
inline int merge_chunks(int nsplit) { return nsplit > kMergeDirect ? (nsplit + kMergeFan - 1) / kMergeFan : 0; }
size_t dec_sparse_part2_offset(const Layer& L, int64_t n_ctx);    // float [rows][chunks][D + 4]

// Prefill.
size_t prefill_ws_bytes(const Layer& L, int64_t C);

// Fused decode step (selection region first, then scoring / sparse / window regions).
size_t step_ws_bytes(const Layer& L, int64_t n_ctx);

}  // namespace rtp

// ---------------------------------------------------------------- device helpers
namespace rtp_dev {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// float -> bf16 round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Monotone key of an fp32 score: a larger score gives a larger key; -0 and +0 tie.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Fixed-point softmax weight of a score: round(exp(s - m) * 2^F), exp argument clamped to
// <= 0, with wscale = 2^F (F from mass_frac_bits: every weight is <= 2^F and a row of n_ctx
// of them sums below 2^63).
__device__ __forceinline__ uint64_t fixed_weight(float s, float m, float wscale) {
  float w = __expf(fminf(s - m, 0.0f));
  return (uint64_t)__builtin_rintf(w * wscale);              // w * 2^F <= 2^42 is exact in float range
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace rtp_dev
