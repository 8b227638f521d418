// rtp_decode_step: the whole decode step of one layer in one call -- indexer scores,
// top-p sets, sparse attention of the retrieval heads and sink+window attention of
// the local heads (abstract, observations (1)-(3); research-map summary, "Approach").
//
// It writes exactly what the four calls write one after the other, in seven launches
// instead of thirteen (four for contexts of at most 8192 tokens, whose selection takes
// one launch):
//   1. scoring blocks and the local heads' split-K blocks in one grid: both stream
//      HBM (indexer keys / sink+window K,V) and do not depend on each other;
//   2. the first radix pass, which also reduces the scoring partials to the row
//      statistics (no separate finalize launch);
//   3-4. the two further radix passes;  5. one block per row resolves the threshold
//      and writes the range index of every selected list from the last pass's records;
//   6. the retrieval heads' split-K blocks, which take each range's members from its
//      scores and write that part of the selected lists;
//   7. one merge launch for the split partials of both head kinds (preceded, when a
//      retrieval row has more than 128 split partials, by a launch that combines
//      them 32 at a time).
#include <algorithm>
#include <cmath>
#include <mutex>

#include "score_dev.hpp"
#include "decode_dev.hpp"

namespace {

static_assert(kScoreThreads == kDecThreads, "scoring and decode blocks share one launch");

// (eight heads per group keep more accumulators than four waves per SIMD leave registers for)
template <int G, int D>
__global__ __launch_bounds__(kDecThreads, G >= 8 ? 2 : 4) void k_step_score_window(ScoreArgs sa, int n_score, int score_gx,
                                                                      DecArgs wa, int win_gx) {
  const int i = blockIdx.x;
  if (i < n_score) {
    score_block<G, D>(sa, i % score_gx, i / score_gx);
  } else {
    const int j = i - n_score;
    decode_block<D, G, false>(wa, j % win_gx, j / win_gx);
  }
}

template <int D, int G>
__global__ __launch_bounds__(kDecThreads, 4) void k_step_sparse(DecArgs a) {
  decode_block<D, G, true, true>(a, blockIdx.x, blockIdx.y);
}

template <int D>
__global__ __launch_bounds__(256) void k_step_merge_pre(MergeArgs ms, float* part2, int nchunks) {
  merge_pre_chunk<D>(ms, part2, nchunks, blockIdx.y, blockIdx.x);
}

// gen: the device-length step's state {pos, n_ctx}; the last launch of the step moves pos
// to n_ctx (no launch of the step reads pos), so the next append writes the next token.
template <int D>
__global__ __launch_bounds__(256) void k_step_merge(MergeArgs ms, int rows_s, MergeArgs mw, int64_t* gen) {
  const int i = blockIdx.x;
  if (i < rows_s) merge_row<D>(ms, i);
  else merge_row<D>(mw, i - rows_s);
  if (gen && i == 0 && threadIdx.x == 0) gen[0] = gen[1];
}

__global__ __launch_bounds__(64) void k_step_finalize(const float2* __restrict__ part, int stride, int n_max,
                                                      const int64_t* live, float* __restrict__ row_max,
                                                      float* __restrict__ row_sum) {
  const int n = live_ctx(live, n_max);
  score_finalize_row(part, stride, (n + kScoreTile - 1) / kScoreTile, row_max, row_sum, blockIdx.x);
}

struct StepLayout {
  size_t sel, score, sparse, window, thr, total;
};

// The selection region comes first and depends on the layer only, so the part of the
// workspace that must stay zero between calls does not move while n_ctx grows.
StepLayout step_layout(const Layer& L, int64_t n_ctx) {
  StepLayout s{};
  size_t off = 0;
  s.sel = off;
  off = round_up(off + (L.n_ret ? sel_layout(L).total : 0), 256);
  s.score = off;
  off = round_up(off + (L.n_ret ? score_ws_bytes(L, n_ctx) : 0), 256);
  s.sparse = off;
  off = round_up(off + (L.n_ret ? dec_ws_bytes(L, n_ctx, true) : 0), 256);
  s.window = off;
  off = round_up(off + (L.n_loc ? dec_ws_bytes(L, n_ctx, false) : 0), 256);
  s.thr = off;                                    // threshold key per retrieval row, for the gather
  off = round_up(off + size_t(L.B) * L.n_ret * L.G * sizeof(uint32_t), 256);
  s.total = off;
  return s;
}

template <int G, int D>
void launch_score_window(unsigned nblocks, hipStream_t s, const ScoreArgs& sa, int n_score, int score_gx,
                         const DecArgs& wa, int win_gx) {
  hipLaunchKernelGGL((k_step_score_window<G, D>), dim3(nblocks), dim3(kDecThreads), 0, s, sa, n_score, score_gx,
                     wa, win_gx);
}

rtp_status dispatch_score_window(const Layer& L, unsigned nblocks, hipStream_t s, const ScoreArgs& sa, int n_score,
                                 int score_gx, const DecArgs& wa, int win_gx) {
#define RTP_STEP_CASE(GG, DD)                                                 \
  if (L.G == GG && L.D == DD) {                                               \
    launch_score_window<GG, DD>(nblocks, s, sa, n_score, score_gx, wa, win_gx); \
    return check_launch("k_step_score_window");                               \
  }
  RTP_STEP_CASE(1, 64) RTP_STEP_CASE(2, 64) RTP_STEP_CASE(4, 64) RTP_STEP_CASE(8, 64)
  RTP_STEP_CASE(1, 128) RTP_STEP_CASE(2, 128) RTP_STEP_CASE(4, 128) RTP_STEP_CASE(8, 128)
#undef RTP_STEP_CASE
  return fail(RTP_EUNSUPPORTED, "rtp_decode_step: unsupported head_dim/group");
}

rtp_status dispatch_sparse(const Layer& L, dim3 grid, hipStream_t s, const DecArgs& a) {
#define RTP_STEP_CASE(GG, DD)                                                          \
  if (L.G == GG && L.D == DD) {                                                        \
    hipLaunchKernelGGL((k_step_sparse<DD, GG>), grid, dim3(kDecThreads), 0, s, a);     \
    return check_launch("k_step_sparse");                                              \
  }
  RTP_STEP_CASE(1, 64) RTP_STEP_CASE(2, 64) RTP_STEP_CASE(4, 64) RTP_STEP_CASE(8, 64)
  RTP_STEP_CASE(1, 128) RTP_STEP_CASE(2, 128) RTP_STEP_CASE(4, 128) RTP_STEP_CASE(8, 128)
#undef RTP_STEP_CASE
  return fail(RTP_EUNSUPPORTED, "rtp_decode_step: unsupported head_dim/group");
}

constexpr float kLog2eStep = 1.4426950408889634f;

}  // namespace

namespace rtp {
size_t step_ws_bytes(const Layer& L, int64_t n_ctx) { return step_layout(L, n_ctx).total; }
}  // namespace rtp

namespace {

// Zero-fill of n 16-byte words (a kernel rather than a memset node, so that a captured
// graph replays it faithfully).
__global__ __launch_bounds__(256) void k_step_clear(uint4* __restrict__ p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += size_t(gridDim.x) * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The whole step; `clear_sel`: zero the selection region first (the allocation-free entry
// point, whose scratch keeps whatever the last call on the device left there).
rtp_status decode_step_impl(const rtp_layer_desc* desc, int64_t n_ctx, const uint16_t* q_pre,
                            const uint16_t* w_q_idx, int64_t w_head_stride, const uint16_t* k_idx,
                            float idx_scale, const uint16_t* q, const uint16_t* k_cache,
                            const uint16_t* v_cache, const uint16_t* k_loc, const uint16_t* v_loc,
                            float top_p, float sm_scale, float* scores,
                            float* row_max, float* row_sum, int32_t* sel_idx, int32_t* sel_count,
                            int32_t* sel_starts, uint16_t* out, void* ws, size_t ws_bytes,
                            void* stream, bool clear_sel, int64_t* gen = nullptr) {
  // gen (device-length step): n_ctx is the bound every grid and stride is sized for, and
  // the live length is gen[1]
  const int64_t* live = gen ? gen + 1 : nullptr;
  Layer L;
  rtp_status st = check_desc(desc, &L);
  if (st != RTP_OK) return st;
  if (n_ctx < 1 || n_ctx > L.n_cap)
    return fail(RTP_EINVAL, "rtp_decode_step: n_ctx must be in [1, n_cap=%lld] (got %lld)", (long long)L.n_cap,
                (long long)n_ctx);
  const bool compact = L.kv_layout == RTP_KV_COMPACT;
  // the local heads' cache: the ring (compact layout) or the shared full cache
  const uint16_t* k_loc_c = compact ? k_loc : k_cache;
  const uint16_t* v_loc_c = compact ? v_loc : v_cache;
  if (!q || !out || (L.n_ret && (!k_cache || !v_cache)) || (L.n_loc && (!k_loc_c || !v_loc_c)))
    return fail(RTP_EINVAL, "rtp_decode_step: NULL tensor pointer");
  if ((k_loc_c && !aligned(k_loc_c, 16)) || (v_loc_c && !aligned(v_loc_c, 16)))
    return fail(RTP_EINVAL, "rtp_decode_step: q/k/v must be 16-byte aligned");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 2))
    return fail(RTP_EINVAL, "rtp_decode_step: q/k/v must be 16-byte aligned");
  if (!std::isfinite(sm_scale)) return fail(RTP_EINVAL, "rtp_decode_step: sm_scale must be finite");
  if (L.n_ret) {
    if (!q_pre || !w_q_idx || !k_idx || !scores || !row_max || !row_sum || !sel_idx || !sel_count)
      return fail(RTP_EINVAL, "rtp_decode_step: NULL tensor pointer");
    if (w_head_stride < 0 || w_head_stride % 8 != 0)
      return fail(RTP_EINVAL, "w_head_stride must be a non-negative multiple of 8 (got %lld)",
                  (long long)w_head_stride);
    if (!std::isfinite(idx_scale)) return fail(RTP_EINVAL, "idx_scale must be finite");
    if (!(top_p > 0.0f)) return fail(RTP_EINVAL, "top_p must be > 0 (got %g)", double(top_p));
    if (top_p < 1.0f && n_ctx > kTopPMaxCtx)
      return fail(RTP_EUNSUPPORTED, "rtp_decode_step: top_p < 1 needs n_ctx <= 2^24 (got %lld)", (long long)n_ctx);
    if (!aligned(k_idx, 16) || !aligned(scores, 16) || !aligned(q_pre, 16) || !aligned(w_q_idx, 16) ||
        !aligned(sel_idx, 16))
      return fail(RTP_EINVAL, "rtp_decode_step: tensors must be 16-byte aligned");
  }
  const StepLayout lay = step_layout(L, n_ctx);
  if (!ws || ws_bytes < lay.total || !aligned(ws, 256))
    return fail(RTP_EWORKSPACE, "rtp_decode_step: workspace needs %zu bytes, 256-aligned (got %zu)", lay.total,
                ws_bytes);
  if (!L.n_ret && !L.n_loc) return ok();
  if (L.n_ret && L.idx != kIdxDim)
    return fail(RTP_EUNSUPPORTED, "rtp_decode_step: idx_dim %d needs the separate calls (fused: 16)", L.idx);
  if ((st = enqueue_gate("rtp_decode_step")) != RTP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  const int n = int(n_ctx);
  if (clear_sel && L.n_ret && top_p < 1.0f) {
    // up to the heavy-tile tables, which a call writes before it reads them (offsets are
    // multiples of 256 bytes)
    const size_t n16 = sel_layout(L).tiletab / 16;
    const unsigned nb = unsigned(std::min<size_t>((n16 + 255) / 256, 1024));
    hipLaunchKernelGGL(k_step_clear, dim3(nb), dim3(256), 0, s, reinterpret_cast<uint4*>(w + lay.sel), n16);
    if ((st = check_launch("k_step_clear")) != RTP_OK) return st;
  }

  // ---- launch 1: scoring blocks + local heads' split-K blocks
  ScoreArgs sa{};
  int n_score = 0, score_gx = 1;
  if (L.n_ret) {
    score_gx = int((n_ctx + kScoreTile - 1) / kScoreTile);
    n_score = score_gx * L.B * L.n_ret;
    sa = ScoreArgs{q_pre, w_q_idx, w_head_stride, k_idx, idx_scale, scores, reinterpret_cast<float2*>(w + lay.score),
                   n, live, L.n_cap, L.Hq, ret_map(L), score_gx};
  }
  DecArgs wa{};
  int win_gx = 1, n_win = 0;
  if (L.n_loc) {
    const int64_t s_end = std::min<int64_t>(L.n_sinks, n_ctx);
    const int64_t w_start = std::max<int64_t>(n_ctx - L.window, s_end);
    const int64_t len = s_end + (n_ctx - w_start);
    wa.wrange = win_range_for(L, n_ctx, len);
    win_gx = int((len + wa.wrange - 1) / wa.wrange);
    n_win = win_gx * L.B * L.n_loc;
    wa.q = q;
    wa.k = k_cache;
    wa.v = v_cache;
    wa.part = reinterpret_cast<float*>(w + lay.window);
    wa.n_ctx = n;
    wa.live = live;
    wa.n_sinks = L.n_sinks;
    wa.window = L.window;
    wa.n_cap = L.n_cap;
    wa.Hq = L.Hq;
    wa.Hkv = L.Hkv;
    wa.nsplit = win_gx;
    wa.scale_log2 = sm_scale * kLog2eStep;
    wa.s_end = int(s_end);
    wa.w_start = int(w_start);
    wa.list_len = int(len);
    wa.map = loc_map(L);
    wa.k = k_loc_c;
    wa.v = v_loc_c;
    set_window_cache(wa, L);
  }
  if ((st = dispatch_score_window(L, unsigned(n_score + n_win), s, sa, n_score, score_gx, wa, win_gx)) != RTP_OK)
    return st;

  // ---- launches 2-5: top-p sets (the first pass also writes the row statistics)
  const int nsplit = int((n_ctx + kDecRange - 1) / kDecRange);
  const int rows_s = L.B * L.n_ret * L.G;
  int32_t* starts = sel_starts;
  if (L.n_ret) {
    if (!starts) starts = reinterpret_cast<int32_t*>(w + lay.sparse + dec_sparse_starts_offset(L, n_ctx));
    const SelLayout sl = sel_layout(L);
    SelArgs a{};
    a.scores = scores;
    a.row_max = nullptr;
    a.score_part = sa.part;
    a.score_nblk = score_gx;
    a.row_max_out = row_max;
    a.row_sum_out = row_sum;
    a.top_p = top_p;
    a.n_ctx = n;
    a.live = live;
    a.n_cap = L.n_cap;
    a.rec_stride = sl.nrec_max;
    a.sel_idx = sel_idx;
    a.sel_count = sel_count;
    a.starts = starts;
    a.nsplit = nsplit;
    a.thr_out = reinterpret_cast<uint32_t*>(w + lay.thr);   // the gather writes the lists
    a.R = sel_rows(w + lay.sel, sl);
    if (top_p >= 1.0f) {           // no radix pass runs: reduce the partials here
      hipLaunchKernelGGL(k_step_finalize, dim3(rows_s), dim3(64), 0, s, sa.part, score_gx, n, live, row_max,
                         row_sum);
      if ((st = check_launch("k_step_finalize")) != RTP_OK) return st;
    }
    if ((st = launch_select(a, rows_s, s)) != RTP_OK) return st;

    // ---- launch 6: retrieval heads' split-K blocks over the union of each group's sets
    DecArgs da{};
    da.q = q;
    da.k = k_cache;
    da.v = v_cache;
    da.starts = starts;
    da.scores = scores;
    da.thr = a.thr_out;
    da.all_tokens = top_p >= 1.0f;                  // every token: the lists are already written
    da.sel_out = top_p >= 1.0f ? nullptr : sel_idx;
    da.part = reinterpret_cast<float*>(w + lay.sparse);
    da.n_ctx = n;
    da.live = live;
    da.n_cap = L.n_cap;
    da.Hq = L.Hq;
    da.Hkv = L.Hkv;
    da.nsplit = nsplit;
    da.scale_log2 = sm_scale * kLog2eStep;
    da.map = ret_map(L);
    set_sparse_cache(da, L);
    if ((st = dispatch_sparse(L, dim3(nsplit * da.nsub, L.B * L.n_ret), s, da)) != RTP_OK) return st;
  }

  // ---- launch 7: merge the split partials of both head kinds
  const int rows_w = L.B * L.n_loc * L.G;
  const int nslots = nsplit * (L.n_ret ? dec_sub(nsplit, L.B * L.n_ret) : 1);   // sparse partials per row
  MergeArgs ms{reinterpret_cast<const float*>(w + lay.sparse), nslots, L.G, L.Hq, ret_map(L), out};
  const int nchunks = L.n_ret ? merge_chunks(nslots) : 0;
  if (nchunks) {           // long rows: merge kMergeFan splits at a time first
    float* part2 = reinterpret_cast<float*>(w + lay.sparse + dec_sparse_part2_offset(L, n_ctx));
    if (L.D == 128)
      hipLaunchKernelGGL(k_step_merge_pre<128>, dim3(nchunks, rows_s), dim3(256), 0, s, ms, part2, nchunks);
    else
      hipLaunchKernelGGL(k_step_merge_pre<64>, dim3(nchunks, rows_s), dim3(256), 0, s, ms, part2, nchunks);
    if ((st = check_launch("k_step_merge_pre")) != RTP_OK) return st;
    ms.part = part2;
    ms.nsplit = nchunks;
  }
  const MergeArgs mw{reinterpret_cast<const float*>(w + lay.window), win_gx, L.G, L.Hq, loc_map(L), out};
  const unsigned mrows = unsigned((L.n_ret ? rows_s : 0) + (L.n_loc ? rows_w : 0));
  const int rs = L.n_ret ? rows_s : 0;
  if (L.D == 128)
    hipLaunchKernelGGL(k_step_merge<128>, dim3(mrows), dim3(256), 0, s, ms, rs, mw, gen);
  else
    hipLaunchKernelGGL(k_step_merge<64>, dim3(mrows), dim3(256), 0, s, ms, rs, mw, gen);
  return check_launch("k_step_merge");
}

}  // namespace

extern "C" rtp_status rtp_decode_step(const rtp_layer_desc* desc, int64_t n_ctx, const uint16_t* q_pre,
                                      const uint16_t* w_q_idx, int64_t w_head_stride, const uint16_t* k_idx,
                                      float idx_scale, const uint16_t* q, const uint16_t* k_cache,
                                      const uint16_t* v_cache, const uint16_t* k_loc, const uint16_t* v_loc,
                                      float top_p, float sm_scale, float* scores,
                                      float* row_max, float* row_sum, int32_t* sel_idx, int32_t* sel_count,
                                      int32_t* sel_starts, uint16_t* out, void* ws, size_t ws_bytes,
                                      void* stream) {
  TraceRange trace_("rtp_decode_step");
  return decode_step_impl(desc, n_ctx, q_pre, w_q_idx, w_head_stride, k_idx, idx_scale, q, k_cache, v_cache, k_loc,
                          v_loc, top_p, sm_scale, scores, row_max, row_sum, sel_idx, sel_count, sel_starts, out, ws,
                          ws_bytes, stream, false);
}

// ---------------------------------------------------------------- device-length variant
extern "C" rtp_status rtp_decode_step_dev(const rtp_layer_desc* desc, int64_t n_max, int64_t* gen,
                                          const uint16_t* q_pre, const uint16_t* w_q_idx, int64_t w_head_stride,
                                          const uint16_t* k_idx, float idx_scale, const uint16_t* q,
                                          const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_loc,
                                          const uint16_t* v_loc, float top_p, float sm_scale, float* scores,
                                          float* row_max, float* row_sum, int32_t* sel_idx, int32_t* sel_count,
                                          int32_t* sel_starts, uint16_t* out, void* ws, size_t ws_bytes,
                                          void* stream) {
  TraceRange trace_("rtp_decode_step_dev");
  if (!gen) return fail(RTP_EINVAL, "rtp_decode_step_dev: NULL generation state");
  if (!aligned(gen, 8)) return fail(RTP_EINVAL, "rtp_decode_step_dev: the generation state must be 8-byte aligned");
  return decode_step_impl(desc, n_max, q_pre, w_q_idx, w_head_stride, k_idx, idx_scale, q, k_cache, v_cache, k_loc,
                          v_loc, top_p, sm_scale, scores, row_max, row_sum, sel_idx, sel_count, sel_starts, out, ws,
                          ws_bytes, stream, false, gen);
}

// ---------------------------------------------------------------- allocation-free variant
// The decode step's scratch in a file-scope device array instead of a caller workspace.
// Each GPU the library runs on holds its own copy (at its own address) until the process
// ends.  Host code never passes the array's name to a kernel: its device address is looked
// up once per device and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

rtp_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(RTP_EDEVICE, "rtp_decode_step_noalloc: cannot read the current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(RTP_EDEVICE, "rtp_decode_step_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

}  // namespace

extern "C" size_t rtp_decode_step_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" rtp_status rtp_decode_step_noalloc(const rtp_layer_desc* desc, int64_t n_ctx, const uint16_t* q_pre,
                                              const uint16_t* w_q_idx, int64_t w_head_stride, const uint16_t* k_idx,
                                              float idx_scale, const uint16_t* q, const uint16_t* k_cache,
                                              const uint16_t* v_cache, const uint16_t* k_loc, const uint16_t* v_loc,
                                              float top_p, float sm_scale, float* scores, float* row_max,
                                              float* row_sum, int32_t* sel_idx, int32_t* sel_count,
                                              int32_t* sel_starts, uint16_t* out, void* stream) {
  TraceRange trace_("rtp_decode_step_noalloc");
  Layer L;
  rtp_status st = check_desc(desc, &L);
  if (st != RTP_OK) return st;
  if (n_ctx < 1 || n_ctx > L.n_cap)
    return fail(RTP_EINVAL, "rtp_decode_step_noalloc: n_ctx must be in [1, n_cap=%lld] (got %lld)",
                (long long)L.n_cap, (long long)n_ctx);
  const size_t need = step_ws_bytes(L, n_ctx);
  if (need > kScratchBytes)
    return fail(RTP_EUNSUPPORTED,
                "rtp_decode_step_noalloc: this layer and context need %zu bytes of scratch; the library holds %zu "
                "(use rtp_decode_step with a workspace)", need, kScratchBytes);
  if ((st = enqueue_gate("rtp_decode_step_noalloc")) != RTP_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != RTP_OK) return st;
  return decode_step_impl(desc, n_ctx, q_pre, w_q_idx, w_head_stride, k_idx, idx_scale, q, k_cache, v_cache, k_loc,
                          v_loc, top_p, sm_scale, scores, row_max, row_sum, sel_idx, sel_count, sel_starts, out, ws,
                          kScratchBytes, stream, true);
}
