// Decode attention for both head kinds.
//
//  rtp_sparse_decode_attn  retrieval heads attend only over their selected tokens
//                          (abstract: full KV kept for retrieval heads, token indexer
//                          for sparse attention).
//  rtp_window_sink_attn    local heads attend over sinks plus a sliding window
//                          (research-map summary, "Approach").
//
// Both are split-K flash decoding.  A block owns one GQA group (batch b, KV head g)
// and one slice of that group's token list; it reads each cached K/V row of the
// slice from HBM once and applies it to all G query heads of the group.  For the
// sparse path the slice is a token-index range [j0, j0+1024): the block unions the
// G heads' selected sets inside the range (per-head membership bytes in LDS, then
// an ordered compaction into an LDS token list with a G-bit head mask per token),
// so a row chosen by several heads of the group is loaded once.  For the window
// path the list is implicit: [0, sinks) U [n_ctx - window, n_ctx).
//
// Inner loop: 16 lanes (D=128; 8 lanes for D=64) hold one cached row, 8 bf16 each
// (one 16-byte load of K and one of V per lane).  q.k uses v_dot2_f32_bf16 on the
// raw bf16 pairs, reduced across the lane group with DPP adds; the online softmax
// runs in the exp2 domain with a lazy rescale (the running reference only moves
// when a logit exceeds it by more than 2^8).  Each block emits, per head, the
// unnormalised accumulator, its reference max and its sum; a merge kernel combines
// the slices (log-sum-exp merge) and rounds the output to bf16.
#include <cmath>

#include "rtp_internal.hpp"

using namespace rtp;
using namespace rtp_dev;

#include "decode_dev.hpp"

namespace {

template <int D, int G, bool SPARSE>
__global__ __launch_bounds__(kDecThreads, 4) void k_decode_partial(DecArgs a) {
  decode_block<D, G, SPARSE>(a, blockIdx.x, blockIdx.y);
}

// Start position, in each selected list, of every token-index range of kDecRange
// tokens (the lists are increasing): starts[row][s] = #{k : sel[k] < s*kDecRange}.
__global__ __launch_bounds__(256) void k_range_starts(const int32_t* __restrict__ sel_idx,
                                                      const int32_t* __restrict__ sel_count,
                                                      int32_t* __restrict__ starts, int64_t n_cap, int n_ctx,
                                                      int nsplit) {
  const int row = blockIdx.y;
  const int cnt = min(max(sel_count[row], 0), n_ctx);
  const int32_t* sr = sel_idx + int64_t(row) * n_cap;
  int32_t* so = starts + int64_t(row) * (nsplit + 1);
  for (int k = blockIdx.x * 256 + threadIdx.x; k <= cnt; k += gridDim.x * 256) {
    int rk = (k == cnt) ? nsplit : sr[k] / kDecRange;
    int rp = (k == 0) ? -1 : sr[k - 1] / kDecRange;
    rk = min(max(rk, 0), nsplit);
    rp = min(max(rp, -1), nsplit);
    for (int q = rp + 1; q <= rk; ++q) so[q] = k;
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_decode_merge(MergeArgs ma) {
  merge_row<D>(ma, blockIdx.x);
}

template <int D, int G, bool SPARSE>
void launch_partial(dim3 grid, hipStream_t s, const DecArgs& a) {
  hipLaunchKernelGGL((k_decode_partial<D, G, SPARSE>), grid, dim3(kDecThreads), 0, s, a);
}

template <bool SPARSE>
rtp_status dispatch_partial(const Layer& L, dim3 grid, hipStream_t s, const DecArgs& a) {
#define RTP_DEC_CASE(DD, GG) \
  if (L.D == DD && L.G == GG) { launch_partial<DD, GG, SPARSE>(grid, s, a); return check_launch("k_decode_partial"); }
  RTP_DEC_CASE(64, 1) RTP_DEC_CASE(64, 2) RTP_DEC_CASE(64, 4) RTP_DEC_CASE(64, 8)
  RTP_DEC_CASE(128, 1) RTP_DEC_CASE(128, 2) RTP_DEC_CASE(128, 4) RTP_DEC_CASE(128, 8)
#undef RTP_DEC_CASE
  return fail(RTP_EUNSUPPORTED, "decode: unsupported head_dim/group");
}

template <int D>
__global__ __launch_bounds__(256) void k_decode_merge_pre(MergeArgs ma, float* part2, int nchunks) {
  merge_pre_chunk<D>(ma, part2, nchunks, blockIdx.y, blockIdx.x);
}

// part2: second-level partials for rows with more than kMergeDirect splits (else unused)
rtp_status launch_merge(const Layer& L, int rows, int nsplit, const HeadMap& map, const float* part,
                        uint16_t* out, hipStream_t s, float* part2 = nullptr) {
  const int nchunks = part2 ? merge_chunks(nsplit) : 0;
  if (nchunks) {
    const MergeArgs m1{part, nsplit, L.G, L.Hq, map, out};
    if (L.D == 128)
      hipLaunchKernelGGL(k_decode_merge_pre<128>, dim3(nchunks, rows), dim3(256), 0, s, m1, part2, nchunks);
    else
      hipLaunchKernelGGL(k_decode_merge_pre<64>, dim3(nchunks, rows), dim3(256), 0, s, m1, part2, nchunks);
    rtp_status st = check_launch("k_decode_merge_pre");
    if (st != RTP_OK) return st;
    part = part2;
    nsplit = nchunks;
  }
  const MergeArgs ma{part, nsplit, L.G, L.Hq, map, out};
  if (L.D == 128)
    hipLaunchKernelGGL(k_decode_merge<128>, dim3(rows), dim3(256), 0, s, ma);
  else
    hipLaunchKernelGGL(k_decode_merge<64>, dim3(rows), dim3(256), 0, s, ma);
  return check_launch("k_decode_merge");
}

rtp_status check_common(const Layer& L, int64_t n_ctx, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        uint16_t* out, float sm_scale, const char* who) {
  if (n_ctx < 1 || n_ctx > L.n_cap)
    return fail(RTP_EINVAL, "%s: n_ctx must be in [1, n_cap=%lld] (got %lld)", who, (long long)L.n_cap,
                (long long)n_ctx);
  if (!q || !k || !v || !out) return fail(RTP_EINVAL, "%s: NULL tensor pointer", who);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 2))
    return fail(RTP_EINVAL, "%s: q/k/v must be 16-byte aligned", who);
  if (!std::isfinite(sm_scale)) return fail(RTP_EINVAL, "%s: sm_scale must be finite", who);
  return ok();
}

}  // namespace

extern "C" rtp_status rtp_sparse_decode_attn(const rtp_layer_desc* desc, int64_t n_ctx, const uint16_t* q,
                                             const uint16_t* k_cache, const uint16_t* v_cache,
                                             const int32_t* sel_idx, const int32_t* sel_count,
                                             const int32_t* sel_starts, float sm_scale, uint16_t* out, void* ws,
                                             size_t ws_bytes, void* stream) {
  TraceRange trace_("rtp_sparse_decode_attn");
  Layer L;
  rtp_status st = check_desc(desc, &L);
  if (st != RTP_OK) return st;
  if ((st = check_common(L, n_ctx, q, k_cache, v_cache, out, sm_scale, "rtp_sparse_decode_attn")) != RTP_OK)
    return st;
  if (L.n_ret == 0) return ok();
  if (!sel_idx || !sel_count) return fail(RTP_EINVAL, "rtp_sparse_decode_attn: NULL selection pointer");
  const size_t need = dec_ws_bytes(L, n_ctx, true);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(RTP_EWORKSPACE, "rtp_sparse_decode_attn: workspace needs %zu bytes, 256-aligned (got %zu)", need,
                ws_bytes);
  if ((st = enqueue_gate("rtp_sparse_decode_attn")) != RTP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int nsplit = int((n_ctx + kDecRange - 1) / kDecRange);
  const int rows = L.B * L.n_ret * L.G;
  float* part = static_cast<float*>(ws);
  const int32_t* starts = sel_starts;
  if (!starts) {
    int32_t* built = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + dec_sparse_starts_offset(L, n_ctx));
    const unsigned sb = unsigned(std::min<int64_t>((n_ctx + 256) / 256, 64));
    hipLaunchKernelGGL(k_range_starts, dim3(sb, rows), dim3(256), 0, s, sel_idx, sel_count, built, L.n_cap,
                       int(n_ctx), nsplit);
    if ((st = check_launch("k_range_starts")) != RTP_OK) return st;
    starts = built;
  }
  DecArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.sel_idx = sel_idx;
  a.starts = starts;
  a.part = part;
  a.n_ctx = int(n_ctx);
  a.n_cap = L.n_cap;
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.nsplit = nsplit;
  a.scale_log2 = sm_scale * kLog2e;
  a.map = ret_map(L);
  set_sparse_cache(a, L);
  if ((st = dispatch_partial<true>(L, dim3(nsplit * a.nsub, L.B * L.n_ret), s, a)) != RTP_OK) return st;
  return launch_merge(L, rows, nsplit * a.nsub, a.map, part, out, s,
                      reinterpret_cast<float*>(static_cast<char*>(ws) + dec_sparse_part2_offset(L, n_ctx)));
}

extern "C" rtp_status rtp_window_sink_attn(const rtp_layer_desc* desc, int64_t n_ctx, const uint16_t* q,
                                           const uint16_t* k_cache, const uint16_t* v_cache, float sm_scale,
                                           uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  TraceRange trace_("rtp_window_sink_attn");
  Layer L;
  rtp_status st = check_desc(desc, &L);
  if (st != RTP_OK) return st;
  if ((st = check_common(L, n_ctx, q, k_cache, v_cache, out, sm_scale, "rtp_window_sink_attn")) != RTP_OK)
    return st;
  if (L.n_loc == 0) return ok();
  const size_t need = dec_ws_bytes(L, n_ctx, false);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(RTP_EWORKSPACE, "rtp_window_sink_attn: workspace needs %zu bytes, 256-aligned (got %zu)", need,
                ws_bytes);
  if ((st = enqueue_gate("rtp_window_sink_attn")) != RTP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t s_end = std::min<int64_t>(L.n_sinks, n_ctx);
  const int64_t w_start = std::max<int64_t>(n_ctx - L.window, s_end);
  const int64_t len = s_end + (n_ctx - w_start);
  const int wr = win_range_for(L, n_ctx, len);
  const int nsplit = int((len + wr - 1) / wr);
  const int rows = L.B * L.n_loc * L.G;
  DecArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.part = static_cast<float*>(ws);
  a.n_ctx = int(n_ctx);
  a.n_cap = L.n_cap;
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.nsplit = nsplit;
  a.scale_log2 = sm_scale * kLog2e;
  a.s_end = int(s_end);
  a.w_start = int(w_start);
  a.list_len = int(len);
  a.wrange = wr;
  a.map = loc_map(L);
  set_window_cache(a, L);
  if ((st = dispatch_partial<false>(L, dim3(nsplit, L.B * L.n_loc), s, a)) != RTP_OK) return st;
  return launch_merge(L, rows, nsplit, a.map, a.part, out, s);
}
