// rtp_indexer_score: 16-dim pre-RoPE indexer scores for every cached token and
// every retrieval query head, plus the softmax statistics (max, sum of exp) of each
// score row.  (Abstract, observation (2): long-range retrieval through a
// 16-dimensional indexer; research-map summary, "Approach": low-dimensional
// pre-RoPE projection.)
//
// Work split: one block per (token tile of 2048, batch b, retrieval KV head r).
// The 32-byte indexer key of each token is read from HBM once and scored against
// all G query heads of the GQA group (the G score rows share that key stream).
// Per-block (max, sum) partials are combined by a one-wave finalize kernel.
#include <cmath>

#include "rtp_internal.hpp"

using namespace rtp;
using namespace rtp_dev;

#include "score_dev.hpp"

namespace {

template <int G, int D, int IDX>
__global__ __launch_bounds__(kScoreThreads) void k_indexer_score(ScoreArgs A) {
  score_block<G, D, IDX>(A, blockIdx.x, blockIdx.y);
}

// One wave per score row: combine the per-block partials into (row_max, row_sum).
__global__ __launch_bounds__(64) void k_score_finalize(const float2* __restrict__ part, int nblk,
                                                       float* __restrict__ row_max, float* __restrict__ row_sum) {
  score_finalize_row(part, nblk, nblk, row_max, row_sum, blockIdx.x);
}

template <int G, int D, int IDX>
void launch_score(dim3 grid, hipStream_t st, const ScoreArgs& A) {
  hipLaunchKernelGGL((k_indexer_score<G, D, IDX>), grid, dim3(kScoreThreads), 0, st, A);
}

template <int IDX>
bool dispatch_score(const Layer& L, dim3 grid, hipStream_t s, const ScoreArgs& A) {
#define RTP_SCORE_CASE(GG, DD)                      \
  if (L.G == GG && L.D == DD) {                     \
    launch_score<GG, DD, IDX>(grid, s, A);          \
    return true;                                    \
  }
  RTP_SCORE_CASE(1, 64) RTP_SCORE_CASE(2, 64) RTP_SCORE_CASE(4, 64)
  RTP_SCORE_CASE(1, 128) RTP_SCORE_CASE(2, 128) RTP_SCORE_CASE(4, 128)
  if constexpr (IDX <= 16) {
    RTP_SCORE_CASE(8, 64) RTP_SCORE_CASE(8, 128)
  }
#undef RTP_SCORE_CASE
  return false;
}

}  // namespace

extern "C" rtp_status rtp_indexer_score(const rtp_layer_desc* desc, int64_t n_ctx, const uint16_t* q_pre,
                                        const uint16_t* w_q_idx, int64_t w_head_stride, const uint16_t* k_idx,
                                        float idx_scale, float* scores, float* row_max, float* row_sum, void* ws,
                                        size_t ws_bytes, void* stream) {
  TraceRange trace_("rtp_indexer_score");
  Layer L;
  rtp_status st = check_desc(desc, &L);
  if (st != RTP_OK) return st;
  if (n_ctx < 1 || n_ctx > L.n_cap)
    return fail(RTP_EINVAL, "n_ctx must be in [1, n_cap=%lld] (got %lld)", (long long)L.n_cap, (long long)n_ctx);
  if (L.n_ret == 0) return ok();
  if (!q_pre || !w_q_idx || !k_idx || !scores || !row_max || !row_sum)
    return fail(RTP_EINVAL, "rtp_indexer_score: NULL tensor pointer");
  if (w_head_stride < 0 || w_head_stride % 8 != 0)
    return fail(RTP_EINVAL, "w_head_stride must be a non-negative multiple of 8 (got %lld)",
                (long long)w_head_stride);
  if (!std::isfinite(idx_scale)) return fail(RTP_EINVAL, "idx_scale must be finite");
  if (!aligned(k_idx, 16) || !aligned(scores, 16) || !aligned(q_pre, 16) || !aligned(w_q_idx, 16))
    return fail(RTP_EINVAL, "rtp_indexer_score: tensors must be 16-byte aligned");
  const size_t need = score_ws_bytes(L, n_ctx);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(RTP_EWORKSPACE, "rtp_indexer_score: workspace needs %zu bytes, 256-aligned (got %zu)", need,
                ws_bytes);

  const int nblk = int((n_ctx + score_tile(L.idx) - 1) / score_tile(L.idx));
  const dim3 grid(nblk, L.B * L.n_ret);
  if ((st = enqueue_gate("rtp_indexer_score")) != RTP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float2* part = reinterpret_cast<float2*>(ws);
  const ScoreArgs A{q_pre, w_q_idx, w_head_stride, k_idx, idx_scale, scores, part, int(n_ctx), nullptr, L.n_cap,
                    L.Hq, ret_map(L), nblk};
  bool launched = false;
  switch (L.idx) {
    case 4: launched = dispatch_score<4>(L, grid, s, A); break;
    case 8: launched = dispatch_score<8>(L, grid, s, A); break;
    case 16: launched = dispatch_score<16>(L, grid, s, A); break;
    case 32: launched = dispatch_score<32>(L, grid, s, A); break;
  }
  if (!launched) return fail(RTP_EUNSUPPORTED, "rtp_indexer_score: unsupported head_dim/group/idx_dim");
  if ((st = check_launch("k_indexer_score")) != RTP_OK) return st;
  hipLaunchKernelGGL(k_score_finalize, dim3(L.B * L.n_ret * L.G), dim3(64), 0, s, part, nblk, row_max, row_sum);
  return check_launch("k_score_finalize");
}
