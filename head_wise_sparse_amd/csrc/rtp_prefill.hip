// rtp_prefill_attn: host validation (kernels follow).
#include <cmath>

#include "rtp_internal.hpp"

using namespace rtp;

namespace rtp {
size_t prefill_ws_bytes(const Layer& L, int64_t C) {
  (void)L;
  (void)C;
  return 256;
}
}  // namespace rtp

extern "C" rtp_status rtp_prefill_attn(const rtp_layer_desc* desc, int64_t c0, int32_t C, const uint16_t* q,
                                       const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_pre,
                                       const uint16_t* w_k_idx, int64_t w_head_stride, uint16_t* k_idx_cache,
                                       float sm_scale, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  Layer L;
  rtp_status st = check_desc(desc, &L);
  if (st != RTP_OK) return st;
  if (L.B != 1) return fail(RTP_EINVAL, "rtp_prefill_attn: batch must be 1 (got %d)", L.B);
  if (C < 1) return fail(RTP_EINVAL, "rtp_prefill_attn: C must be >= 1 (got %d)", C);
  if (c0 < 0 || c0 + C > L.n_cap)
    return fail(RTP_EINVAL, "rtp_prefill_attn: need 0 <= c0 and c0 + C <= n_cap (c0=%lld, C=%d, n_cap=%lld)",
                (long long)c0, C, (long long)L.n_cap);
  return fail(RTP_EUNSUPPORTED, "rtp_prefill_attn: not available in this build");
}
