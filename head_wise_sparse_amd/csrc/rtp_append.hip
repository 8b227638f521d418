// rtp_append_token: store one new token of every sequence in the caches a decode step
// reads -- its post-RoPE key and value (every head), and for retrieval heads its
// 16-dim pre-RoPE indexer key (abstract, observation (2); research-map summary,
// "Approach": only retrieval heads keep the whole history, local heads keep their sinks
// and window).
//
// One block per (batch, KV head): 16 lanes copy the 256-byte K and V rows, and for a
// retrieval head 64 lanes form the 16 projections (4 lanes per output, fp32
// accumulation, one bf16 rounding to nearest even).
#include "rtp_internal.hpp"

using namespace rtp;
using namespace rtp_dev;

namespace {

struct AppendArgs {
  int64_t pos;
  int64_t* gen;                // device-length variant: {pos, n_ctx} (pos read here, n_ctx = pos + 1 written)
  int64_t n_sinks, window;
  const uint16_t* k_new;       // [B][Hkv][D]
  const uint16_t* v_new;
  const uint16_t* k_pre;       // [B][Hkv][D]
  const uint16_t* w_k;         // [Hkv_r][D][16], w_stride elements apart
  int64_t w_stride;
  uint16_t* k_ret;             // full: [B][Hkv][n_cap][D]; compact: [B][Hkv_r][n_cap][D]
  uint16_t* v_ret;
  uint16_t* k_idx;             // [B][Hkv_r][n_cap][16]
  uint16_t* k_loc;             // compact: [B][Hkv_l][n_sinks + window][D]
  uint16_t* v_loc;
  int Hkv, D, n_ret, n_loc, idx;
  int64_t n_cap;
  int compact;
  int64_t ring_rows;           // compact: rows per local head (n_sinks + window)
  int64_t loc_row;             // compact: ring row of `pos`
  int rank[kMaxHeads];         // KV head -> rank within its kind
  uint8_t role[kMaxHeads];     // 1 = retrieval
};

__global__ __launch_bounds__(64) void k_append(AppendArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const bool ret = a.role[g];
  const int r = a.rank[g];
  const int64_t src = (int64_t(b) * a.Hkv + g) * a.D;
  int64_t pos = a.pos, loc_row = a.loc_row;
  if (a.gen) {               // the position from the generation state; the next decode sees pos + 1
    pos = a.gen[0];
    if (g == 0 && b == 0 && lane == 0) a.gen[1] = pos + 1 < 1 ? 1 : (pos + 1 > a.n_cap ? a.n_cap : pos + 1);
    if (pos < 0 || pos >= a.n_cap) return;                 // outside the cache: nothing is written
    loc_row = pos < a.n_sinks ? pos : a.n_sinks + (pos - a.n_sinks) % a.window;
  }
  uint16_t *kd, *vd;
  if (!a.compact) {
    kd = a.k_ret + ((int64_t(b) * a.Hkv + g) * a.n_cap + pos) * a.D;
    vd = a.v_ret + ((int64_t(b) * a.Hkv + g) * a.n_cap + pos) * a.D;
  } else if (ret) {
    kd = a.k_ret + ((int64_t(b) * a.n_ret + r) * a.n_cap + pos) * a.D;
    vd = a.v_ret + ((int64_t(b) * a.n_ret + r) * a.n_cap + pos) * a.D;
  } else {
    kd = a.k_loc + ((int64_t(b) * a.n_loc + r) * a.ring_rows + loc_row) * a.D;
    vd = a.v_loc + ((int64_t(b) * a.n_loc + r) * a.ring_rows + loc_row) * a.D;
  }
  const int nv = a.D / 8;                  // 16-byte pieces per row
  if (lane < nv) {
    reinterpret_cast<uint4*>(kd)[lane] = reinterpret_cast<const uint4*>(a.k_new + src)[lane];
    reinterpret_cast<uint4*>(vd)[lane] = reinterpret_cast<const uint4*>(a.v_new + src)[lane];
  }
  if (!ret) return;
  // k_idx[b][r][pos][c] = bf16(sum_d k_pre[d] * W[r][d][c]).  The key row and the matrix
  // are staged in LDS with 16-byte loads (all in flight at once); then the 64 / idx lanes
  // of output c split d and a lane-group sum closes the dot product.
  __shared__ uint4 s_w[128 * 32 / 8];
  __shared__ uint4 s_kp[128 / 8];
  const uint4* wg = reinterpret_cast<const uint4*>(a.w_k + int64_t(r) * a.w_stride);
  const int nw = a.D * a.idx / 8;
#pragma unroll 8
  for (int i = lane; i < nw; i += 64) s_w[i] = wg[i];
  if (lane < a.D / 8) s_kp[lane] = reinterpret_cast<const uint4*>(a.k_pre + src)[lane];
  __syncthreads();
  const uint16_t* w = reinterpret_cast<const uint16_t*>(s_w);
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(s_kp);
  const int lpo = 64 / a.idx;
  const int c = lane / lpo, part = lane % lpo;
  float acc = 0.0f;
  for (int d = part; d < a.D; d += lpo) acc = fmaf(bf16_to_f32(kp[d]), bf16_to_f32(w[d * a.idx + c]), acc);
  for (int o = 1; o < lpo; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (part == 0) a.k_idx[((int64_t(b) * a.n_ret + r) * a.n_cap + pos) * a.idx + c] = f32_to_bf16(acc);
}

}  // namespace

namespace {

rtp_status append_impl(const rtp_layer_desc* desc, int64_t pos, int64_t* gen, const uint16_t* k_new,
                       const uint16_t* v_new, const uint16_t* k_pre, const uint16_t* w_k_idx, int64_t w_head_stride,
                       uint16_t* k_cache, uint16_t* v_cache, uint16_t* k_idx_cache, uint16_t* k_loc,
                       uint16_t* v_loc, void* stream) {
  Layer L;
  rtp_status st = check_desc(desc, &L);
  if (st != RTP_OK) return st;
  if (!gen && (pos < 0 || pos >= L.n_cap))
    return fail(RTP_EINVAL, "rtp_append_token: pos must be in [0, n_cap=%lld) (got %lld)", (long long)L.n_cap,
                (long long)pos);
  if (gen && !aligned(gen, 8))
    return fail(RTP_EINVAL, "rtp_append_token_dev: the generation state must be 8-byte aligned");
  const bool compact = L.kv_layout == RTP_KV_COMPACT;
  if (!k_new || !v_new) return fail(RTP_EINVAL, "rtp_append_token: NULL tensor pointer");
  if ((L.n_ret || !compact) && (!k_cache || !v_cache)) return fail(RTP_EINVAL, "rtp_append_token: NULL cache");
  if (compact && L.n_loc && (!k_loc || !v_loc)) return fail(RTP_EINVAL, "rtp_append_token: NULL local ring");
  if (L.n_ret && (!k_pre || !w_k_idx || !k_idx_cache)) return fail(RTP_EINVAL, "rtp_append_token: NULL indexer");
  if (w_head_stride < 0 || w_head_stride % 8 != 0)
    return fail(RTP_EINVAL, "w_head_stride must be a non-negative multiple of 8 (got %lld)", (long long)w_head_stride);
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(k_loc, 16) || !aligned(v_loc, 16) || !aligned(k_idx_cache, 2) || !aligned(k_pre, 16) ||
      !aligned(w_k_idx, 16))
    return fail(RTP_EINVAL, "rtp_append_token: tensors must be 16-byte aligned");
  AppendArgs a{};
  a.pos = pos;
  a.gen = gen;
  a.n_sinks = L.n_sinks;
  a.window = L.window;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pre = k_pre;
  a.w_k = w_k_idx;
  a.w_stride = w_head_stride;
  a.k_ret = k_cache;
  a.v_ret = v_cache;
  a.k_idx = k_idx_cache;
  a.k_loc = k_loc;
  a.v_loc = v_loc;
  a.Hkv = L.Hkv;
  a.D = L.D;
  a.n_ret = L.n_ret;
  a.n_loc = L.n_loc;
  a.n_cap = L.n_cap;
  a.idx = L.idx;
  a.compact = compact;
  const int64_t S = L.n_sinks, W = L.window;
  a.ring_rows = S + W;
  a.loc_row = gen ? 0 : (pos < S ? pos : S + (pos - S) % W);
  for (int i = 0; i < L.n_ret; ++i) {
    a.rank[L.ret_kv[i]] = i;
    a.role[L.ret_kv[i]] = 1;
  }
  for (int i = 0; i < L.n_loc; ++i) {
    a.rank[L.loc_kv[i]] = i;
    a.role[L.loc_kv[i]] = 0;
  }
  if ((st = enqueue_gate("rtp_append_token")) != RTP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_append, dim3(L.Hkv, L.B), dim3(64), 0, s, a);
  return check_launch("k_append");
}

}  // namespace

extern "C" rtp_status rtp_append_token(const rtp_layer_desc* desc, int64_t pos, const uint16_t* k_new,
                                       const uint16_t* v_new, const uint16_t* k_pre, const uint16_t* w_k_idx,
                                       int64_t w_head_stride, uint16_t* k_cache, uint16_t* v_cache,
                                       uint16_t* k_idx_cache, uint16_t* k_loc, uint16_t* v_loc, void* stream) {
  TraceRange trace_("rtp_append_token");
  return append_impl(desc, pos, nullptr, k_new, v_new, k_pre, w_k_idx, w_head_stride, k_cache, v_cache, k_idx_cache,
                     k_loc, v_loc, stream);
}

extern "C" rtp_status rtp_append_token_dev(const rtp_layer_desc* desc, int64_t* gen, const uint16_t* k_new,
                                           const uint16_t* v_new, const uint16_t* k_pre, const uint16_t* w_k_idx,
                                           int64_t w_head_stride, uint16_t* k_cache, uint16_t* v_cache,
                                           uint16_t* k_idx_cache, uint16_t* k_loc, uint16_t* v_loc, void* stream) {
  TraceRange trace_("rtp_append_token_dev");
  if (!gen) return fail(RTP_EINVAL, "rtp_append_token_dev: NULL generation state");
  return append_impl(desc, 0, gen, k_new, v_new, k_pre, w_k_idx, w_head_stride, k_cache, v_cache, k_idx_cache, k_loc,
                     v_loc, stream);
}
