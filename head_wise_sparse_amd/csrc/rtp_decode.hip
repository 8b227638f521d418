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

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;           // log2 headroom before the reference max moves

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over the LPT consecutive lanes of a lane group (LPT = 8 or 16, inside one DPP row).
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror
  if (LPT == 16) v += dpp<0x140>(v);   // row_mirror
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct DecArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* sel_idx;     // sparse only
  const int32_t* starts;      // sparse only: [rows][nsplit + 1]
  float* part;                // [rows][nsplit][D + 2]
  int n_ctx;
  int64_t n_cap;
  int Hq, Hkv;
  int nsplit;
  float scale_log2;           // sm_scale * log2(e)
  int s_end, w_start, list_len;   // window only
  HeadMap map;
};

template <int D, int G, bool SPARSE>
__global__ __launch_bounds__(kDecThreads, 4) void k_decode_partial(DecArgs a) {
  constexpr int LPT = D / 8;            // lanes per cached row
  constexpr int TPW = 64 / LPT;         // rows per wave step
  constexpr int NLG = (kDecThreads / 64) * TPW;
  constexpr int RANGE = SPARSE ? kDecRange : kWinRange;
  constexpr int NW = kDecThreads / 64;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lg = wave * TPW + lane / LPT;
  const int li = lane % LPT;
  const int split = blockIdx.x, grp = blockIdx.y;
  const int b = grp / a.map.n, rr = grp % a.map.n, g = a.map.kv[rr];
  const uint16_t* kb = a.k + (int64_t(b) * a.Hkv + g) * a.n_cap * D + li * 8;
  const uint16_t* vb = a.v + (int64_t(b) * a.Hkv + g) * a.n_cap * D + li * 8;

  __shared__ uint16_t s_list[SPARSE ? RANGE : 1];
  __shared__ uint8_t s_lmask[SPARSE ? RANGE : 1];
  __shared__ uint32_t s_hm[SPARSE ? G * RANGE / 4 : 1];
  __shared__ int s_wcnt[NW];
  __shared__ float s_wm[NW][G], s_wl[NW][G];
  __shared__ float s_wacc[NW][G][D];

  uint32_t qw[G][4];
#pragma unroll
  for (int t = 0; t < G; ++t) {
    const uint4 qv = *reinterpret_cast<const uint4*>(a.q + (int64_t(b) * a.Hq + g * G + t) * D + li * 8);
    qw[t][0] = qv.x;
    qw[t][1] = qv.y;
    qw[t][2] = qv.z;
    qw[t][3] = qv.w;
  }

  int U, j0 = 0, p0 = 0;
  if constexpr (SPARSE) {
    j0 = split * RANGE;
    for (int i = tid; i < G * RANGE / 4; i += kDecThreads) s_hm[i] = 0;
    __syncthreads();
    uint8_t* hm = reinterpret_cast<uint8_t*>(s_hm);
    // A head's selected indices are distinct, so at most RANGE of them fall in the
    // range: SP per thread.  All loads are issued before any membership byte is set.
    constexpr int SP = RANGE / kDecThreads;
    int lo[G], hi[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
      const int64_t so = int64_t(grp * G + t) * (a.nsplit + 1) + split;
      // clamped: the range index may come from the caller
      hi[t] = min(max(a.starts[so + 1], 0), a.n_ctx);
      lo[t] = min(max(a.starts[so], 0), hi[t]);
    }
    int pos[G][SP];
#pragma unroll
    for (int t = 0; t < G; ++t) {
      const int32_t* sr = a.sel_idx + int64_t(grp * G + t) * a.n_cap;
#pragma unroll
      for (int u = 0; u < SP; ++u) {
        // unconditional load (index 0 stands in for out-of-range slots) so that the
        // compiler keeps every load in flight instead of waiting inside a branch
        const int k = lo[t] + u * kDecThreads + tid;
        const int v = sr[k < hi[t] ? k : 0];
        pos[t][u] = (k < hi[t]) ? v - j0 : -1;
      }
    }
#pragma unroll
    for (int t = 0; t < G; ++t)
#pragma unroll
      for (int u = 0; u < SP; ++u)
        if (pos[t][u] >= 0 && pos[t][u] < RANGE) hm[t * RANGE + pos[t][u]] = 1;
    __syncthreads();
    // ordered union of the G membership arrays: thread tid owns positions tid*8 .. tid*8+7
    constexpr int PER = RANGE / kDecThreads;
    uint8_t mk[PER];
    int c = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int p = tid * PER + e;
      uint32_t m = 0;
#pragma unroll
      for (int t = 0; t < G; ++t) m |= uint32_t(hm[t * RANGE + p]) << t;
      mk[e] = uint8_t(m);
      c += (m != 0);
    }
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_wcnt[wave] = incl;
    __syncthreads();
    int off = incl - c;
    int total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) off += s_wcnt[w];
      total += s_wcnt[w];
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (mk[e]) {
        s_list[off] = uint16_t(tid * PER + e);
        s_lmask[off] = mk[e];
        ++off;
      }
    }
    U = total;
    __syncthreads();
  } else {
    p0 = split * RANGE;
    U = min(RANGE, a.list_len - p0);
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int t = 0; t < G; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[t][i] = 0.0f;
  }

  auto token_of = [&](int e, uint32_t& mask) -> int64_t {
    if constexpr (SPARSE) {
      mask = s_lmask[e];
      return int64_t(j0) + s_list[e];
    } else {
      mask = (1u << G) - 1u;
      const int p = p0 + e;
      return p < a.s_end ? int64_t(p) : int64_t(a.w_start) + (p - a.s_end);
    }
  };

  auto consume = [&](const uint4& kv4, const uint4& vv4, uint32_t mask) {
    const uint32_t kw[4] = {kv4.x, kv4.y, kv4.z, kv4.w};
    float x[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) d = dot2(qw[t][i], kw[i], d);
      x[t] = group_sum<LPT>(d) * a.scale_log2;
    }
    const uint32_t vw[4] = {vv4.x, vv4.y, vv4.z, vv4.w};
    float vf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vf[2 * i] = bf16_lo(vw[i]);
      vf[2 * i + 1] = bf16_hi(vw[i]);
    }
#pragma unroll
    for (int t = 0; t < G; ++t) {
      if (mask & (1u << t)) {
        if (x[t] > m[t] + kLazy) {
          const float al = fast_exp2(m[t] - x[t]);
          l[t] *= al;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[t][i] *= al;
          m[t] = x[t];
        }
        const float p = fast_exp2(x[t] - m[t]);
        l[t] += p;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[t][i] = fmaf(p, vf[i], acc[t][i]);
      }
    }
  };

  // Software pipeline: kDecUnroll rows per lane group per stage, two register stages.
  // The loads of the next stage are issued before the current one is consumed, so
  // every wave keeps K/V loads in flight.  Loads are unconditional (list position
  // clamped to U-1; out-of-range rows get an empty head mask) so that none of them
  // waits inside a branch.
  constexpr int STEP = kDecUnroll * NLG;
  auto load_stage = [&](int base, uint4 (&kk)[kDecUnroll], uint4 (&vv)[kDecUnroll], uint32_t (&mk)[kDecUnroll]) {
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int e = base + u * NLG + lg;
      uint32_t msk;
      const int64_t j = token_of(e < U ? e : U - 1, msk);
      mk[u] = e < U ? msk : 0u;
      kk[u] = *reinterpret_cast<const uint4*>(kb + j * D);
      vv[u] = *reinterpret_cast<const uint4*>(vb + j * D);
    }
  };
  if (U > 0) {
    uint4 ka[kDecUnroll], va[kDecUnroll], kb2[kDecUnroll], vb2[kDecUnroll];
    uint32_t ma[kDecUnroll], mb[kDecUnroll];
    load_stage(0, ka, va, ma);
    for (int base = 0; base < U; base += 2 * STEP) {
      const bool more_b = base + STEP < U;
      if (more_b) load_stage(base + STEP, kb2, vb2, mb);
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) consume(ka[u], va[u], ma[u]);
      if (!more_b) break;
      if (base + 2 * STEP < U) load_stage(base + 2 * STEP, ka, va, ma);
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) consume(kb2[u], vb2[u], mb[u]);
    }
  }

  // ---- merge the lane groups of each wave, then the waves
#pragma unroll
  for (int t = 0; t < G; ++t) {
    float mw = m[t];
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1) mw = fmaxf(mw, __shfl_xor(mw, o, 64));
    const float f = (m[t] == -INFINITY) ? 0.0f : fast_exp2(m[t] - mw);
    float lw = l[t] * f;
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1) lw += __shfl_xor(lw, o, 64);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float y = acc[t][i] * f;
#pragma unroll
      for (int o = LPT; o < 64; o <<= 1) y += __shfl_xor(y, o, 64);
      acc[t][i] = y;
    }
    if (lane < LPT) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s_wacc[wave][t][li * 8 + i] = acc[t][i];
      if (lane == 0) {
        s_wm[wave][t] = mw;
        s_wl[wave][t] = lw;
      }
    }
  }
  __syncthreads();
  for (int o = tid; o < G * D; o += kDecThreads) {
    const int t = o / D, d = o % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_wm[w][t]);
    float A = 0.0f, Lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = (s_wm[w][t] == -INFINITY) ? 0.0f : fast_exp2(s_wm[w][t] - M);
      A += s_wacc[w][t][d] * f;
      Lsum += s_wl[w][t] * f;
    }
    float* pr = a.part + ((int64_t(grp) * G + t) * a.nsplit + split) * (D + 2);
    pr[d] = A;
    if (d == 0) {
      pr[D] = M;
      pr[D + 1] = Lsum;
    }
  }
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

// Combine the per-slice partials of one (batch, head) row into the bf16 output.
// 256 threads per row: SG = 256/D split groups, each thread sums the splits of its group
// for one output dimension (independent loads, unrolled), then the groups are combined.
template <int D>
__global__ __launch_bounds__(256) void k_decode_merge(const float* __restrict__ part, int nsplit, int G, int Hq,
                                                      HeadMap map, uint16_t* __restrict__ out) {
  constexpr int SG = 256 / D;
  const int row = blockIdx.x, tid = threadIdx.x;
  const int d = tid % D, sg = tid / D;
  const int grp = row / G, t = row % G;
  const int b = grp / map.n, rr = grp % map.n;
  const int h = map.kv[rr] * G + t;
  const float* pr = part + int64_t(row) * nsplit * (D + 2);
  __shared__ float s_red[4];
  __shared__ float s_a[SG][D], s_l[SG][D];
  // reference max over the splits
  float M = -INFINITY;
  for (int s = tid; s < nsplit; s += 256) M = fmaxf(M, pr[int64_t(s) * (D + 2) + D]);
  M = wave_max(M);
  if ((tid & 63) == 0) s_red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float A = 0.0f, Lsum = 0.0f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s = sg; s < nsplit; s += SG) {
      const float* ps = pr + int64_t(s) * (D + 2);
      const float ms = ps[D];
      const float f = (ms == -INFINITY) ? 0.0f : fast_exp2(ms - M);
      A = fmaf(ps[d], f, A);
      Lsum = fmaf(ps[D + 1], f, Lsum);
    }
  }
  s_a[sg][d] = A;
  s_l[sg][d] = Lsum;
  __syncthreads();
  if (sg == 0) {
#pragma unroll
    for (int i = 1; i < SG; ++i) {
      A += s_a[i][d];
      Lsum += s_l[i][d];
    }
    out[(int64_t(b) * Hq + h) * D + d] = f32_to_bf16(Lsum > 0.0f ? A / Lsum : 0.0f);
  }
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

rtp_status launch_merge(const Layer& L, int rows, int nsplit, const HeadMap& map, const float* part,
                        uint16_t* out, hipStream_t s) {
  if (L.D == 128)
    hipLaunchKernelGGL(k_decode_merge<128>, dim3(rows), dim3(256), 0, s, part, nsplit, L.G, L.Hq, map, out);
  else
    hipLaunchKernelGGL(k_decode_merge<64>, dim3(rows), dim3(256), 0, s, part, nsplit, L.G, L.Hq, map, out);
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
  if ((st = dispatch_partial<true>(L, dim3(nsplit, L.B * L.n_ret), s, a)) != RTP_OK) return st;
  return launch_merge(L, rows, nsplit, a.map, part, out, s);
}

extern "C" rtp_status rtp_window_sink_attn(const rtp_layer_desc* desc, int64_t n_ctx, const uint16_t* q,
                                           const uint16_t* k_cache, const uint16_t* v_cache, float sm_scale,
                                           uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
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
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t s_end = std::min<int64_t>(L.n_sinks, n_ctx);
  const int64_t w_start = std::max<int64_t>(n_ctx - L.window, s_end);
  const int64_t len = s_end + (n_ctx - w_start);
  const int nsplit = int((len + kWinRange - 1) / kWinRange);
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
  a.map = loc_map(L);
  if ((st = dispatch_partial<false>(L, dim3(nsplit, L.B * L.n_loc), s, a)) != RTP_OK) return st;
  return launch_merge(L, rows, nsplit, a.map, a.part, out, s);
}
