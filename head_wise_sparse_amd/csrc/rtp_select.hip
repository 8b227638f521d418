// rtp_topp_select: query-adaptive top-p token sets (abstract, observation (3):
// the useful token budget depends on the query, so a dynamic top-p rule replaces a
// fixed top-k; research-map summary, "Approach": query-adaptive top-p threshold).
//
// For one score row, rank tokens by score (higher first, equal scores by lower
// index) and keep the shortest prefix of the ranking whose softmax mass reaches p.
// The prefix is exactly {key(s_j) > t} plus the first r tokens (by index) with
// key(s_j) == t, where key() is the order-preserving uint32 image of the fp32
// score, t the threshold key and r a tie count.  The search runs in O(N):
//
//   level 0..2  radix histograms on key bits [31:21], [20:10], [9:0].  Each bin
//               carries the token count and the softmax mass in 2^-42 fixed point
//               (u64, so the sums are exact and independent of summation order).
//               Tokens outside the prefix resolved so far are skipped.  The last
//               block of each level (atomic ticket) scans the row's histogram from
//               the top and resolves the next digit.
//   compaction  every tile counts its "above" and "tied" tokens, gets the counts of
//               all earlier tiles through a decoupled look-back chain, and writes
//               its selected indices in increasing order.
#include <cmath>

#include "rtp_internal.hpp"

using namespace rtp;
using namespace rtp_dev;

namespace {

constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagIncl = 2ull << 62;

__device__ __forceinline__ uint64_t ld_acq(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rel(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_rlx(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_rlx(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct SelPtrs {
  uint64_t* mass;        // [rows][3][kBins]
  uint32_t* cnt;         // [rows][3][kBins]
  SelRowState* state;    // [rows]
  uint64_t* lookback;    // [rows][nblk]
  uint32_t* tile_ctr;    // [1]
};

__device__ __forceinline__ int level_shift(int level) { return level == 0 ? 21 : (level == 1 ? 10 : 0); }
__device__ __forceinline__ int level_bins(int level) { return level == 2 ? 1024 : 2048; }

// Zero every histogram, row state, look-back word and the tile counter.
__global__ __launch_bounds__(256) void k_sel_zero(uint4* __restrict__ p, size_t n16) {
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += size_t(gridDim.x) * 256) p[i] = z;
}

// Suffix scan of one histogram level by a whole block; resolves the digit where the
// cumulative mass from the top first reaches what is still needed.
__device__ void scan_level(const SelPtrs& P, int row, int level, float top_p, float row_m,
                           int32_t* __restrict__ sel_count) {
  const int tid = threadIdx.x;
  const int nb = level_bins(level);
  const int per = nb / kSelThreads;                    // 8 or 4 bins per thread
  const uint64_t* hm = P.mass + (int64_t(row) * 3 + level) * kBins;
  const uint32_t* hc = P.cnt + (int64_t(row) * 3 + level) * kBins;
  SelRowState* st = P.state + row;

  __shared__ uint64_t s_m[kSelThreads];
  __shared__ uint32_t s_c[kSelThreads];
  __shared__ uint64_t s_need, s_target, s_above;
  __shared__ uint32_t s_prefix, s_cnt_above;

  uint64_t bm[8];
  uint32_t bc[8];
  uint64_t tm = 0;
  uint32_t tc = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bm[i] = (i < per) ? ld_rlx(hm + tid * per + i) : 0ull;
    bc[i] = (i < per) ? ld_rlx(hc + tid * per + i) : 0u;
    tm += bm[i];
    tc += bc[i];
  }
  s_m[tid] = tm;
  s_c[tid] = tc;
  __syncthreads();
  if (tid == 0) {
    uint64_t need;
    if (level == 0) {
      uint64_t z = 0;
      for (int i = 0; i < kSelThreads; ++i) z += s_m[i];
      double tgt = ceil(double(top_p) * double(z));
      uint64_t t = tgt < 1.0 ? 1ull : (uint64_t)tgt;
      if (t > z) t = z;
      st->target = t;
      s_target = t;
      s_above = 0;
      s_cnt_above = 0;
      s_prefix = 0;
      need = t;
    } else {
      s_target = st->target;
      s_above = st->above;
      s_cnt_above = st->cnt_above;
      s_prefix = st->prefix;
      need = s_target - s_above;
    }
    s_need = need;
    // exclusive suffix sums over threads (thread i gets the sum of threads > i)
    uint64_t am = 0;
    uint32_t ac = 0;
    for (int i = kSelThreads - 1; i >= 0; --i) {
      const uint64_t m = s_m[i];
      const uint32_t c = s_c[i];
      s_m[i] = am;
      s_c[i] = ac;
      am += m;
      ac += c;
    }
  }
  __syncthreads();
  const uint64_t need = s_need;
  uint64_t suf = s_m[tid];
  uint32_t sufc = s_c[tid];
  // The owning thread is the one whose bins straddle `need`: suf < need <= suf + tm.
  if (suf < need && need <= suf + tm) {
    int d = 0;            // stays 0 only if the histogram were inconsistent
    bool found = false;
    uint32_t tied = bc[0];
#pragma unroll
    for (int k = 7; k >= 0; --k) {
      if (k < per && !found) {
        if (suf + bm[k] >= need) {
          found = true;
          d = k;
          tied = bc[k];
        } else {
          suf += bm[k];
          sufc += bc[k];
        }
      }
    }
    const uint32_t digit = uint32_t(tid * per + d);
    const uint32_t prefix = (level == 0) ? digit : ((s_prefix << (level == 1 ? 11 : 10)) | digit);
    const uint64_t above = s_above + suf;
    const uint32_t cnt_above = s_cnt_above + sufc;
    st->prefix = prefix;
    st->above = above;
    st->cnt_above = cnt_above;
    if (level == 2) {
      // prefix is now the full threshold key; tied tokens share one weight
      const uint64_t w = fixed_weight(key_score(prefix), row_m);
      const uint64_t rem = s_target - above;
      uint64_t r = (w == 0) ? tied : (rem + w - 1) / w;
      if (r < 1) r = 1;
      if (r > tied) r = tied;
      st->take_ties = uint32_t(r);
      sel_count[row] = int32_t(cnt_above + uint32_t(r));
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void k_sel_hist(const float* __restrict__ scores,
                                                          const float* __restrict__ row_max, SelPtrs P,
                                                          int level, int n_ctx, int64_t n_cap, int nblk,
                                                          float top_p, int32_t* __restrict__ sel_count) {
  const int tid = threadIdx.x;
  const int blk = blockIdx.x, row = blockIdx.y;
  __shared__ uint64_t h_m[kBins];
  __shared__ uint32_t h_c[kBins];
  __shared__ int s_last;
  const int nb = level_bins(level);
  for (int i = tid; i < nb; i += kSelThreads) {
    h_m[i] = 0;
    h_c[i] = 0;
  }
  const float m = row_max[row];
  const uint32_t prefix = level == 0 ? 0u : P.state[row].prefix;
  const int shift = level_shift(level);
  const int pshift = level == 0 ? 32 : (level == 1 ? 21 : 10);
  const uint32_t dmask = uint32_t(nb - 1);
  __syncthreads();

  const float* sp = scores + int64_t(row) * n_cap;
  const int64_t base = int64_t(blk) * kSelTile;
  float sv[kSelItems];
#pragma unroll
  for (int it = 0; it < kSelItems; ++it) {
    const int64_t j = base + it * kSelThreads + tid;
    sv[it] = (j < n_ctx) ? sp[j] : 0.0f;
  }
#pragma unroll
  for (int it = 0; it < kSelItems; ++it) {
    const int64_t j = base + it * kSelThreads + tid;
    if (j < n_ctx) {
      const uint32_t key = score_key(sv[it]);
      const bool match = (level == 0) || ((key >> pshift) == prefix);
      if (match) {
        const uint32_t d = (key >> shift) & dmask;
        atomicAdd(reinterpret_cast<unsigned long long*>(&h_m[d]), (unsigned long long)fixed_weight(sv[it], m));
        atomicAdd(&h_c[d], 1u);
      }
    }
  }
  __syncthreads();
  uint64_t* gm = P.mass + (int64_t(row) * 3 + level) * kBins;
  uint32_t* gc = P.cnt + (int64_t(row) * 3 + level) * kBins;
  for (int i = tid; i < nb; i += kSelThreads) {
    if (h_c[i]) {
      atomicAdd(reinterpret_cast<unsigned long long*>(gm + i), (unsigned long long)h_m[i]);
      atomicAdd(gc + i, h_c[i]);
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&P.state[row].done[level], 1u);
    s_last = (old == uint32_t(nblk - 1));
  }
  __syncthreads();
  if (s_last) {
    __threadfence();
    scan_level(P, row, level, top_p, m, sel_count);
  }
}

// Ordered compaction of {key > t} U {first r tokens with key == t}.
__global__ __launch_bounds__(kSelThreads) void k_sel_compact(const float* __restrict__ scores, SelPtrs P,
                                                             int n_ctx, int64_t n_cap, int nblk,
                                                             int32_t* __restrict__ sel_idx) {
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  __shared__ uint32_t s_id;
  __shared__ uint32_t s_wa[kSelItems][kSelThreads / 64], s_we[kSelItems][kSelThreads / 64];
  __shared__ uint32_t s_pa, s_pe;
  if (tid == 0) s_id = atomicAdd(P.tile_ctr, 1u);
  __syncthreads();
  const uint32_t id = s_id;
  const int row = int(id / uint32_t(nblk)), tile = int(id % uint32_t(nblk));
  const uint32_t t = P.state[row].prefix;
  const uint32_t r = P.state[row].take_ties;

  const float* sp = scores + int64_t(row) * n_cap;
  const int64_t base = int64_t(tile) * kSelTile;
  bool fa[kSelItems], fe[kSelItems];
#pragma unroll
  for (int it = 0; it < kSelItems; ++it) {
    const int64_t j = base + it * kSelThreads + tid;
    const float s = (j < n_ctx) ? sp[j] : 0.0f;
    const uint32_t key = score_key(s);
    fa[it] = (j < n_ctx) && key > t;
    fe[it] = (j < n_ctx) && key == t;
  }
  uint64_t ba[kSelItems], be[kSelItems];
#pragma unroll
  for (int it = 0; it < kSelItems; ++it) {
    ba[it] = __ballot(fa[it]);
    be[it] = __ballot(fe[it]);
    if (lane == 0) {
      s_wa[it][wave] = __popcll(ba[it]);
      s_we[it][wave] = __popcll(be[it]);
    }
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t a = 0, e = 0;
    for (int it = 0; it < kSelItems; ++it)
      for (int w = 0; w < kSelThreads / 64; ++w) {
        a += s_wa[it][w];
        e += s_we[it][w];
      }
    uint64_t* lb = P.lookback + int64_t(row) * nblk;
    uint64_t pa = 0, pe = 0;
    if (tile == 0) {
      st_rel(lb, kFlagIncl | (uint64_t(a) << 31) | e);
    } else {
      st_rel(lb + tile, kFlagAgg | (uint64_t(a) << 31) | e);
      int k = tile - 1;
      while (true) {
        const uint64_t v = ld_acq(lb + k);
        const uint64_t f = v >> 62;
        if (f == 0) {
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        pa += (v >> 31) & 0x7FFFFFFFull;
        pe += v & 0x7FFFFFFFull;
        if (f == 2) break;
        --k;
      }
      st_rel(lb + tile, kFlagIncl | ((pa + a) << 31) | (pe + e));
    }
    s_pa = uint32_t(pa);
    s_pe = uint32_t(pe);
  }
  __syncthreads();
  uint32_t ca = s_pa, ce = s_pe;              // counts of every earlier token
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* out = sel_idx + int64_t(row) * n_cap;
#pragma unroll
  for (int it = 0; it < kSelItems; ++it) {
    uint32_t wa = 0, we = 0;
    for (int w = 0; w < wave; ++w) {
      wa += s_wa[it][w];
      we += s_we[it][w];
    }
    const uint32_t a_before = ca + wa + __popcll(ba[it] & lt);
    const uint32_t e_before = ce + we + __popcll(be[it] & lt);
    const bool take = fa[it] || (fe[it] && e_before < r);
    if (take) {
      const uint32_t pos = a_before + (e_before < r ? e_before : r);
      out[pos] = int32_t(base + it * kSelThreads + tid);
    }
    for (int w = 0; w < kSelThreads / 64; ++w) {
      ca += s_wa[it][w];
      ce += s_we[it][w];
    }
  }
}

// top_p >= 1: every token, in order.
__global__ __launch_bounds__(256) void k_sel_all(int n_ctx, int64_t n_cap, int32_t* __restrict__ sel_idx,
                                                 int32_t* __restrict__ sel_count) {
  const int row = blockIdx.y;
  const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (j < n_ctx) sel_idx[int64_t(row) * n_cap + j] = int32_t(j);
  if (j == 0) sel_count[row] = n_ctx;
}

}  // namespace

extern "C" rtp_status rtp_topp_select(const rtp_layer_desc* desc, int64_t n_ctx, const float* scores,
                                      const float* row_max, const float* row_sum, float top_p, int32_t* sel_idx,
                                      int32_t* sel_count, void* ws, size_t ws_bytes, void* stream) {
  (void)row_sum;
  Layer L;
  rtp_status st = check_desc(desc, &L);
  if (st != RTP_OK) return st;
  if (n_ctx < 1 || n_ctx > L.n_cap)
    return fail(RTP_EINVAL, "n_ctx must be in [1, n_cap=%lld] (got %lld)", (long long)L.n_cap, (long long)n_ctx);
  if (!(top_p > 0.0f)) return fail(RTP_EINVAL, "top_p must be > 0 (got %g)", double(top_p));
  if (L.n_ret == 0) return ok();
  if (!scores || !row_max || !sel_idx || !sel_count) return fail(RTP_EINVAL, "rtp_topp_select: NULL tensor pointer");
  if (!aligned(scores, 16) || !aligned(sel_idx, 16))
    return fail(RTP_EINVAL, "rtp_topp_select: tensors must be 16-byte aligned");
  const int rows = L.B * L.n_ret * L.G;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (top_p >= 1.0f) {
    hipLaunchKernelGGL(k_sel_all, dim3(unsigned((n_ctx + 255) / 256), rows), dim3(256), 0, s, int(n_ctx), L.n_cap,
                       sel_idx, sel_count);
    return check_launch("k_sel_all");
  }
  const SelLayout lay = sel_layout(L, n_ctx);
  if (!ws || ws_bytes < lay.total || !aligned(ws, 256))
    return fail(RTP_EWORKSPACE, "rtp_topp_select: workspace needs %zu bytes, 256-aligned (got %zu)", lay.total,
                ws_bytes);
  char* w = static_cast<char*>(ws);
  SelPtrs P{reinterpret_cast<uint64_t*>(w + lay.hist_mass), reinterpret_cast<uint32_t*>(w + lay.hist_cnt),
            reinterpret_cast<SelRowState*>(w + lay.state), reinterpret_cast<uint64_t*>(w + lay.lookback),
            reinterpret_cast<uint32_t*>(w + lay.tile_ctr)};
  const size_t n16 = lay.total / 16;
  const unsigned zb = unsigned(std::min<size_t>((n16 + 255) / 256, 2048));
  hipLaunchKernelGGL(k_sel_zero, dim3(zb), dim3(256), 0, s, reinterpret_cast<uint4*>(ws), n16);
  if ((st = check_launch("k_sel_zero")) != RTP_OK) return st;
  const dim3 grid(lay.nblk, rows);
  for (int level = 0; level < 3; ++level) {
    hipLaunchKernelGGL(k_sel_hist, grid, dim3(kSelThreads), 0, s, scores, row_max, P, level, int(n_ctx), L.n_cap,
                       lay.nblk, top_p, sel_count);
    if ((st = check_launch("k_sel_hist")) != RTP_OK) return st;
  }
  hipLaunchKernelGGL(k_sel_compact, dim3(unsigned(lay.nblk) * unsigned(rows)), dim3(kSelThreads), 0, s, scores, P,
                     int(n_ctx), L.n_cap, lay.nblk, sel_idx);
  return check_launch("k_sel_compact");
}
