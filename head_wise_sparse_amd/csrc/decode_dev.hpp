// Device bodies of the split-K decode attention and of the split merge (shared by
// the decode calls and the fused decode step).  See rtp_decode.hip for the design.
#pragma once

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
  // sparse, members taken from the scores (the decode step): the scores [rows][n_cap], the
  // threshold key of every row, and the lists to write (null: not written); all_tokens:
  // every token of the context is a member (top_p >= 1)
  const float* scores;
  const uint32_t* thr;
  int32_t* sel_out;
  int all_tokens;
  float* part;                // [rows][nsplit * nsub][D + 4]: accumulator, max, sum (16-byte rows)
  int n_ctx;                  // the context (device-length step: its bound n_max)
  const int64_t* live;        // device-length step: the context's device word, else null
  int n_sinks, window;        // window path: the layer's sinks and window (live list bounds)
  int64_t n_cap;
  int Hq, Hkv;
  int nsplit;                 // sparse: index ranges of n_ctx (row stride of `starts` is nsplit + 1);
                              // window: slices of the bound's list (the partials' row stride)
  int nsub;                   // sparse: blocks per range, each taking one slice of its union list
  int wrange;                 // window: list positions per block
  float scale_log2;           // sm_scale * log2(e)
  int s_end, w_start, list_len;   // window only
  HeadMap map;
  // cache addressing: head index = rank (compact layout) or KV head; rows per head;
  // ring_w > 0: a local ring (token j >= ring_s at row ring_s + (j - ring_s) % ring_w)
  int cache_heads;
  int by_rank;
  int64_t cache_rows;
  int ring_s, ring_w;
  int ring_off;               // (w_start - ring_s) % ring_w: ring row of the first window token
};

// One block of split-K decode: partial slot `slot` of group `grp` (= b * n_heads_of_kind
// + rank).  Sparse path: slot = range * nsub + sub; the block builds the union list of
// index range `range` and takes the sub-th of nsub equal slices of it (whole stages).
// A head's members of the range come from its selected list (FROM_SCORES false) or, in
// the decode step, from its scores, threshold key t and range index (FROM_SCORES true):
// every token with key > t, and the first (starts[q+1] - starts[q] - #above) tokens with
// key == t, which is the list the compaction writes.  The block with sub == 0 writes that
// part of the list, last.
template <int D, int G, bool SPARSE, bool FROM_SCORES = false>
__device__ __forceinline__ void decode_block(const DecArgs& a, int slot, int grp) {
  const int split = SPARSE ? slot / a.nsub : slot;       // index range (sparse) / list slice (window)
  const int sub = SPARSE ? slot % a.nsub : 0;
  constexpr int LPT = D / 8;            // lanes per cached row
  constexpr int TPW = 64 / LPT;         // rows per wave step
  constexpr int NLG = (kDecThreads / 64) * TPW;
  constexpr int RANGE = kDecRange;      // sparse path (the window path slices a.wrange positions)
  constexpr int NW = kDecThreads / 64;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lg = wave * TPW + lane / LPT;
  const int li = lane % LPT;
  const int b = grp / a.map.n, rr = grp % a.map.n, g = a.map.kv[rr];
  // the live context: its length, and (window path) its sink + window list.  Slices and
  // ranges past it write empty partials, which add exact zeros in the merge.
  const int n_ctx = live_ctx(a.live, a.n_ctx);
  int s_end = a.s_end, w_start = a.w_start, list_len = a.list_len, ring_off = a.ring_off;
  if (!SPARSE && a.live) {
    s_end = min(a.n_sinks, n_ctx);
    w_start = max(n_ctx - a.window, s_end);
    list_len = s_end + (n_ctx - w_start);
    ring_off = (a.ring_w > 0 && w_start >= a.ring_s) ? (w_start - a.ring_s) % a.ring_w : 0;
  }
  const int nsplit_live = SPARSE ? (n_ctx + RANGE - 1) / RANGE : a.nsplit;
  const int64_t head_off = (int64_t(b) * a.cache_heads + (a.by_rank ? rr : g)) * a.cache_rows * D + li * 8;
  const uint16_t* kb = a.k + head_off;
  const uint16_t* vb = a.v + head_off;

  __shared__ uint16_t s_list[SPARSE ? RANGE : 1];
  __shared__ uint8_t s_lmask[SPARSE ? RANGE : 1];
  __shared__ uint32_t s_hm[(SPARSE && !FROM_SCORES) ? G * RANGE / 4 : 1];
  __shared__ int s_wcnt[NW];
  __shared__ float s_wm[NW][G], s_wl[NW][G];
  __shared__ float s_wacc[NW][G][D];
  // decode step (members from the membership words): per (head, item, wave) above / tied
  // counts, then their exclusive prefixes; ties taken per head; list bounds; member flags
  constexpr int NE = (RANGE / kDecThreads) * NW;
  constexpr int GF = (SPARSE && FROM_SCORES) ? G : 1;
  static_assert(!(SPARSE && FROM_SCORES) || (G * NE <= kDecThreads && 64 % NE == 0), "one lane per entry");
  __shared__ __align__(16) uint32_t s_ca[GF * NE];
  __shared__ __align__(16) uint32_t s_ce[GF * NE];
  __shared__ uint32_t s_take[GF];
  __shared__ int s_lo[GF], s_hi[GF];
  __shared__ uint16_t s_sel[GF][(SPARSE && FROM_SCORES) ? RANGE : 1];   // the range's list part per head
  __shared__ __align__(16) uint32_t s_uc[(SPARSE && FROM_SCORES) ? NE : 4];   // union count per (item, wave)

  uint32_t qw[G][4];
#pragma unroll
  for (int t = 0; t < G; ++t) {
    const uint4 qv = *reinterpret_cast<const uint4*>(a.q + (int64_t(b) * a.Hq + g * G + t) * D + li * 8);
    qw[t][0] = qv.x;
    qw[t][1] = qv.y;
    qw[t][2] = qv.z;
    qw[t][3] = qv.w;
  }

  int U, j0 = 0, p0 = 0, e0 = 0;
  if constexpr (SPARSE) {
    j0 = split * RANGE;
    // A head's selected indices are distinct, so at most RANGE of them fall in the
    // range: SP per thread.  All loads are issued before any membership byte is set.
    constexpr int SP = RANGE / kDecThreads;
    // range index entries: loaded unconditionally (every launched range has both), so that
    // they are one batch of loads rather than a chain of guarded ones
    // (a zero held in a vector register makes them vector loads, whose wait is separate from
    // that of the scalar loads of the kernel arguments and membership words)
    int vz = 0;
    asm volatile("" : "+v"(vz));
    int lo[G], hi[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
      const int64_t so = int64_t(grp * G + t) * (a.nsplit + 1) + split + vz;
      lo[t] = a.starts[so];
      hi[t] = a.starts[so + 1];
    }
    // members from the scores: the range's scores (position u * kDecThreads + tid) and the
    // threshold keys of every head
    float sc[FROM_SCORES ? G : 1][SP];
    uint32_t thr[FROM_SCORES ? G : 1];
    if constexpr (FROM_SCORES) {
      if (!a.all_tokens) {
#pragma unroll
        for (int t = 0; t < G; ++t) {
          const float* sr = a.scores + int64_t(grp * G + t) * a.n_cap;
#pragma unroll
          for (int u = 0; u < SP; ++u) {
            const int j = j0 + u * kDecThreads + tid;
            sc[t][u] = sr[j < n_ctx ? j : n_ctx - 1];             // unconditional, clamped
          }
          thr[t] = a.thr[grp * G + t];
        }
      }
    }
#pragma unroll
    for (int t = 0; t < G; ++t) {
      // clamped: the range index may come from the caller; a range past the live context is empty
      hi[t] = split < nsplit_live ? min(max(hi[t], 0), n_ctx) : 0;
      lo[t] = split < nsplit_live ? min(max(lo[t], 0), hi[t]) : 0;
    }
    if constexpr (FROM_SCORES) {
      // Position u * kDecThreads + tid of the range; wave w holds positions u * kDecThreads +
      // 64 w + lane of item u, so (item, wave, lane) order is position order.  Per head and
      // item, this wave's tokens as words (ballots): above t (A) and tied with t (T).
      const bool live_range = split < nsplit_live;
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      uint64_t wA[G][SP], wT[G][SP];
#pragma unroll
      for (int t = 0; t < G; ++t) {
#pragma unroll
        for (int u = 0; u < SP; ++u) {
          const bool in = live_range && j0 + u * kDecThreads + tid < n_ctx;
          bool above = in, tied = false;                        // every token (top_p >= 1)
          if (!a.all_tokens) {
            const uint32_t key = score_key(sc[t][u]);
            above = in && key > thr[t];
            tied = in && key == thr[t];
          }
          wA[t][u] = __ballot(above);
          wT[t][u] = __ballot(tied);
          if (lane == 0) {
            s_ca[t * NE + u * NW + wave] = __popcll(wA[t][u]);
            s_ce[t * NE + u * NW + wave] = __popcll(wT[t][u]);
          }
        }
      }
      if (tid == 0) {
#pragma unroll
        for (int t = 0; t < G; ++t) {
          s_lo[t] = lo[t];
          s_hi[t] = hi[t];
        }
      }
      __syncthreads();
      if (tid < G) {                     // thread h: exclusive prefixes of head h's NE entries
        uint4* pa = reinterpret_cast<uint4*>(s_ca + tid * NE);
        uint4* pe = reinterpret_cast<uint4*>(s_ce + tid * NE);
        uint4 va[NE / 4], ve[NE / 4];
#pragma unroll
        for (int k = 0; k < NE / 4; ++k) {
          va[k] = pa[k];
          ve[k] = pe[k];
        }
        uint32_t xa = 0, xe = 0;
#pragma unroll
        for (int k = 0; k < NE / 4; ++k) {
          const uint32_t a0 = va[k].x, a1 = va[k].y, a2 = va[k].z, a3 = va[k].w;
          const uint32_t e0 = ve[k].x, e1 = ve[k].y, e2 = ve[k].z, e3 = ve[k].w;
          pa[k] = make_uint4(xa, xa + a0, xa + a0 + a1, xa + a0 + a1 + a2);
          pe[k] = make_uint4(xe, xe + e0, xe + e0 + e1, xe + e0 + e1 + e2);
          xa += a0 + a1 + a2 + a3;
          xe += e0 + e1 + e2 + e3;
        }
        // ties this range takes: its list length minus its tokens above t (every tie, for
        // the all-tokens lists, which hold no ties)
        int lo_h = lo[0], hi_h = hi[0];
#pragma unroll
        for (int t = 1; t < G; ++t)
          if (tid == t) {
            lo_h = lo[t];
            hi_h = hi[t];
          }
        const int take_i = hi_h - lo_h - int(xa);
        s_take[tid] = take_i < 0 ? 0u : (uint32_t(take_i) > xe ? xe : uint32_t(take_i));
      }
      __syncthreads();
      // members: A, and the first take ties of the range; each member's place in its head's
      // list part (kept in LDS, written out after the attention); the union over the heads,
      // with each position's head mask, and its count per (item, wave)
      uint32_t pa[G][SP], pe[G][SP], take[G];
#pragma unroll
      for (int t = 0; t < G; ++t) {
        take[t] = s_take[t];
#pragma unroll
        for (int u = 0; u < SP; ++u) {
          pa[t][u] = s_ca[t * NE + u * NW + wave];
          pe[t][u] = s_ce[t * NE + u * NW + wave];
        }
      }
      uint64_t wU[SP];
      uint32_t mk[SP];
#pragma unroll
      for (int u = 0; u < SP; ++u) {
        wU[u] = 0;
        mk[u] = 0;
#pragma unroll
        for (int t = 0; t < G; ++t) {
          const uint32_t a_before = pa[t][u] + __popcll(wA[t][u] & lt);
          const uint32_t e_before = pe[t][u] + __popcll(wT[t][u] & lt);
          const bool mem = ((wA[t][u] >> lane) & 1ull) || (((wT[t][u] >> lane) & 1ull) && e_before < take[t]);
          if (mem) s_sel[t][a_before + (e_before < take[t] ? e_before : take[t])] = uint16_t(u * kDecThreads + tid);
          const uint64_t wm = wT[t][u] ? __ballot(mem) : wA[t][u];
          wU[u] |= wm;
          mk[u] |= uint32_t(mem) << t;
        }
        if (lane == 0) s_uc[u * NW + wave] = __popcll(wU[u]);
      }
      __syncthreads();
      // list offsets: counts of the (item, wave) pairs before, in position order
      uint32_t uc[SP * NW];
#pragma unroll
      for (int k = 0; k < SP * NW / 4; ++k) {
        const uint4 v = reinterpret_cast<const uint4*>(s_uc)[k];
        uc[4 * k] = v.x;
        uc[4 * k + 1] = v.y;
        uc[4 * k + 2] = v.z;
        uc[4 * k + 3] = v.w;
      }
      uint32_t total = 0;
#pragma unroll
      for (int u = 0; u < SP; ++u) {
        uint32_t off = total;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          if (w < wave) off += uc[u * NW + w];
          total += uc[u * NW + w];
        }
        if (mk[u]) {
          const uint32_t at = off + __popcll(wU[u] & lt);
          s_list[at] = uint16_t(u * kDecThreads + tid);
          s_lmask[at] = uint8_t(mk[u]);
        }
      }
      U = int(total);
    } else {
      for (int i = tid; i < G * RANGE / 4; i += kDecThreads) s_hm[i] = 0;
      __syncthreads();
      uint8_t* hm = reinterpret_cast<uint8_t*>(s_hm);
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
          // an index outside [0, n_ctx) (a malformed list from the caller) is dropped, so no
          // cache row at or past n_ctx is ever read
          pos[t][u] = (k < hi[t] && v >= 0 && v < n_ctx) ? v - j0 : -1;
        }
      }
#pragma unroll
      for (int t = 0; t < G; ++t)
#pragma unroll
        for (int u = 0; u < SP; ++u)
          if (pos[t][u] >= 0 && pos[t][u] < RANGE) hm[t * RANGE + pos[t][u]] = 1;
      __syncthreads();
      // ordered union of the G membership arrays: thread tid owns positions tid*PER .. tid*PER+PER-1
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
    }
    __syncthreads();
    if (a.nsub > 1) {          // this block's slice of the union list: positions [e0, e0 + U)
      constexpr int STEP0 = kDecUnroll * NLG;
      const int chunk = ((U + a.nsub - 1) / a.nsub + STEP0 - 1) / STEP0 * STEP0;
      e0 = min(U, sub * chunk);
      U = min(U, e0 + chunk) - e0;
    }
  } else {
    p0 = split * a.wrange;
    U = min(a.wrange, list_len - p0);
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
      mask = s_lmask[e0 + e];
      return int64_t(j0) + s_list[e0 + e];
    } else {
      mask = (1u << G) - 1u;
      const int p = p0 + e;
      if (p < s_end) return int64_t(p);
      if (a.ring_w > 0) {                      // window token w_start + (p - s_end) in the ring
        int t = ring_off + (p - s_end);        // < 2 * ring_w: the window holds at most ring_w tokens
        if (t >= a.ring_w) t -= a.ring_w;
        return int64_t(a.ring_s) + t;
      }
      return int64_t(w_start) + (p - s_end);
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
    float* pr = a.part + ((int64_t(grp) * G + t) * a.nsplit * a.nsub + slot) * (D + 4);
    pr[d] = A;
    if (d == 0) {
      pr[D] = M;
      pr[D + 1] = Lsum;
    }
  }
  if constexpr (SPARSE && FROM_SCORES) {
    // this range's part of the selected lists, written last (a barrier waits for every
    // store in flight, and none follows here), from its copy in LDS
    if (a.sel_out && sub == 0 && !a.all_tokens) {
#pragma unroll
      for (int t = 0; t < G; ++t) {
        const int lo_t = s_lo[t], n_t = s_hi[t] - s_lo[t];      // its members: the list part [lo, hi)
        int32_t* out = a.sel_out + int64_t(grp * G + t) * a.n_cap + lo_t;
        for (int i = tid; i < n_t; i += kDecThreads) out[i] = j0 + s_sel[t][i];
      }
    }
  }
}

// Combine the per-slice partials of one (batch, head) row into the bf16 output.
// 256 threads per row: D/4 lanes read one split's accumulator as float4s, 256/(D/4)
// split groups take every SG-th split (independent loads, unrolled), then the groups
// are combined in LDS.
struct MergeArgs {
  const float* part;           // [rows][nsplit][D + 4]
  int nsplit;
  int G, Hq;
  HeadMap map;
  uint16_t* out;               // [B][Hq][D]
};

template <int D>
__device__ __forceinline__ void merge_row(const MergeArgs& ma, int row) {
  constexpr int PS = D + 4;                 // partial row stride (floats)
  constexpr int Q = D / 4;                  // float4 columns
  constexpr int SG = 256 / Q;               // split groups
  const float* __restrict__ part = ma.part;
  const int nsplit = ma.nsplit, G = ma.G, Hq = ma.Hq;
  const HeadMap& map = ma.map;
  uint16_t* __restrict__ out = ma.out;
  const int tid = threadIdx.x;
  const int q = tid % Q, sg = tid / Q;
  const int grp = row / G, t = row % G;
  const int b = grp / map.n, rr = grp % map.n;
  const int h = map.kv[rr] * G + t;
  const float* pr = part + int64_t(row) * nsplit * PS;
  __shared__ float s_red[4];
  __shared__ float4 s_a[SG][Q];
  __shared__ float s_l[SG];
  // reference max over the splits
  float M = -INFINITY;
  for (int s = tid; s < nsplit; s += 256) M = fmaxf(M, pr[int64_t(s) * PS + D]);
  M = wave_max(M);
  if ((tid & 63) == 0) s_red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float4 A = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float Lsum = 0.0f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s = sg; s < nsplit; s += SG) {
      const float* ps = pr + int64_t(s) * PS;
      const float ms = ps[D];
      const float f = (ms == -INFINITY) ? 0.0f : fast_exp2(ms - M);
      const float4 o = *reinterpret_cast<const float4*>(ps + 4 * q);
      A.x = fmaf(o.x, f, A.x);
      A.y = fmaf(o.y, f, A.y);
      A.z = fmaf(o.z, f, A.z);
      A.w = fmaf(o.w, f, A.w);
      Lsum = fmaf(ps[D + 1], f, Lsum);
    }
  }
  s_a[sg][q] = A;
  if (q == 0) s_l[sg] = Lsum;
  __syncthreads();
  if (tid < D) {
    const int qq = tid >> 2, e = tid & 3;
    float a = 0.0f, l = 0.0f;
#pragma unroll
    for (int i = 0; i < SG; ++i) {
      const float4 v = s_a[i][qq];
      a += e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
      l += s_l[i];
    }
    out[(int64_t(b) * Hq + h) * D + tid] = f32_to_bf16(l > 0.0f ? a / l : 0.0f);
  }
}

// First level of a two-level merge: splits [chunk*kMergeFan, +kMergeFan) of one row
// combined into one partial of the same form (accumulator relative to its own max, max,
// sum), at part2[row][chunk].  256 threads: D/4 float4 lanes x 256/(D/4) split groups.
template <int D>
__device__ __forceinline__ void merge_pre_chunk(const MergeArgs& ma, float* __restrict__ part2, int nchunks,
                                                int row, int chunk) {
  constexpr int PS = D + 4;
  constexpr int Q = D / 4;
  constexpr int SG = 256 / Q;
  const int tid = threadIdx.x;
  const int q = tid % Q, sg = tid / Q;
  const int s0 = chunk * kMergeFan, s1 = min(ma.nsplit, s0 + kMergeFan);
  const float* pr = ma.part + int64_t(row) * ma.nsplit * PS;
  __shared__ float s_red[4];
  __shared__ float4 s_a[SG][Q];
  __shared__ float s_l[SG];
  float M = -INFINITY;
  if (s0 + tid < s1) M = pr[int64_t(s0 + tid) * PS + D];
  M = wave_max(M);
  if ((tid & 63) == 0) s_red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float4 A = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float Lsum = 0.0f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s = s0 + sg; s < s1; s += SG) {
      const float* ps = pr + int64_t(s) * PS;
      const float ms = ps[D];
      const float f = (ms == -INFINITY) ? 0.0f : fast_exp2(ms - M);
      const float4 o = *reinterpret_cast<const float4*>(ps + 4 * q);
      A.x = fmaf(o.x, f, A.x);
      A.y = fmaf(o.y, f, A.y);
      A.z = fmaf(o.z, f, A.z);
      A.w = fmaf(o.w, f, A.w);
      Lsum = fmaf(ps[D + 1], f, Lsum);
    }
  }
  s_a[sg][q] = A;
  if (q == 0) s_l[sg] = Lsum;
  __syncthreads();
  float* po = part2 + (int64_t(row) * nchunks + chunk) * PS;
  if (tid < D) {
    const int qq = tid >> 2, e = tid & 3;
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < SG; ++i) {
      const float4 v = s_a[i][qq];
      a += e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
    }
    po[tid] = a;
  }
  if (tid == 0) {
    float l = 0.0f;
#pragma unroll
    for (int i = 0; i < SG; ++i) l += s_l[i];
    po[D] = M;
    po[D + 1] = l;
  }
}

// Cache addressing of the two decode kinds for the descriptor's layout (host side).
inline void set_sparse_cache(DecArgs& a, const Layer& L) {
  const bool compact = L.kv_layout == RTP_KV_COMPACT;
  a.cache_heads = compact ? L.n_ret : L.Hkv;
  a.by_rank = compact;
  a.cache_rows = L.n_cap;
  a.ring_s = a.ring_w = a.ring_off = 0;
  a.nsub = dec_sub(a.nsplit, L.B * L.n_ret);
}
inline void set_window_cache(DecArgs& a, const Layer& L) {      // after s_end / w_start are set
  a.nsub = 1;
  if (L.kv_layout == RTP_KV_COMPACT) {
    a.cache_heads = L.n_loc;
    a.by_rank = 1;
    a.cache_rows = int64_t(L.n_sinks) + L.window;
    a.ring_s = L.n_sinks;
    a.ring_w = L.window;
    a.ring_off = a.w_start >= L.n_sinks ? int((int64_t(a.w_start) - L.n_sinks) % L.window) : 0;
  } else {
    a.cache_heads = L.Hkv;
    a.by_rank = 0;
    a.cache_rows = L.n_cap;
    a.ring_s = a.ring_w = a.ring_off = 0;
  }
}

}  // namespace
