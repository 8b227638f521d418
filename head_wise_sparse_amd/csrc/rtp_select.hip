// rtp_topp_select: query-adaptive top-p token sets (abstract, observation (3):
// the useful token budget depends on the query, so a dynamic top-p rule replaces a
// fixed top-k; research-map summary, "Approach": query-adaptive top-p threshold).
//
// For one score row, rank tokens by score (higher first, equal scores by lower
// index) and keep the shortest prefix of the ranking whose softmax mass reaches p.
// That prefix is exactly {key(s_j) > t} plus the first r tokens (by index) with
// key(s_j) == t, where key() is the order-preserving uint32 image of the fp32 score,
// t the threshold key and r a tie count.  The search is O(N) and takes four launches:
//
//   hist<0>   histogram of key bits [31:21] over the whole row.  Each bin carries the
//             token count and the softmax mass exp(s - max) in 2^-42 fixed point (u64:
//             exact sums, independent of order, bit-reproducible).  Bins are built in
//             LDS per block and added to the row's histogram with global atomics, with a
//             64-bin coarse summary (32 fine bins each) beside it.
//   hist<1,2> the same on key bits [20:10] and [9:0], only for tokens whose higher
//             bits equal the digits resolved so far.  Before that, one wave of every
//             block resolves the previous level's digit from the coarse summary, then
//             from the 32 fine bins under the chosen coarse bin (two small reads): the
//             digit is where the mass accumulated from the top first reaches what is
//             still needed.  The kernel boundary is the only synchronisation.
//             hist<2> also leaves one record per tile: how many of its tokens lie above
//             the 22-bit prefix (certainly selected) and, for up to kRecPairs distinct
//             low 10-bit digits among the tokens that share it (candidates), the digit
//             and its count.
//   compact   resolves the last digit (t is now the full key), the tie count r in
//             closed form (tied tokens carry equal weight), and writes the selected
//             indices in increasing order.  A tile's output offset comes from the
//             records of the earlier tiles (written by the previous launch: no waiting
//             on other blocks): tokens above the prefix, plus candidates above t, plus
//             at most r ties.  Candidates share 22 key bits with t, so a tile holds few
//             distinct ones (exact ties collapse into one pair); only for a tile with
//             more distinct candidates than its record keeps does the block count them
//             again from that tile's scores.
//             It also writes the range index of every list when asked for.
// The workspace is all zero when a call starts and when it ends: each launch clears
// what earlier launches left and nobody reads any more (hist<2> the level-0
// histogram, compact the level-1 histogram), and the last compaction block of a row
// to finish clears the rest of that row (level-2 histogram, tile records, row state
// and counters).
#include <cmath>

#include "rtp_internal.hpp"
#include "score_dev.hpp"

using namespace rtp;
using namespace rtp_dev;

namespace {

constexpr int kCoarse = 64;          // coarse bins of levels 0/1 (32 at level 2)
constexpr int kFinePer = 32;         // fine bins under one coarse bin
constexpr int kRecPairs = 3;         // (digit, count) pairs a tile record holds (one per 32-bit word)
constexpr int kMaxHeavy = 256;       // heavy earlier tiles a compaction block recounts one by one

__device__ __forceinline__ uint64_t ld_rlx(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_rlx(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T wave_suffix_incl(T v, int lane) {      // sum over lanes >= lane
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_down(v, o, 64);
    if (lane + o < 64) v += y;
  }
  return v;
}

__device__ __forceinline__ int level_bins(int level) { return level == 2 ? 1024 : 2048; }

struct Resolved {            // result of resolving one level's digit
  uint32_t prefix;           // digits resolved so far
  uint64_t above;            // mass strictly above the prefix
  uint32_t cnt_above;        // tokens strictly above the prefix
  uint64_t target;           // mass the set must reach
  uint32_t tied;             // count in the resolved bin (meaningful at level 2)
};

// Resolve the digit of `level` from the finished histogram of that level.  Called by
// one full wave; every lane returns the same result.  `in` carries the state after
// the previous level (ignored for level 0, where the target is ceil(p * Z), or k when
// the bins are weighed by their counts for the static top-k rule).
__device__ Resolved resolve_level(const SelRows& R, int row, int level, const Resolved& in, float top_p,
                                  bool by_count, int64_t k_target, int lane) {
  const int nc = level == 2 ? 32 : kCoarse;
  const uint64_t* cm = R.cmass + (int64_t(row) * 3 + level) * kCoarse;
  const uint32_t* cc = R.ccnt + (int64_t(row) * 3 + level) * kCoarse;
  const uint32_t c_l = lane < nc ? ld_rlx(cc + lane) : 0u;
  const uint64_t m_l = by_count ? uint64_t(c_l) : (lane < nc ? ld_rlx(cm + lane) : 0ull);
  Resolved o = in;
  if (level == 0) {
    const uint64_t z = wave_sum<uint64_t>(m_l);
    uint64_t t;
    if (by_count) {
      t = uint64_t(k_target);
    } else {
      const double tgt = ceil(double(top_p) * double(z));
      t = tgt < 1.0 ? 1ull : (uint64_t)tgt;
    }
    o.target = t > z ? z : t;
    o.above = 0;
    o.cnt_above = 0;
    o.prefix = 0;
  }
  uint64_t need = o.target - o.above;
  // coarse: S(c) = mass of coarse bins >= c; the owner satisfies S(c+1) < need <= S(c)
  const uint64_t S = wave_suffix_incl<uint64_t>(m_l, lane);
  const uint32_t SC = wave_suffix_incl<uint32_t>(c_l, lane);
  const uint64_t own = __ballot(lane < nc && S >= need && S - m_l < need);
  const int cs = own ? __ffsll((unsigned long long)own) - 1 : 0;
  const uint64_t above_c = __shfl(S - m_l, cs, 64);
  const uint32_t cnt_above_c = __shfl(SC - c_l, cs, 64);
  need -= above_c;
  // fine bins under the chosen coarse bin
  const uint64_t* fm = R.mass + (int64_t(row) * 3 + level) * kBins + cs * kFinePer;
  const uint32_t* fc = R.cnt + (int64_t(row) * 3 + level) * kBins + cs * kFinePer;
  const uint32_t fc_l = lane < kFinePer ? ld_rlx(fc + lane) : 0u;
  const uint64_t fm_l = by_count ? uint64_t(fc_l) : (lane < kFinePer ? ld_rlx(fm + lane) : 0ull);
  const uint64_t FS = wave_suffix_incl<uint64_t>(fm_l, lane);
  const uint32_t FSC = wave_suffix_incl<uint32_t>(fc_l, lane);
  const uint64_t fown = __ballot(lane < kFinePer && FS >= need && FS - fm_l < need);
  const int fs = fown ? __ffsll((unsigned long long)fown) - 1 : 0;
  const uint32_t digit = uint32_t(cs * kFinePer + fs);
  o.above += above_c + __shfl(FS - fm_l, fs, 64);
  o.cnt_above += cnt_above_c + __shfl(FSC - fc_l, fs, 64);
  o.tied = __shfl(fc_l, fs, 64);
  o.prefix = level == 0 ? digit : ((o.prefix << (level == 1 ? 11 : 10)) | digit);
  return o;
}

// Level 2 (1024 bins, histogram complete since the previous launch) in one round trip:
// lane l loads bins 16l .. 16l+15 and the owner bin is found by the same rule as above
// (mass of the bins above < need <= that plus the bin's own mass), from lane suffix sums
// and a scan inside the owning lane.
__device__ Resolved resolve_level2_direct(const SelRows& R, int row, const Resolved& in, bool by_count, int lane) {
  constexpr int PER = 1024 / 64;
  const uint32_t* fc = R.cnt + (int64_t(row) * 3 + 2) * kBins + lane * PER;
  const uint64_t* fm = R.mass + (int64_t(row) * 3 + 2) * kBins + lane * PER;
  uint32_t c[PER];
  uint64_t m[PER];
#pragma unroll
  for (int k = 0; k < PER / 4; ++k) {
    const uint4 v = reinterpret_cast<const uint4*>(fc)[k];
    c[4 * k] = v.x;
    c[4 * k + 1] = v.y;
    c[4 * k + 2] = v.z;
    c[4 * k + 3] = v.w;
  }
  if (!by_count) {
#pragma unroll
    for (int k = 0; k < PER / 2; ++k) {
      const uint4 v = reinterpret_cast<const uint4*>(fm)[k];
      m[2 * k] = uint64_t(v.x) | (uint64_t(v.y) << 32);
      m[2 * k + 1] = uint64_t(v.z) | (uint64_t(v.w) << 32);
    }
  } else {
#pragma unroll
    for (int k = 0; k < PER; ++k) m[k] = c[k];
  }
  uint64_t lm = 0;
  uint32_t lc = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    lm += m[k];
    lc += c[k];
  }
  Resolved o = in;
  const uint64_t need = o.target - o.above;
  const uint64_t S = wave_suffix_incl<uint64_t>(lm, lane);
  const uint32_t SC = wave_suffix_incl<uint32_t>(lc, lane);
  const uint64_t own = __ballot(S >= need && S - lm < need);
  const int ol = own ? __ffsll((unsigned long long)own) - 1 : 0;
  // inside the owning lane: bins from the top down
  uint64_t acc = S - lm;
  uint32_t cacc = SC - lc;
  int fb = 0;
  uint32_t tied = c[0];
  uint64_t above_f = acc;
  uint32_t cnt_above_f = cacc;
  bool found = false;
#pragma unroll
  for (int k = PER - 1; k >= 0; --k) {
    if (!found && acc + m[k] >= need) {
      found = true;
      fb = k;
      tied = c[k];
      above_f = acc;
      cnt_above_f = cacc;
    }
    acc += m[k];
    cacc += c[k];
  }
  const uint32_t digit = uint32_t(ol * PER + __shfl(fb, ol, 64));
  o.above += __shfl(above_f, ol, 64);
  o.cnt_above += __shfl(cnt_above_f, ol, 64);
  o.tied = __shfl(tied, ol, 64);
  o.prefix = (o.prefix << 10) | digit;
  return o;
}

// Clear one level's histogram of a row (plain stores: the next launch sees them).
// Block `blk` of `nblk` clears its share.
__device__ __forceinline__ void clear_level(const SelRows& R, int row, int level, int blk, int nblk) {
  uint64_t* gm = R.mass + (int64_t(row) * 3 + level) * kBins;
  uint32_t* gc = R.cnt + (int64_t(row) * 3 + level) * kBins;
  for (int i = blk * kSelThreads + int(threadIdx.x); i < kBins; i += nblk * kSelThreads) {
    gm[i] = 0;
    gc[i] = 0;
  }
  if (blk == nblk - 1 && threadIdx.x < kCoarse) {
    R.cmass[(int64_t(row) * 3 + level) * kCoarse + threadIdx.x] = 0;
    R.ccnt[(int64_t(row) * 3 + level) * kCoarse + threadIdx.x] = 0;
  }
}

// Row max (and, by the first block, the row statistics) from the scoring's per-block
// (max, sum of exp) partials.
__device__ float row_max_from_partials(const SelArgs& a, int row, int blk, int tid, float* s_red) {
  const float2* p = a.score_part + int64_t(row) * a.score_nblk;
  float m = -INFINITY;
  for (int i = tid; i < a.score_nblk; i += kSelThreads) m = fmaxf(m, p[i].x);
  m = wave_max(m);
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  // the row statistics, by the same one-wave reduction as rtp_indexer_score's
  if (blk == 0 && a.row_max_out && tid < 64)
    score_finalize_row(a.score_part, a.score_nblk, a.row_max_out, a.row_sum_out, row);
  return m;
}

template <int LEVEL, int ITEMS>
__global__ __launch_bounds__(kSelThreads) void k_sel_hist(SelArgs a) {
  constexpr int TILE = kSelThreads * ITEMS;
  constexpr int NB = LEVEL == 2 ? 1024 : 2048;
  constexpr int SHIFT = LEVEL == 0 ? 21 : (LEVEL == 1 ? 10 : 0);
  constexpr int PSHIFT = LEVEL == 1 ? 21 : 10;                     // prefix bits start (levels 1, 2)
  const int tid = threadIdx.x, lane = tid & 63;
  const int blk = blockIdx.x, row = blockIdx.y;
  __shared__ uint64_t h_m[NB];
  __shared__ uint32_t h_c[NB];
  __shared__ uint32_t s_prefix;
  __shared__ float s_red[kSelThreads / 64];
  __shared__ uint32_t s_na[kSelThreads / 64], s_np, s_pair[kRecPairs];   // level 2: tile record

  // scores of the tile: unconditional loads (index clamped), validity kept aside
  const float* sp = a.scores + int64_t(row) * a.n_cap;
  const int64_t base = int64_t(blk) * TILE;
  float sv[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int64_t j = base + it * kSelThreads + tid;
    sv[it] = sp[j < a.n_ctx ? j : a.n_ctx - 1];
  }
  for (int i = tid; i < NB; i += kSelThreads) {
    h_m[i] = 0;
    h_c[i] = 0;
  }
  if (LEVEL == 2 && tid == 0) s_np = 0;
  float m = 0.0f;                                   // unused by the static top-k rule
  if constexpr (LEVEL == 0) {
    if (!a.by_count) m = a.score_part ? row_max_from_partials(a, row, blk, tid, s_red) : a.row_max[row];
    if (blk == 0 && tid == 0) a.R.state[row].ref_max = m;
  } else {
    m = a.R.state[row].ref_max;                      // written by the level-0 launch
  }
  if constexpr (LEVEL == 2) clear_level(a.R, row, 0, blk, a.nblk);   // read last by hist<1>
  if (LEVEL > 0 && tid < 64) {
    Resolved in{};
    if (LEVEL == 2) {
      const SelLevelState& ls = a.R.state[row].lvl[0];
      in.prefix = ls.prefix;
      in.above = ls.above;
      in.cnt_above = ls.cnt_above;
      in.target = ls.target;
    }
    const Resolved o = resolve_level(a.R, row, LEVEL - 1, in, a.top_p, a.by_count, a.k_target, lane);
    if (lane == 0) {
      s_prefix = o.prefix;
      if (blk == 0) {          // one block publishes; this launch's blocks read only lvl[LEVEL-2]
        SelLevelState& ls = a.R.state[row].lvl[LEVEL - 1];
        ls.prefix = o.prefix;
        ls.above = o.above;
        ls.cnt_above = o.cnt_above;
        ls.target = o.target;
      }
    }
  }
  __syncthreads();
  const uint32_t prefix = LEVEL > 0 ? s_prefix : 0u;
  uint32_t n_above = 0;                             // level 2: tokens above the 22-bit prefix
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int64_t j = base + it * kSelThreads + tid;
    const uint32_t key = score_key(sv[it]);
    const bool match = (j < a.n_ctx) && (LEVEL == 0 || (key >> PSHIFT) == prefix);
    if (match) {
      const uint32_t d = (key >> SHIFT) & uint32_t(NB - 1);
      if (!a.by_count) atomicAdd(reinterpret_cast<unsigned long long*>(&h_m[d]), (unsigned long long)fixed_weight(sv[it], m));
      atomicAdd(&h_c[d], 1u);
    }
    if constexpr (LEVEL == 2) n_above += uint32_t((j < a.n_ctx) && (key >> PSHIFT) > prefix);
  }
  if constexpr (LEVEL == 2) {
    n_above = wave_sum(n_above);
    if (lane == 0) s_na[tid / 64] = n_above;
  }
  __syncthreads();

  uint64_t* gm = a.R.mass + (int64_t(row) * 3 + LEVEL) * kBins;
  uint32_t* gc = a.R.cnt + (int64_t(row) * 3 + LEVEL) * kBins;
  for (int i = tid; i < NB; i += kSelThreads) {
    if (h_c[i]) {
      if (!a.by_count) atomicAdd(reinterpret_cast<unsigned long long*>(gm + i), (unsigned long long)h_m[i]);
      atomicAdd(gc + i, h_c[i]);
      if constexpr (LEVEL == 2) {              // this tile's distinct candidate digits
        const uint32_t k = atomicAdd(&s_np, 1u);
        if (k < uint32_t(kRecPairs)) s_pair[k] = uint32_t(i) | (h_c[i] << 10);
      }
    }
  }
  if constexpr (LEVEL == 2) {
    __syncthreads();
    if (tid == 0) {
      uint32_t na = 0;
#pragma unroll
      for (int w = 0; w < kSelThreads / 64; ++w) na += s_na[w];
      const uint32_t np = s_np;
      uint32_t pw[kRecPairs];
#pragma unroll
      for (int k = 0; k < kRecPairs; ++k) pw[k] = uint32_t(k) < np ? s_pair[k] : 0u;
      a.R.tilerec[int64_t(row) * a.rec_stride + blk] = make_uint4(na | (np << 16), pw[0], pw[1], pw[2]);
    }
  }
  // coarse summary: thread c < NB/32 sums its 32 fine bins, starting at a different
  // one per thread so that the lanes of a wave read different LDS banks
  if (tid < NB / kFinePer) {
    uint64_t sm = 0;
    uint32_t sc = 0;
#pragma unroll 8
    for (int i = 0; i < kFinePer; ++i) {
      const int f = tid * kFinePer + ((i + tid) & (kFinePer - 1));
      sm += h_m[f];
      sc += h_c[f];
    }
    if (sc) {
      if (!a.by_count)
        atomicAdd(reinterpret_cast<unsigned long long*>(a.R.cmass + (int64_t(row) * 3 + LEVEL) * kCoarse + tid),
                  (unsigned long long)sm);
      atomicAdd(a.R.ccnt + (int64_t(row) * 3 + LEVEL) * kCoarse + tid, sc);
    }
  }
}

// Resolve the last digit, then write {key > t} U {first r with key == t} in order.
template <int ITEMS>
__global__ __launch_bounds__(kSelThreads) void k_sel_compact(SelArgs a) {
  constexpr int TILE = kSelThreads * ITEMS;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int row = blockIdx.y, tile = blockIdx.x;
  constexpr int NW = kSelThreads / 64;
  constexpr int PL = ITEMS * NW / 64;                 // (item, wave) counts per lane of the scanning wave
  static_assert(ITEMS * NW % 64 == 0 && ITEMS <= 32, "one wave scans the per-(item, wave) counts");
  __shared__ uint32_t s_t, s_r;
  __shared__ uint32_t s_wa[ITEMS * NW], s_we[ITEMS * NW];   // counts, then exclusive prefixes
  __shared__ uint32_t s_pa, s_pe, s_heavy, s_last;
  __shared__ uint32_t s_ra[NW], s_re[NW];
  __shared__ uint32_t s_heavy_list[kMaxHeavy];
  uint32_t* ctr = a.R.ctr + 2 * int64_t(row);
  const uint4* rec = a.R.tilerec + int64_t(row) * a.rec_stride;
  const float* sp = a.scores + int64_t(row) * a.n_cap;
  const int64_t base = int64_t(tile) * TILE;
  float sv[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int64_t j = base + it * kSelThreads + tid;
    sv[it] = sp[j < a.n_ctx ? j : a.n_ctx - 1];
  }
  uint4 rec0 = make_uint4(0u, 0u, 0u, 0u);           // records of the first 64 earlier tiles
  if (wave == 1 && lane < tile) rec0 = rec[lane];
  if (wave == 0) {
    const SelLevelState& ls = a.R.state[row].lvl[1];
    Resolved in{};
    in.prefix = ls.prefix;
    in.above = ls.above;
    in.cnt_above = ls.cnt_above;
    in.target = ls.target;
    const Resolved o = resolve_level2_direct(a.R, row, in, a.by_count, lane);
    if (lane == 0) {
      // tied tokens share one weight (1 for top-k): take just enough of them to reach the target
      s_t = o.prefix;
      const uint64_t w = a.by_count ? 1ull : fixed_weight(key_score(o.prefix), a.R.state[row].ref_max);
      const uint64_t rem = o.target - o.above;
      uint64_t r = (w == 0) ? o.tied : (rem + w - 1) / w;
      if (r < 1) r = 1;
      if (r > o.tied) r = o.tied;
      s_r = uint32_t(r);
      if (tile == 0) {
        const uint32_t cnt = o.cnt_above + uint32_t(r);
        a.sel_count[row] = int32_t(cnt);
        if (a.starts) a.starts[int64_t(row) * (a.nsplit + 1) + a.nsplit] = int32_t(cnt);
      }
    }
  }
  __syncthreads();
  clear_level(a.R, row, 1, tile, a.nblk);             // read last by hist<2>
  const uint32_t t = s_t, r = s_r;
  // ---- tokens of earlier tiles with key > t (pa) and key == t (pe), from their records;
  // tiles whose record overflowed ("heavy") are listed and counted from their scores
  if (wave == 1) {
    const uint32_t tl = t & 1023u;
    uint32_t ca = 0, ce = 0, nh = 0;
    for (int c = 0; c < tile; c += 64) {
      const int i = c + lane;
      const uint4 q = (c == 0) ? rec0 : (i < tile ? rec[i] : make_uint4(0u, 0u, 0u, 0u));
      const uint32_t np = q.x >> 16;
      ca += q.x & 0xFFFFu;
      const bool heavy = np > uint32_t(kRecPairs);
      if (!heavy) {
        const uint32_t pw[kRecPairs] = {q.y, q.z, q.w};
#pragma unroll
        for (int k = 0; k < kRecPairs; ++k) {
          const uint32_t dig = pw[k] & 1023u, cnt = pw[k] >> 10;   // empty pairs have cnt 0
          ca += dig > tl ? cnt : 0u;
          ce += dig == tl ? cnt : 0u;
        }
      }
      const uint64_t hb = __ballot(heavy);
      if (heavy) {
        const uint32_t slot = nh + __popcll(hb & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        if (slot < uint32_t(kMaxHeavy)) s_heavy_list[slot] = uint32_t(i);
      }
      nh += __popcll(hb);
    }
    ca = wave_sum(ca);
    ce = wave_sum(ce);
    if (lane == 0) {
      s_pa = ca;
      s_pe = ce;
      s_heavy = nh;
    }
  }
  // this thread's tokens above t / tied with t, one bit per item (ballots are taken again
  // when writing, so that they need not stay in registers)
  uint32_t fa = 0, fe = 0;
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int64_t j = base + it * kSelThreads + tid;
    const uint32_t key = score_key(sv[it]);
    const bool above = (j < a.n_ctx) && key > t, tied = (j < a.n_ctx) && key == t;
    fa |= uint32_t(above) << it;
    fe |= uint32_t(tied) << it;
    const uint64_t ba = __ballot(above), be = __ballot(tied);
    if (lane == 0) {
      s_wa[it * NW + wave] = __popcll(ba);
      s_we[it * NW + wave] = __popcll(be);
    }
  }
  __syncthreads();
  const uint32_t nheavy = s_heavy;
  if (nheavy) {
    // candidates of the heavy tiles (all earlier tiles when there are too many of them)
    const bool listed = nheavy <= uint32_t(kMaxHeavy);
    const int nt = listed ? int(nheavy) : tile;
    uint32_t ga = 0, ge = 0;
    for (int h = 0; h < nt; ++h) {
      const int64_t tb = int64_t(listed ? s_heavy_list[h] : h) * TILE;
#pragma unroll 4
      for (int k = tid; k < TILE; k += kSelThreads) {
        const uint32_t key = score_key(sp[tb + k]);          // earlier tiles are full: tb + k < base
        const bool cand = (key >> 10) == (t >> 10);
        ga += uint32_t(cand && key > t);
        ge += uint32_t(key == t);
      }
    }
    ga = wave_sum(ga);
    ge = wave_sum(ge);
    if (lane == 0) {
      s_ra[wave] = ga;
      s_re[wave] = ge;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t ga_all = 0, ge_all = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        ga_all += s_ra[w];
        ge_all += s_re[w];
      }
      if (listed) {                 // the records already gave the light tiles' candidates
        s_pa += ga_all;
        s_pe += ge_all;
      } else {                      // recounted every earlier tile: keep only the above-prefix sum
        uint32_t na = 0;
        for (int i = 0; i < tile; ++i) na += rec[i].x & 0xFFFFu;
        s_pa = na + ga_all;
        s_pe = ge_all;
      }
    }
  }
  // This block reads no more of the tile records, the level-2 histogram or the row state:
  // count it as done now, and learn whether it was the last one only at the end.
  uint32_t done_before = 0;
  if (tid == 0) done_before = atomicAdd(ctr + 1, 1u);
  // exclusive prefix of the per-(item, wave) counts, in token order (item-major)
  if (wave == 0) {
    uint32_t va[PL], ve[PL], sa = 0, se = 0;      // lane takes entries PL*lane .. PL*lane+PL-1
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      va[k] = s_wa[PL * lane + k];
      ve[k] = s_we[PL * lane + k];
      sa += va[k];
      se += ve[k];
    }
    uint32_t xa = sa, xe = se;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t ya = __shfl_up(xa, o, 64), ye = __shfl_up(xe, o, 64);
      if (lane >= o) {
        xa += ya;
        xe += ye;
      }
    }
    xa -= sa;
    xe -= se;
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      s_wa[PL * lane + k] = xa;
      s_we[PL * lane + k] = xe;
      xa += va[k];
      xe += ve[k];
    }
  }
  __syncthreads();
  const uint32_t pa = s_pa, pe = s_pe;                 // counts of every earlier token
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* out = a.sel_idx + int64_t(row) * a.n_cap;
  constexpr int IT_PER_RANGE = kDecRange / kSelThreads;      // items per decode range
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const uint32_t ca = pa + s_wa[it * NW + wave], ce = pe + s_we[it * NW + wave];
    if (a.starts && it % IT_PER_RANGE == 0 && tid == 0) {
      // first token of a decode range: the number of selected tokens before it
      const int64_t q = (base + it * kSelThreads) / kDecRange;
      if (q < a.nsplit) a.starts[int64_t(row) * (a.nsplit + 1) + q] = int32_t(ca + (ce < r ? ce : r));
    }
    const bool above = (fa >> it) & 1u, tied = (fe >> it) & 1u;
    const uint32_t a_before = ca + __popcll(__ballot(above) & lt);
    const uint32_t e_before = ce + __popcll(__ballot(tied) & lt);
    const bool take = above || (tied && e_before < r);
    if (take) out[a_before + (e_before < r ? e_before : r)] = int32_t(base + it * kSelThreads + tid);
  }
  // the last block of the row to be counted clears what this launch read: every other
  // block has finished its reads of the tile records, the level-2 histogram and the state
  if (tid == 0) s_last = (done_before == uint32_t(a.nblk - 1));
  __syncthreads();
  if (s_last) {
    for (int i = tid; i < a.nblk; i += kSelThreads) a.R.tilerec[int64_t(row) * a.rec_stride + i] = make_uint4(0u, 0u, 0u, 0u);
    uint32_t* st = reinterpret_cast<uint32_t*>(a.R.state + row);
    if (tid < int(sizeof(SelRowState) / 4)) st[tid] = 0;
    clear_level(a.R, row, 2, 0, 1);
    if (tid == 0) {
      ctr[0] = 0;
      ctr[1] = 0;
    }
  }
}

// top_p >= 1: every token, in order.
__global__ __launch_bounds__(256) void k_sel_all(int n_ctx, int64_t n_cap, int32_t* __restrict__ sel_idx,
                                                 int32_t* __restrict__ sel_count, int32_t* __restrict__ starts,
                                                 int nsplit) {
  const int row = blockIdx.y;
  const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (j < n_ctx) sel_idx[int64_t(row) * n_cap + j] = int32_t(j);
  if (j == 0) sel_count[row] = n_ctx;
  if (starts && j <= nsplit) starts[int64_t(row) * (nsplit + 1) + j] = int32_t(j == nsplit ? n_ctx : j * kDecRange);
}

}  // namespace

namespace rtp {

SelRows sel_rows(void* ws, const SelLayout& lay) {
  char* w = static_cast<char*>(ws);
  return SelRows{reinterpret_cast<uint64_t*>(w + lay.hist_mass), reinterpret_cast<uint32_t*>(w + lay.hist_cnt),
                 reinterpret_cast<uint64_t*>(w + lay.coarse_mass), reinterpret_cast<uint32_t*>(w + lay.coarse_cnt),
                 reinterpret_cast<SelRowState*>(w + lay.state), reinterpret_cast<uint32_t*>(w + lay.ctr),
                 reinterpret_cast<uint4*>(w + lay.tilerec)};
}

}  // namespace rtp

extern "C" rtp_status rtp_topp_select(const rtp_layer_desc* desc, int64_t n_ctx, const float* scores,
                                      const float* row_max, const float* row_sum, float top_p, int32_t* sel_idx,
                                      int32_t* sel_count, int32_t* sel_starts, void* ws, size_t ws_bytes,
                                      void* stream) {
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
  const SelLayout lay = sel_layout(L);
  if (top_p < 1.0f && (!ws || ws_bytes < lay.total || !aligned(ws, 256)))
    return fail(RTP_EWORKSPACE, "rtp_topp_select: workspace needs %zu bytes, 256-aligned (got %zu)", lay.total,
                ws_bytes);
  const int nsplit = int((n_ctx + kDecRange - 1) / kDecRange);
  if (top_p >= 1.0f) {
    hipLaunchKernelGGL(k_sel_all, dim3(unsigned((n_ctx + 255) / 256 + 1), rows), dim3(256), 0, s, int(n_ctx),
                       L.n_cap, sel_idx, sel_count, sel_starts, nsplit);
    return check_launch("k_sel_all");
  }
  SelArgs a{};
  a.scores = scores;
  a.row_max = row_max;
  a.top_p = top_p;
  a.n_ctx = int(n_ctx);
  a.n_cap = L.n_cap;
  a.rec_stride = lay.nblk_max;
  a.sel_idx = sel_idx;
  a.sel_count = sel_count;
  a.starts = sel_starts;
  a.nsplit = nsplit;
  a.R = sel_rows(ws, lay);
  return launch_select(a, rows, s);
}

extern "C" rtp_status rtp_topk_select(const rtp_layer_desc* desc, int64_t n_ctx, const float* scores, int64_t k,
                                      int32_t* sel_idx, int32_t* sel_count, int32_t* sel_starts, void* ws,
                                      size_t ws_bytes, void* stream) {
  Layer L;
  rtp_status st = check_desc(desc, &L);
  if (st != RTP_OK) return st;
  if (n_ctx < 1 || n_ctx > L.n_cap)
    return fail(RTP_EINVAL, "n_ctx must be in [1, n_cap=%lld] (got %lld)", (long long)L.n_cap, (long long)n_ctx);
  if (k < 1) return fail(RTP_EINVAL, "rtp_topk_select: k must be >= 1 (got %lld)", (long long)k);
  if (L.n_ret == 0) return ok();
  if (!scores || !sel_idx || !sel_count) return fail(RTP_EINVAL, "rtp_topk_select: NULL tensor pointer");
  if (!aligned(scores, 16) || !aligned(sel_idx, 16))
    return fail(RTP_EINVAL, "rtp_topk_select: tensors must be 16-byte aligned");
  const int rows = L.B * L.n_ret * L.G;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const SelLayout lay = sel_layout(L);
  if (k < n_ctx && (!ws || ws_bytes < lay.total || !aligned(ws, 256)))
    return fail(RTP_EWORKSPACE, "rtp_topk_select: workspace needs %zu bytes, 256-aligned (got %zu)", lay.total,
                ws_bytes);
  SelArgs a{};
  a.scores = scores;
  a.top_p = k >= n_ctx ? 1.0f : 0.5f;          // >= 1: every token (the k_sel_all path)
  a.by_count = 1;
  a.k_target = k;
  a.n_ctx = int(n_ctx);
  a.n_cap = L.n_cap;
  a.rec_stride = lay.nblk_max;
  a.sel_idx = sel_idx;
  a.sel_count = sel_count;
  a.starts = sel_starts;
  a.nsplit = int((n_ctx + kDecRange - 1) / kDecRange);
  a.R = sel_rows(ws, lay);
  return launch_select(a, rows, s);
}

namespace rtp {

rtp_status launch_select(const SelArgs& a0, int rows, hipStream_t s) {
  rtp_status st;
  const SelArgs& a = a0;
  if (a.top_p >= 1.0f) {
    hipLaunchKernelGGL(k_sel_all, dim3(unsigned((a.n_ctx + 255) / 256 + 1), rows), dim3(256), 0, s, a.n_ctx,
                       a.n_cap, a.sel_idx, a.sel_count, a.starts, a.nsplit);
    return check_launch("k_sel_all");
  }
  // tile size: 16 scores per thread, or 32 when that keeps a pass to one round of blocks
  SelArgs b = a;
  const int64_t nblk16 = (int64_t(a.n_ctx) + kSelTile - 1) / kSelTile;
  b.items = nblk16 * rows > kDecBlocksTarget ? kSelItemsLong : kSelItems;
  b.nblk = int((int64_t(a.n_ctx) + kSelThreads * b.items - 1) / (kSelThreads * b.items));
  const dim3 grid(b.nblk, rows);
  if (b.items == kSelItems) {
    hipLaunchKernelGGL((k_sel_hist<0, kSelItems>), grid, dim3(kSelThreads), 0, s, b);
    if ((st = check_launch("k_sel_hist<0>")) != RTP_OK) return st;
    hipLaunchKernelGGL((k_sel_hist<1, kSelItems>), grid, dim3(kSelThreads), 0, s, b);
    if ((st = check_launch("k_sel_hist<1>")) != RTP_OK) return st;
    hipLaunchKernelGGL((k_sel_hist<2, kSelItems>), grid, dim3(kSelThreads), 0, s, b);
    if ((st = check_launch("k_sel_hist<2>")) != RTP_OK) return st;
    hipLaunchKernelGGL((k_sel_compact<kSelItems>), grid, dim3(kSelThreads), 0, s, b);
  } else {
    hipLaunchKernelGGL((k_sel_hist<0, kSelItemsLong>), grid, dim3(kSelThreads), 0, s, b);
    if ((st = check_launch("k_sel_hist<0>")) != RTP_OK) return st;
    hipLaunchKernelGGL((k_sel_hist<1, kSelItemsLong>), grid, dim3(kSelThreads), 0, s, b);
    if ((st = check_launch("k_sel_hist<1>")) != RTP_OK) return st;
    hipLaunchKernelGGL((k_sel_hist<2, kSelItemsLong>), grid, dim3(kSelThreads), 0, s, b);
    if ((st = check_launch("k_sel_hist<2>")) != RTP_OK) return st;
    hipLaunchKernelGGL((k_sel_compact<kSelItemsLong>), grid, dim3(kSelThreads), 0, s, b);
  }
  return check_launch("k_sel_compact");
}

}  // namespace rtp
