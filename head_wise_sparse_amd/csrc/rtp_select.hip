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
//             token count and the softmax mass exp(s - max) in u64 fixed point (2^-42
//             up to 2^20 tokens, see mass_frac_bits: exact sums, independent of order,
//             bit-reproducible).  Bins are built in
//             LDS per block and added to the row's histogram with global atomics, with a
//             64-bin coarse summary (32 fine bins each) beside it.
//   hist<1,2> the same on key bits [20:10] and [9:0], only for tokens whose higher
//             bits equal the digits resolved so far.  Before that, one wave of every
//             block resolves the previous level's digit from the coarse summary, then
//             from the 32 fine bins under the chosen coarse bin (two small reads): the
//             digit is where the mass accumulated from the top first reaches what is
//             still needed.  The kernel boundary is the only synchronisation.
//             hist<2> also leaves one record per kRecTok tokens (one decode range): how
//             many of them lie above the 22-bit prefix (certainly selected) and, for up
//             to kRecPairs distinct low 10-bit digits among the tokens that share it
//             (candidates), the digit and its count; a record with more such digits
//             than that also gets a table.
//   compact   resolves the last digit (t is now the full key), the tie count r in
//             closed form (tied tokens carry equal weight), and writes the selected
//             indices in increasing order.  A tile's output offset comes from the
//             records of the earlier tiles (written by the previous launch: no waiting
//             on other blocks): tokens above the prefix, plus candidates above t, plus
//             at most r ties.  Candidates share 22 key bits with t, so a record holds few
//             distinct ones (exact ties collapse into one pair).  A record with more
//             distinct candidates than it keeps ("heavy") comes with a table of its
//             candidate counts at or above each low digit, and the block reads the two
//             entries at t from it: O(1) per earlier record whatever the scores.
//             It also writes the range index of every list when asked for.
// The decode step replaces the compaction with k_sel_resolve: one block per row resolves
// t and r and forms the range index from the records alone (the step's gather then takes
// each range's members from its scores and writes the lists).
// Rows of at most kSelSmallMax tokens take one launch instead (k_sel_small): one block per
// row keeps the row's scores in registers and each level's histogram in LDS, and applies
// the same rules, so it writes the same lists, counts and range index.
// The workspace is all zero when a call starts and when it ends, but for the heavy
// records' tables, which the last pass writes whole before anyone reads them: each launch
// clears what earlier launches left and nobody reads any more (hist<2> the level-0
// histogram, compact the level-1 histogram), and the last compaction block of a row to
// finish (in the decode step, the row's resolve block) clears the rest of that row
// (level-2 histogram, records, row state and counters).
#include <cmath>

#include "rtp_internal.hpp"
#include "score_dev.hpp"

using namespace rtp;
using namespace rtp_dev;

namespace {

constexpr int kCoarse = 64;          // coarse bins of levels 0/1 (32 at level 2)
constexpr int kFinePer = 32;         // fine bins under one coarse bin
constexpr int kRecPairs = 3;         // (digit, count) pairs a record holds (one per 32-bit word)

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

// Loads of a finished histogram: global (relaxed atomics, written by earlier launches
// through atomics) or LDS (the single-block path).
struct LdGlobal {
  __device__ __forceinline__ uint64_t operator()(const uint64_t* p) const { return ld_rlx(p); }
  __device__ __forceinline__ uint32_t operator()(const uint32_t* p) const { return ld_rlx(p); }
};
struct LdShared {
  __device__ __forceinline__ uint64_t operator()(const uint64_t* p) const { return *p; }
  __device__ __forceinline__ uint32_t operator()(const uint32_t* p) const { return *p; }
};

// Resolve the digit of `level` from a finished histogram: its coarse summary (nc bins
// of kFinePer fine bins each: cm, cc) and its fine bins (fm, fc).  Called by one full
// wave; every lane returns the same result.  `in` carries the state after the previous
// level (ignored for level 0, where the target is ceil(p * Z), or k when the bins are
// weighed by their counts for the static top-k rule).  The digit is the one where the
// mass accumulated from the top first reaches what is still needed: unique, so any
// split of the bins into coarse groups finds the same one.
template <typename LD>
__device__ __forceinline__ Resolved resolve_digit(const uint64_t* cm, const uint32_t* cc, const uint64_t* fm0,
                                                  const uint32_t* fc0, int nc, int level, const Resolved& in,
                                                  float top_p, bool by_count, int64_t k_target, int lane, LD ld) {
  const uint32_t c_l = lane < nc ? ld(cc + lane) : 0u;
  const uint64_t m_l = by_count ? uint64_t(c_l) : (lane < nc ? ld(cm + lane) : 0ull);
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
  const uint64_t* fm = fm0 + cs * kFinePer;
  const uint32_t* fc = fc0 + cs * kFinePer;
  const uint32_t fc_l = lane < kFinePer ? ld(fc + lane) : 0u;
  const uint64_t fm_l = by_count ? uint64_t(fc_l) : (lane < kFinePer ? ld(fm + lane) : 0ull);
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

// The same from a row's histogram in the workspace.
__device__ Resolved resolve_level(const SelRows& R, int row, int level, const Resolved& in, float top_p,
                                  bool by_count, int64_t k_target, int lane) {
  const int64_t h = int64_t(row) * 3 + level;
  return resolve_digit(R.cmass + h * kCoarse, R.ccnt + h * kCoarse, R.mass + h * kBins, R.cnt + h * kBins,
                       level == 2 ? 32 : kCoarse, level, in, top_p, by_count, k_target, lane, LdGlobal{});
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

// Clear records [0, nrec) of a row (the whole block).  The heavy records' tables are left:
// the last pass writes a record's table whole before anyone reads it.
__device__ __forceinline__ void clear_records(const SelRows& R, int row, int rec_stride, int nrec) {
  uint4* rrow = R.tilerec + int64_t(row) * rec_stride;
  for (int i = threadIdx.x; i < nrec; i += kSelThreads) rrow[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Row max (and, by the first block, the row statistics) from the scoring's per-block
// (max, sum of exp) partials.
__device__ float row_max_from_partials(const SelArgs& a, int row, int blk, int tid, float* s_red, int n_ctx) {
  const float2* p = a.score_part + int64_t(row) * a.score_nblk;
  const int nb = (n_ctx + kScoreTile - 1) / kScoreTile;        // partials of the live context
  float m = -INFINITY;
  for (int i = tid; i < nb; i += kSelThreads) m = fmaxf(m, p[i].x);
  m = wave_max(m);
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  // the row statistics, by the same one-wave reduction as rtp_indexer_score's
  if (blk == 0 && a.row_max_out && tid < 64)
    score_finalize_row(a.score_part, a.score_nblk, nb, a.row_max_out, a.row_sum_out, row);
  return m;
}

template <int LEVEL, int ITEMS>
__global__ __launch_bounds__(kSelThreads) void k_sel_hist(SelArgs a) {
  constexpr int TILE = kSelThreads * ITEMS;
  constexpr int NB = LEVEL == 2 ? 1024 : 2048;
  constexpr int SHIFT = LEVEL == 0 ? 21 : (LEVEL == 1 ? 10 : 0);
  constexpr int PSHIFT = LEVEL == 1 ? 21 : 10;                     // prefix bits start (levels 1, 2)
  constexpr int IPR = kRecTok / kSelThreads;                       // items per record
  constexpr int NR = LEVEL == 2 ? ITEMS / IPR : 1;                 // level 2: records per tile (even)
  constexpr int NW = kSelThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int blk = blockIdx.x, row = blockIdx.y;
  __shared__ uint64_t h_m[NB];
  __shared__ uint32_t h_c[NB];
  __shared__ uint32_t s_prefix;
  __shared__ float s_red[NW];
  // level 2: per record, tokens above the prefix (per wave), distinct candidate digits and
  // the first kRecPairs (digit, count) pairs; candidate counts per low digit, two records
  // per word (16-bit halves: a record holds at most kRecTok tokens); cross-wave sums
  __shared__ uint32_t s_na[NR][NW], s_np[NR], s_pair[NR][kRecPairs];
  __shared__ uint32_t h_s[LEVEL == 2 ? NR / 2 : 1][LEVEL == 2 ? 1024 : 1];
  __shared__ uint32_t s_wt[LEVEL == 2 ? NR / 2 : 1][NW];
  const int n_ctx = live_ctx(a.live, a.n_ctx);
  const int nblk = int((int64_t(n_ctx) + TILE - 1) / TILE);       // tiles of the live context
  if (blk >= nblk) return;
  const float wscale = mass_wscale(n_ctx);

  // scores of the tile: unconditional loads (index clamped), validity kept aside
  const float* sp = a.scores + int64_t(row) * a.n_cap;
  const int64_t base = int64_t(blk) * TILE;
  float sv[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int64_t j = base + it * kSelThreads + tid;
    sv[it] = sp[j < n_ctx ? j : n_ctx - 1];
  }
  for (int i = tid; i < NB; i += kSelThreads) {
    h_m[i] = 0;
    h_c[i] = 0;
  }
  if constexpr (LEVEL == 2) {
    for (int i = tid; i < NR / 2 * 1024; i += kSelThreads) (&h_s[0][0])[i] = 0;
    if (tid < NR) s_np[tid] = 0;
  }
  float m = 0.0f;                                   // unused by the static top-k rule
  if constexpr (LEVEL == 0) {
    if (!a.by_count) m = a.score_part ? row_max_from_partials(a, row, blk, tid, s_red, n_ctx) : a.row_max[row];
    if (blk == 0 && tid == 0) a.R.state[row].ref_max = m;
  } else {
    m = a.R.state[row].ref_max;                      // written by the level-0 launch
  }
  if constexpr (LEVEL == 2) clear_level(a.R, row, 0, blk, nblk);   // read last by hist<1>
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
  uint32_t n_above[NR] = {};                        // level 2: tokens above the 22-bit prefix, per record
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int64_t j = base + it * kSelThreads + tid;
    const uint32_t key = score_key(sv[it]);
    const bool match = (j < n_ctx) && (LEVEL == 0 || (key >> PSHIFT) == prefix);
    if (match) {
      const uint32_t d = (key >> SHIFT) & uint32_t(NB - 1);
      if (!a.by_count) atomicAdd(reinterpret_cast<unsigned long long*>(&h_m[d]), (unsigned long long)fixed_weight(sv[it], m, wscale));
      atomicAdd(&h_c[d], 1u);
      if constexpr (LEVEL == 2) atomicAdd(&h_s[it / IPR / 2][d], 1u << (16 * ((it / IPR) & 1)));
    }
    if constexpr (LEVEL == 2) n_above[it / IPR] += uint32_t((j < n_ctx) && (key >> PSHIFT) > prefix);
  }
  if constexpr (LEVEL == 2) {
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const uint32_t na = wave_sum(n_above[k]);
      if (lane == 0) s_na[k][tid / 64] = na;
    }
  }
  __syncthreads();

  uint64_t* gm = a.R.mass + (int64_t(row) * 3 + LEVEL) * kBins;
  uint32_t* gc = a.R.cnt + (int64_t(row) * 3 + LEVEL) * kBins;
  for (int i = tid; i < NB; i += kSelThreads) {
    if (h_c[i]) {
      if (!a.by_count) atomicAdd(reinterpret_cast<unsigned long long*>(gm + i), (unsigned long long)h_m[i]);
      atomicAdd(gc + i, h_c[i]);
      if constexpr (LEVEL == 2) {              // each record's distinct candidate digits
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const uint32_t c = (h_s[k / 2][i] >> (16 * (k & 1))) & 0xFFFFu;
          if (c) {
            const uint32_t e = atomicAdd(&s_np[k], 1u);
            if (e < uint32_t(kRecPairs)) s_pair[k][e] = uint32_t(i) | (c << 10);
          }
        }
      }
    }
  }
  if constexpr (LEVEL == 2) {
    __syncthreads();
    const int64_t rec0 = int64_t(blk) * NR;                       // this tile's first record
    if (tid < NR && (rec0 + tid) * kRecTok < n_ctx) {             // records of the live context
      uint32_t na = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) na += s_na[tid][w];
      const uint32_t np = s_np[tid];
      uint32_t pw[kRecPairs];
#pragma unroll
      for (int k = 0; k < kRecPairs; ++k) pw[k] = uint32_t(k) < np ? s_pair[tid][k] : 0u;
      a.R.tilerec[int64_t(row) * a.rec_stride + rec0 + tid] = make_uint4(na | (np << 16), pw[0], pw[1], pw[2]);
    }
    bool heavy = false;
#pragma unroll
    for (int k = 0; k < NR; ++k) heavy |= s_np[k] > uint32_t(kRecPairs);
    if (heavy) {
      // A record that cannot hold its candidates: leave their counts at or above every low
      // digit d (inclusive suffix sums of the record's level-2 counts, <= kRecTok), from
      // which the range index reads the two it needs once the threshold digit is known.
      // Two records per word are summed at once (16-bit halves never carry).  Thread tid
      // owns digits 4 tid .. 4 tid + 3; higher threads hold higher digits.
      uint32_t c[NR / 2][4], own[NR / 2], in_wave[NR / 2];
#pragma unroll
      for (int w = 0; w < NR / 2; ++w) {
#pragma unroll
        for (int k = 0; k < 4; ++k) c[w][k] = h_s[w][4 * tid + k];
        own[w] = c[w][0] + c[w][1] + c[w][2] + c[w][3];
        in_wave[w] = wave_suffix_incl<uint32_t>(own[w], lane);   // own + higher lanes of the wave
        if (lane == 0) s_wt[w][tid / 64] = in_wave[w];
      }
      __syncthreads();
#pragma unroll
      for (int w = 0; w < NR / 2; ++w) {
        uint32_t hi = in_wave[w] - own[w];                         // digits above this thread's four
        for (int v = tid / 64 + 1; v < NW; ++v) hi += s_wt[w][v];
        const uint32_t s3 = hi + c[w][3], s2 = s3 + c[w][2], s1 = s2 + c[w][1], s0 = s1 + c[w][0];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (s_np[2 * w + h] > uint32_t(kRecPairs)) {
            const int sh = 16 * h;
            const uint32_t e0 = (s0 >> sh) & 0xFFFFu, e1 = (s1 >> sh) & 0xFFFFu;
            const uint32_t e2 = (s2 >> sh) & 0xFFFFu, e3 = (s3 >> sh) & 0xFFFFu;
            uint2* tab = reinterpret_cast<uint2*>(a.R.tiletab +
                                                  (int64_t(row) * a.rec_stride + rec0 + 2 * w + h) * kTabDigits);
            tab[tid] = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
          }
        }
      }
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
  __shared__ uint32_t s_pa[NW], s_pe[NW], s_last;
  const int n_ctx = live_ctx(a.live, a.n_ctx);
  const int nblk = int((int64_t(n_ctx) + TILE - 1) / TILE);       // tiles of the live context
  if (tile >= nblk) return;
  const int nsplit = (n_ctx + kDecRange - 1) / kDecRange;         // ranges of the live context
  const float wscale = mass_wscale(n_ctx);
  uint32_t* ctr = a.R.ctr + 2 * int64_t(row);
  const uint4* rec = a.R.tilerec + int64_t(row) * a.rec_stride;
  const float* sp = a.scores + int64_t(row) * a.n_cap;
  const int64_t base = int64_t(tile) * TILE;
  float sv[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int64_t j = base + it * kSelThreads + tid;
    sv[it] = sp[j < n_ctx ? j : n_ctx - 1];
  }
  const int nrec = tile * (TILE / kRecTok);           // records of the earlier tiles
  constexpr int RPT = 4;                              // records per thread per round
  uint4 rq[RPT];                                      // the first round, issued before the resolve
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int i = tid * RPT + k;
    rq[k] = i < nrec ? rec[i] : make_uint4(0u, 0u, 0u, 0u);
  }
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
      const uint64_t w = a.by_count ? 1ull : fixed_weight(key_score(o.prefix), a.R.state[row].ref_max, wscale);
      const uint64_t rem = o.target - o.above;
      uint64_t r = (w == 0) ? o.tied : (rem + w - 1) / w;
      if (r < 1) r = 1;
      if (r > o.tied) r = o.tied;
      s_r = uint32_t(r);
      if (tile == 0) {
        const uint32_t cnt = o.cnt_above + uint32_t(r);
        a.sel_count[row] = int32_t(cnt);
        if (a.starts) a.starts[int64_t(row) * (a.nsplit + 1) + nsplit] = int32_t(cnt);
      }
    }
  }
  __syncthreads();
  clear_level(a.R, row, 1, tile, nblk);             // read last by hist<2>
  const uint32_t t = s_t, r = s_r;
  // ---- tokens of earlier tiles with key > t (pa) and key == t (pe), from their records,
  // or, for a record that overflowed ("heavy"), from two entries of its table; the whole
  // block takes RPT records per thread per round
  const uint16_t* tab = a.R.tiletab + int64_t(row) * a.rec_stride * kTabDigits;
  {
    const uint32_t tl = t & 1023u;
    uint32_t ca = 0, ce = 0;
    for (int c0 = 0; c0 < nrec; c0 += kSelThreads * RPT) {
      if (c0 > 0) {
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
          const int i = c0 + tid * RPT + k;
          rq[k] = i < nrec ? rec[i] : make_uint4(0u, 0u, 0u, 0u);
        }
      }
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const uint4 q = rq[k];
        ca += q.x & 0xFFFFu;
        if ((q.x >> 16) > uint32_t(kRecPairs)) {
          const uint16_t* ti = tab + int64_t(c0 + tid * RPT + k) * kTabDigits;
          const uint32_t ge = ti[tl], gt = tl < 1023u ? uint32_t(ti[tl + 1]) : 0u;   // digit >= tl, > tl
          ca += gt;
          ce += ge - gt;
        } else {
          const uint32_t pw[kRecPairs] = {q.y, q.z, q.w};
#pragma unroll
          for (int e = 0; e < kRecPairs; ++e) {
            const uint32_t dig = pw[e] & 1023u, cnt = pw[e] >> 10;   // empty pairs have cnt 0
            ca += dig > tl ? cnt : 0u;
            ce += dig == tl ? cnt : 0u;
          }
        }
      }
    }
    ca = wave_sum(ca);
    ce = wave_sum(ce);
    if (lane == 0) {
      s_pa[wave] = ca;
      s_pe[wave] = ce;
    }
  }
  // this thread's tokens above t / tied with t, one bit per item (ballots are taken again
  // when writing, so that they need not stay in registers)
  uint32_t fa = 0, fe = 0;
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int64_t j = base + it * kSelThreads + tid;
    const uint32_t key = score_key(sv[it]);
    const bool above = (j < n_ctx) && key > t, tied = (j < n_ctx) && key == t;
    fa |= uint32_t(above) << it;
    fe |= uint32_t(tied) << it;
    const uint64_t ba = __ballot(above), be = __ballot(tied);
    if (lane == 0) {
      s_wa[it * NW + wave] = __popcll(ba);
      s_we[it * NW + wave] = __popcll(be);
    }
  }
  __syncthreads();
  // This block reads no more of the records and tables, the level-2 histogram or the row state:
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
  uint32_t pa = 0, pe = 0;                            // counts of every earlier token
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    pa += s_pa[w];
    pe += s_pe[w];
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* out = a.sel_idx + int64_t(row) * a.n_cap;
  constexpr int IT_PER_RANGE = kDecRange / kSelThreads;      // items per decode range
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const uint32_t ca = pa + s_wa[it * NW + wave], ce = pe + s_we[it * NW + wave];
    if (a.starts && it % IT_PER_RANGE == 0 && tid == 0) {
      // first token of a decode range: the number of selected tokens before it
      const int64_t q = (base + it * kSelThreads) / kDecRange;
      if (q < nsplit) a.starts[int64_t(row) * (a.nsplit + 1) + q] = int32_t(ca + (ce < r ? ce : r));
    }
    const bool above = (fa >> it) & 1u, tied = (fe >> it) & 1u;
    const uint32_t a_before = ca + __popcll(__ballot(above) & lt);
    const uint32_t e_before = ce + __popcll(__ballot(tied) & lt);
    const bool take = above || (tied && e_before < r);
    if (take) out[a_before + (e_before < r ? e_before : r)] = int32_t(base + it * kSelThreads + tid);
  }
  // the last block of the row to be counted clears what this launch read: every other
  // block has finished its reads of the records, the level-2 histogram and the state
  if (tid == 0) s_last = (done_before == uint32_t(nblk - 1));
  __syncthreads();
  if (s_last) {
    clear_records(a.R, row, a.rec_stride, (n_ctx + kRecTok - 1) / kRecTok);   // those of the live context
    uint32_t* st = reinterpret_cast<uint32_t*>(a.R.state + row);
    if (tid < int(sizeof(SelRowState) / 4)) st[tid] = 0;
    clear_level(a.R, row, 2, 0, 1);
    if (tid == 0) {
      ctr[0] = 0;
      ctr[1] = 0;
    }
  }
}

// Decode step, after hist<2>: one block per row resolves the last digit and the tie count,
// writes the count, the threshold key t and the range index, and clears the row's
// workspace.  Range q's entry is the number of selected tokens below its start: the
// tokens above t and at most r of the ties in the records of ranges 0 .. q-1 (a scan
// over the records).  The gather then takes range q's members from its own scores: every
// token with key > t, and the first (starts[q+1] - starts[q] - #above) with key == t --
// the same list the compaction writes.
__global__ __launch_bounds__(kSelThreads) void k_sel_resolve(SelArgs a) {
  constexpr int NW = kSelThreads / 64;
  constexpr int RPT = 4;                                         // records per thread per round
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int row = blockIdx.x;
  __shared__ uint32_t s_t, s_r;
  __shared__ uint32_t s_wa[NW], s_we[NW];
  const int n_ctx = live_ctx(a.live, a.n_ctx);
  const int nrec = (n_ctx + kRecTok - 1) / kRecTok;              // records = ranges of the live context
  const float wscale = mass_wscale(n_ctx);
  const uint4* rec = a.R.tilerec + int64_t(row) * a.rec_stride;
  const uint16_t* tab = a.R.tiletab + int64_t(row) * a.rec_stride * kTabDigits;
  int32_t* st_out = a.starts + int64_t(row) * (a.nsplit + 1);
  uint4 q[RPT];                                                  // the first round, loaded beside the resolve
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int i = tid * RPT + k;
    q[k] = i < nrec ? rec[i] : make_uint4(0u, 0u, 0u, 0u);
  }
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
      const uint64_t w = a.by_count ? 1ull : fixed_weight(key_score(o.prefix), a.R.state[row].ref_max, wscale);
      const uint64_t rem = o.target - o.above;
      uint64_t r = (w == 0) ? o.tied : (rem + w - 1) / w;
      if (r < 1) r = 1;
      if (r > o.tied) r = o.tied;
      s_t = o.prefix;
      s_r = uint32_t(r);
      const uint32_t cnt = o.cnt_above + uint32_t(r);
      a.sel_count[row] = int32_t(cnt);
      st_out[nrec] = int32_t(cnt);
      a.thr_out[row] = o.prefix;
    }
  }
  __syncthreads();
  const uint32_t t = s_t, r = s_r, tl = t & 1023u;
  uint32_t carry_a = 0, carry_e = 0;                             // counts of the earlier rounds
  for (int c0 = 0; c0 < nrec; c0 += kSelThreads * RPT) {
    if (c0 > 0) {
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int i = c0 + tid * RPT + k;
        q[k] = i < nrec ? rec[i] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // each record's tokens above t (ca) and tied with t (ce): the pairs, or two entries of
    // its table when it overflowed
    uint32_t ca[RPT], ce[RPT], ta = 0, te = 0;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int i = c0 + tid * RPT + k;
      ca[k] = q[k].x & 0xFFFFu;
      ce[k] = 0;
      if ((q[k].x >> 16) > uint32_t(kRecPairs)) {
        const uint16_t* ti = tab + int64_t(i) * kTabDigits;
        const uint32_t ge = ti[tl], gt = tl < 1023u ? uint32_t(ti[tl + 1]) : 0u;   // digit >= tl, > tl
        ca[k] += gt;
        ce[k] = ge - gt;
      } else {
        const uint32_t pw[kRecPairs] = {q[k].y, q[k].z, q[k].w};
#pragma unroll
        for (int e = 0; e < kRecPairs; ++e) {
          const uint32_t dig = pw[e] & 1023u, cnt = pw[e] >> 10;   // empty pairs have cnt 0
          ca[k] += dig > tl ? cnt : 0u;
          ce[k] += dig == tl ? cnt : 0u;
        }
      }
      ta += ca[k];
      te += ce[k];
    }
    // exclusive prefix over the records in index order (thread-major, RPT per thread)
    uint32_t ia = ta, ie = te;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t ya = __shfl_up(ia, o, 64), ye = __shfl_up(ie, o, 64);
      if (lane >= o) {
        ia += ya;
        ie += ye;
      }
    }
    if (lane == 63) {
      s_wa[wave] = ia;
      s_we[wave] = ie;
    }
    __syncthreads();
    uint32_t xa = carry_a + ia - ta, xe = carry_e + ie - te;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) {
        xa += s_wa[w];
        xe += s_we[w];
      }
      carry_a += s_wa[w];
      carry_e += s_we[w];
    }
    uint4* rw = a.R.tilerec + int64_t(row) * a.rec_stride;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int i = c0 + tid * RPT + k;
      if (i < nrec) {
        st_out[i] = int32_t(xa + (xe < r ? xe : r));
        rw[i] = make_uint4(0u, 0u, 0u, 0u);                      // this block is the records' last reader
      }
      xa += ca[k];
      xe += ce[k];
    }
    __syncthreads();                                             // s_wa / s_we are reused
  }
  // this block was the only reader of the level-2 histogram and the state (the heavy records'
  // tables are left: each is written whole before it is read)
  clear_level(a.R, row, 1, 0, 1);
  clear_level(a.R, row, 2, 0, 1);
  uint32_t* st = reinterpret_cast<uint32_t*>(a.R.state + row);
  if (tid < int(sizeof(SelRowState) / 4)) st[tid] = 0;
}

// Rows of at most kSelSmallMax tokens: one block holds the whole row in registers, so the
// three levels and the compaction run in one launch, with each level's histogram in LDS
// and no workspace.  The keys, fixed-point weights, row max, owner rule and tie count are
// those of the four-launch path; the list, its count and the range index are unique
// functions of them, so both paths write the same bits.
template <int LEVEL, int ITEMS>
__device__ __forceinline__ Resolved small_level(const SelArgs& a, const float (&sv)[ITEMS], float m, float wscale,
                                                int n_ctx, const Resolved& in, uint64_t* h_m, uint32_t* h_c,
                                                uint64_t* c_m, uint32_t* c_c, Resolved* s_res) {
  constexpr int NB = LEVEL == 2 ? 1024 : 2048;
  constexpr int SHIFT = LEVEL == 0 ? 21 : (LEVEL == 1 ? 10 : 0);
  constexpr int PSHIFT = LEVEL == 1 ? 21 : 10;
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < NB; i += kSelThreads) {
    h_m[i] = 0;
    h_c[i] = 0;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int j = it * kSelThreads + tid;
    const uint32_t key = score_key(sv[it]);
    if (j < n_ctx && (LEVEL == 0 || (key >> PSHIFT) == in.prefix)) {
      const uint32_t d = (key >> SHIFT) & uint32_t(NB - 1);
      if (!a.by_count) atomicAdd(reinterpret_cast<unsigned long long*>(&h_m[d]), (unsigned long long)fixed_weight(sv[it], m, wscale));
      atomicAdd(&h_c[d], 1u);
    }
  }
  __syncthreads();
  if (tid < NB / kFinePer) {
    uint64_t sm = 0;
    uint32_t sc = 0;
#pragma unroll 8
    for (int i = 0; i < kFinePer; ++i) {
      const int f = tid * kFinePer + ((i + tid) & (kFinePer - 1));
      sm += h_m[f];
      sc += h_c[f];
    }
    c_m[tid] = sm;
    c_c[tid] = sc;
  }
  __syncthreads();
  if (tid < 64) {
    const Resolved o =
        resolve_digit(c_m, c_c, h_m, h_c, NB / kFinePer, LEVEL, in, a.top_p, a.by_count, a.k_target, lane, LdShared{});
    if (lane == 0) *s_res = o;
  }
  __syncthreads();
  return *s_res;
}

template <int ITEMS>
__global__ __launch_bounds__(kSelThreads) void k_sel_small(SelArgs a) {
  constexpr int NW = kSelThreads / 64;
  constexpr int PL = ITEMS * NW / 64;                 // (item, wave) counts per lane of the scanning wave
  static_assert(ITEMS * NW % 64 == 0 && ITEMS * kSelThreads <= kSelSmallMax, "one block, one scanning wave");
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int row = blockIdx.x;
  __shared__ uint64_t h_m[kBins];
  __shared__ uint32_t h_c[kBins];
  __shared__ uint64_t c_m[kCoarse];
  __shared__ uint32_t c_c[kCoarse];
  __shared__ Resolved s_res;
  __shared__ float s_red[NW];
  __shared__ uint32_t s_wa[ITEMS * NW], s_we[ITEMS * NW];   // counts, then exclusive prefixes
  __shared__ uint32_t s_r;
  const int n_ctx = live_ctx(a.live, a.n_ctx);
  const int nsplit = (n_ctx + kDecRange - 1) / kDecRange;         // ranges of the live context
  const float wscale = mass_wscale(n_ctx);
  const float* sp = a.scores + int64_t(row) * a.n_cap;
  float sv[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int j = it * kSelThreads + tid;
    sv[it] = sp[j < n_ctx ? j : n_ctx - 1];
  }
  float m = 0.0f;                                   // unused by the static top-k rule
  if (!a.by_count) m = a.score_part ? row_max_from_partials(a, row, 0, tid, s_red, n_ctx) : a.row_max[row];
  Resolved res{};
  res = small_level<0, ITEMS>(a, sv, m, wscale, n_ctx, res, h_m, h_c, c_m, c_c, &s_res);
  res = small_level<1, ITEMS>(a, sv, m, wscale, n_ctx, res, h_m, h_c, c_m, c_c, &s_res);
  res = small_level<2, ITEMS>(a, sv, m, wscale, n_ctx, res, h_m, h_c, c_m, c_c, &s_res);
  const uint32_t t = res.prefix;
  constexpr int IT_PER_RANGE = kDecRange / kSelThreads;      // items per decode range
  if (tid == 0) {
    // tied tokens share one weight (1 for top-k): take just enough of them to reach the target
    const uint64_t w = a.by_count ? 1ull : fixed_weight(key_score(t), m, wscale);
    const uint64_t rem = res.target - res.above;
    uint64_t r = (w == 0) ? res.tied : (rem + w - 1) / w;
    if (r < 1) r = 1;
    if (r > res.tied) r = res.tied;
    s_r = uint32_t(r);
    const uint32_t cnt = res.cnt_above + uint32_t(r);
    a.sel_count[row] = int32_t(cnt);
    if (a.starts) a.starts[int64_t(row) * (a.nsplit + 1) + nsplit] = int32_t(cnt);
    if (a.thr_out) a.thr_out[row] = t;
  }
  uint32_t fa = 0, fe = 0;
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int j = it * kSelThreads + tid;
    const uint32_t key = score_key(sv[it]);
    const bool above = j < n_ctx && key > t, tied = j < n_ctx && key == t;
    fa |= uint32_t(above) << it;
    fe |= uint32_t(tied) << it;
    const uint64_t ba = __ballot(above), be = __ballot(tied);
    if (lane == 0) {
      s_wa[it * NW + wave] = __popcll(ba);
      s_we[it * NW + wave] = __popcll(be);
    }
  }
  __syncthreads();
  // exclusive prefix of the per-(item, wave) counts, in token order (item-major)
  if (wave == 0) {
    uint32_t va[PL], ve[PL], sa = 0, se = 0;
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
  const uint32_t r = s_r;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* out = a.sel_idx + int64_t(row) * a.n_cap;
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const uint32_t ca = s_wa[it * NW + wave], ce = s_we[it * NW + wave];
    if (a.starts && it % IT_PER_RANGE == 0 && tid == 0 && it / IT_PER_RANGE < nsplit)
      a.starts[int64_t(row) * (a.nsplit + 1) + it / IT_PER_RANGE] = int32_t(ca + (ce < r ? ce : r));
    const bool above = (fa >> it) & 1u, tied = (fe >> it) & 1u;
    const uint32_t a_before = ca + __popcll(__ballot(above) & lt);
    const uint32_t e_before = ce + __popcll(__ballot(tied) & lt);
    const bool take = above || (tied && e_before < r);
    if (take && !a.thr_out) out[a_before + (e_before < r ? e_before : r)] = it * kSelThreads + tid;
  }
}

// top_p >= 1: every token, in order.
// (nsplit: the range index's row stride - 1; live: the device-length step's context word)
__global__ __launch_bounds__(256) void k_sel_all(int n_max, const int64_t* live, int64_t n_cap,
                                                 int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count,
                                                 int32_t* __restrict__ starts, int nsplit) {
  const int row = blockIdx.y;
  const int n_ctx = live_ctx(live, n_max);
  const int nl = (n_ctx + kDecRange - 1) / kDecRange;
  const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (j < n_ctx) sel_idx[int64_t(row) * n_cap + j] = int32_t(j);
  if (j == 0) sel_count[row] = n_ctx;
  if (starts && j <= nl) starts[int64_t(row) * (nsplit + 1) + j] = int32_t(j == nl ? n_ctx : j * kDecRange);
}

}  // namespace

namespace rtp {

SelRows sel_rows(void* ws, const SelLayout& lay) {
  char* w = static_cast<char*>(ws);
  return SelRows{reinterpret_cast<uint64_t*>(w + lay.hist_mass), reinterpret_cast<uint32_t*>(w + lay.hist_cnt),
                 reinterpret_cast<uint64_t*>(w + lay.coarse_mass), reinterpret_cast<uint32_t*>(w + lay.coarse_cnt),
                 reinterpret_cast<SelRowState*>(w + lay.state), reinterpret_cast<uint32_t*>(w + lay.ctr),
                 reinterpret_cast<uint4*>(w + lay.tilerec), reinterpret_cast<uint16_t*>(w + lay.tiletab)};
}

}  // namespace rtp

extern "C" rtp_status rtp_topp_select(const rtp_layer_desc* desc, int64_t n_ctx, const float* scores,
                                      const float* row_max, const float* row_sum, float top_p, int32_t* sel_idx,
                                      int32_t* sel_count, int32_t* sel_starts, void* ws, size_t ws_bytes,
                                      void* stream) {
  TraceRange trace_("rtp_topp_select");
  (void)row_sum;
  Layer L;
  rtp_status st = check_desc(desc, &L);
  if (st != RTP_OK) return st;
  if (n_ctx < 1 || n_ctx > L.n_cap)
    return fail(RTP_EINVAL, "n_ctx must be in [1, n_cap=%lld] (got %lld)", (long long)L.n_cap, (long long)n_ctx);
  if (!(top_p > 0.0f)) return fail(RTP_EINVAL, "top_p must be > 0 (got %g)", double(top_p));
  if (top_p < 1.0f && n_ctx > kTopPMaxCtx)
    return fail(RTP_EUNSUPPORTED, "rtp_topp_select: top_p < 1 needs n_ctx <= 2^24 (got %lld)", (long long)n_ctx);
  if (L.n_ret == 0) return ok();
  if (!scores || !row_max || !sel_idx || !sel_count) return fail(RTP_EINVAL, "rtp_topp_select: NULL tensor pointer");
  if (!aligned(scores, 16) || !aligned(sel_idx, 16))
    return fail(RTP_EINVAL, "rtp_topp_select: tensors must be 16-byte aligned");
  const int rows = L.B * L.n_ret * L.G;
  if ((st = enqueue_gate("rtp_topp_select")) != RTP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const SelLayout lay = sel_layout(L);
  if (top_p < 1.0f && (!ws || ws_bytes < lay.total || !aligned(ws, 256)))
    return fail(RTP_EWORKSPACE, "rtp_topp_select: workspace needs %zu bytes, 256-aligned (got %zu)", lay.total,
                ws_bytes);
  const int nsplit = int((n_ctx + kDecRange - 1) / kDecRange);
  if (top_p >= 1.0f) {
    hipLaunchKernelGGL(k_sel_all, dim3(unsigned((n_ctx + 255) / 256 + 1), rows), dim3(256), 0, s, int(n_ctx),
                       nullptr, L.n_cap, sel_idx, sel_count, sel_starts, nsplit);
    return check_launch("k_sel_all");
  }
  SelArgs a{};
  a.scores = scores;
  a.row_max = row_max;
  a.top_p = top_p;
  a.n_ctx = int(n_ctx);
  a.n_cap = L.n_cap;
  a.rec_stride = lay.nrec_max;
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
  TraceRange trace_("rtp_topk_select");
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
  if ((st = enqueue_gate("rtp_topk_select")) != RTP_OK) return st;
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
  a.rec_stride = lay.nrec_max;
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
                       a.live, a.n_cap, a.sel_idx, a.sel_count, a.starts, a.nsplit);
    return check_launch("k_sel_all");
  }
  if (a.n_ctx <= kSelSmallMax) {         // one block per row (with thr_out: no lists, the gather writes them)
    if (a.n_ctx <= kSelThreads * kSelItems)
      hipLaunchKernelGGL((k_sel_small<kSelItems>), dim3(rows), dim3(kSelThreads), 0, s, a);
    else
      hipLaunchKernelGGL((k_sel_small<kSelItemsLong>), dim3(rows), dim3(kSelThreads), 0, s, a);
    return check_launch("k_sel_small");
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
    if (b.thr_out) {
      hipLaunchKernelGGL(k_sel_resolve, dim3(rows), dim3(kSelThreads), 0, s, b);
      return check_launch("k_sel_resolve");
    }
    hipLaunchKernelGGL((k_sel_compact<kSelItems>), grid, dim3(kSelThreads), 0, s, b);
  } else {
    hipLaunchKernelGGL((k_sel_hist<0, kSelItemsLong>), grid, dim3(kSelThreads), 0, s, b);
    if ((st = check_launch("k_sel_hist<0>")) != RTP_OK) return st;
    hipLaunchKernelGGL((k_sel_hist<1, kSelItemsLong>), grid, dim3(kSelThreads), 0, s, b);
    if ((st = check_launch("k_sel_hist<1>")) != RTP_OK) return st;
    hipLaunchKernelGGL((k_sel_hist<2, kSelItemsLong>), grid, dim3(kSelThreads), 0, s, b);
    if ((st = check_launch("k_sel_hist<2>")) != RTP_OK) return st;
    if (b.thr_out) {
      hipLaunchKernelGGL(k_sel_resolve, dim3(rows), dim3(kSelThreads), 0, s, b);
      return check_launch("k_sel_resolve");
    }
    hipLaunchKernelGGL((k_sel_compact<kSelItemsLong>), grid, dim3(kSelThreads), 0, s, b);
  }
  return check_launch("k_sel_compact");
}

}  // namespace rtp
