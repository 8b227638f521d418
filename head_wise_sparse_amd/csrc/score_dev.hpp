// Device body of the indexer scoring (shared by rtp_indexer_score and the fused
// decode step).  See rtp_score.hip for what it computes.
#pragma once

#include "rtp_internal.hpp"

using namespace rtp;
using namespace rtp_dev;

namespace {

struct ScoreArgs {
  const uint16_t* q_pre;       // [B][Hq][D]
  const uint16_t* w_q;         // per retrieval query head, w_stride elements apart
  int64_t w_stride;
  const uint16_t* k_idx;       // [B][Hkv_r][n_cap][16]
  float idx_scale;
  float* scores;               // [B][Hq_r][n_cap]
  float2* part;                // [B][Hq_r][nblk] per-block (max, sum of exp)
  int n_ctx;                   // the context (device-length step: its bound)
  const int64_t* live;         // device-length step: the context's device word, else null
  int64_t n_cap;
  int Hq;
  HeadMap map;
  int nblk;                    // tiles of n_ctx: the row stride of `part`
};

// One block of the indexer scoring: token tile `blk` of group `grp` (= b * n_ret + r),
// indexer dimension IDX (16 on the pages' design).
template <int G, int D, int IDX = kIdxDim>
__device__ __forceinline__ void score_block(const ScoreArgs& A, int blk, int grp) {
  constexpr int ITEMS = score_items(IDX);
  constexpr int TILE = score_tile(IDX);
  constexpr int KW = IDX / 2;                             // 32-bit words of one indexer key
  const uint16_t* __restrict__ q_pre = A.q_pre;
  const uint16_t* __restrict__ w_q = A.w_q;
  const int64_t w_stride = A.w_stride;
  const uint16_t* __restrict__ k_idx = A.k_idx;
  const float idx_scale = A.idx_scale;
  float* __restrict__ scores = A.scores;
  float2* __restrict__ part = A.part;
  const int n_ctx = live_ctx(A.live, A.n_ctx);
  if (int64_t(blk) * TILE >= n_ctx) return;              // a tile past the live context
  const int64_t n_cap = A.n_cap;
  const int Hq = A.Hq;
  const HeadMap& map = A.map;
  const int nblk = A.nblk;
  const int tid = threadIdx.x;
  const int b = grp / map.n, r = grp % map.n;
  const int g = map.kv[r];

  // LDS: raw bf16 q_pre rows and projection matrices of the group (padded so that every
  // lane of a direct-to-LDS load has a slot), the fp32 q_idx vectors, reduction scratch
  constexpr int QV = G * D / 8;                           // 16-byte pieces of q_pre
  constexpr int WV = G * D * IDX / 8;                     // 16-byte pieces of the G matrices
  constexpr int QV_PAD = QV < 64 ? 64 : QV;
  constexpr int WPT = (WV + kScoreThreads - 1) / kScoreThreads;
  __shared__ uint4 s_qraw[QV_PAD];
  __shared__ uint4 s_w[WPT * kScoreThreads];
  __shared__ float s_qidx[G][IDX];
  __shared__ float s_red[kScoreThreads / 64][G];
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  typedef __attribute__((address_space(1))) const void* glb_ptr_t;
  const int wave = tid / 64, lane = tid % 64;

  // ---- every global load of the block is issued up front.  q_pre and W_q_idx go
  // straight to LDS (global_load_lds_dwordx4: no registers, lane i writes 16 bytes at
  // the wave's LDS base + 16*i); indices are clamped in range so every lane loads.
  if (wave * 64 < QV_PAD) {
    const int pidx = min(wave * 64 + lane, QV - 1);
    const uint16_t* src = q_pre + (int64_t(b) * Hq + g * G + pidx / (D / 8)) * D + (pidx % (D / 8)) * 8;
    __builtin_amdgcn_global_load_lds((glb_ptr_t)src, (lds_ptr_t)(s_qraw + wave * 64), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int pidx = min(i * kScoreThreads + tid, WV - 1);
    const int t = pidx / (D * IDX / 8), off = pidx % (D * IDX / 8);
    const uint16_t* src = w_q + int64_t(r * G + t) * w_stride + off * 8;
    __builtin_amdgcn_global_load_lds((glb_ptr_t)src, (lds_ptr_t)(s_w + i * kScoreThreads + wave * 64), 16, 0, 0);
  }
  // The wait below (vmcnt(NK)) relies on every direct-to-LDS copy being issued before the
  // NK key loads: this barrier keeps the compiler from moving any key load above it.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  // this tile's keys: thread tid takes tokens base + it*256 + tid (coalesced 2*IDX-byte rows)
  const int64_t base = int64_t(blk) * TILE;
  const uint16_t* kp = k_idx + int64_t(grp) * n_cap * IDX;
  uint32_t kw[ITEMS][KW];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    int64_t j = base + it * kScoreThreads + tid;
    j = j < n_ctx ? j : n_ctx - 1;
    if constexpr (IDX == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(kp + j * IDX);
      kw[it][0] = u.x;
      kw[it][1] = u.y;
    } else {
#pragma unroll
      for (int c = 0; c < IDX / 8; ++c) {
        const uint4 u = reinterpret_cast<const uint4*>(kp + j * IDX)[c];
        kw[it][4 * c] = u.x;
        kw[it][4 * c + 1] = u.y;
        kw[it][4 * c + 2] = u.z;
        kw[it][4 * c + 3] = u.w;
      }
    }
  }
  // wait for the LDS-direct loads only: vmcnt retires in issue order, so leaving the
  // NK key loads outstanding is vmcnt(NK)
  constexpr int NK = ITEMS * (IDX >= 8 ? IDX / 8 : 1);
  static_assert(NK < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((NK & 0xF) | ((NK >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  __builtin_amdgcn_s_barrier();   // a bare barrier: __syncthreads' fence would wait for the key loads too

  // ---- q_idx = q_pre . W_q_idx for the G heads of this group (fp32, not rounded)
  {
    constexpr int P = kScoreThreads / (G * IDX);         // threads per output
    static_assert(P >= 1 && P <= 64, "one wave reduces an output");
    const int o = tid / P, pi = tid % P;
    const int t = o / IDX, c = o % IDX;
    const uint16_t* w = reinterpret_cast<const uint16_t*>(s_w) + t * D * IDX;
    const uint16_t* qr = reinterpret_cast<const uint16_t*>(s_qraw) + t * D;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < D / P; ++i) {
      const int d = pi + i * P;
      acc = fmaf(bf16_to_f32(qr[d]), bf16_to_f32(w[d * IDX + c]), acc);
    }
#pragma unroll
    for (int off = P / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (pi == 0) s_qidx[t][c] = acc * idx_scale;
  }
  __syncthreads();
  // q_idx is the same for every lane: keep it in scalar registers (frees G*IDX VGPRs)
  float qi[G][IDX];
#pragma unroll
  for (int t = 0; t < G; ++t)
#pragma unroll
    for (int c = 0; c < IDX; ++c)
      qi[t][c] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_qidx[t][c])));

  // ---- score the tile (keys were loaded before the q_idx prologue)
  float sc[ITEMS][G];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int64_t j = base + it * kScoreThreads + tid;
    float kf[IDX];
#pragma unroll
    for (int e = 0; e < KW; ++e) {
      kf[2 * e] = bf16_lo(kw[it][e]);
      kf[2 * e + 1] = bf16_hi(kw[it][e]);
    }
#pragma unroll
    for (int t = 0; t < G; ++t) {
      float s = 0.0f;
#pragma unroll
      for (int c = 0; c < IDX; ++c) s = fmaf(qi[t][c], kf[c], s);
      sc[it][t] = (j < n_ctx) ? s : -INFINITY;
      if (j < n_ctx) scores[(int64_t(grp) * G + t) * n_cap + j] = s;
    }
  }

  // ---- per-block max and sum of exp for each of the G rows
  float mt[G];
#pragma unroll
  for (int t = 0; t < G; ++t) {
    float m = -INFINITY;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) m = fmaxf(m, sc[it][t]);
    m = wave_max(m);
    if (lane == 0) s_red[wave][t] = m;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < G; ++t) {
    float m = s_red[0][t];
#pragma unroll
    for (int w = 1; w < kScoreThreads / 64; ++w) m = fmaxf(m, s_red[w][t]);
    mt[t] = m;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < G; ++t) {
    float z = 0.0f;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) z += __expf(sc[it][t] - mt[t]);
    z = wave_sum(z);
    if (lane == 0) s_red[wave][t] = z;
  }
  __syncthreads();
  if (tid < G) {
    float z = 0.0f;
#pragma unroll
    for (int w = 0; w < kScoreThreads / 64; ++w) z += s_red[w][tid];
    part[(int64_t(grp) * G + tid) * nblk + blk] = make_float2(mt[tid], z);
  }
}

// One wave: combine the first nblk per-block partials of score row `row` (rows `stride`
// apart) into (row_max, row_sum).
__device__ __forceinline__ void score_finalize_row(const float2* __restrict__ part, int stride, int nblk,
                                                   float* __restrict__ row_max, float* __restrict__ row_sum,
                                                   int row) {
  const int lane = threadIdx.x & 63;
  const float2* p = part + int64_t(row) * stride;
  float m = -INFINITY;
  for (int i = lane; i < nblk; i += 64) m = fmaxf(m, p[i].x);
  m = wave_max(m);
  float z = 0.0f;
  for (int i = lane; i < nblk; i += 64) z += p[i].y * __expf(p[i].x - m);
  z = wave_sum(z);
  if (lane == 0) {
    row_max[row] = m;
    row_sum[row] = z;
  }
}

}  // namespace
