// rtp_prefill_attn: one causal prefill chunk of one sequence.
//
//  * retrieval heads: dense causal attention (research-map summary, "Limitations":
//    retrieval heads keep dense attention in prefill);
//  * local heads: causal attention over the sink tokens plus a sliding window
//    (summary, "Approach");
//  * the chunk's 16-dim indexer keys, bf16(k_pre . W_k_idx), for every retrieval KV
//    head (pre-RoPE projection, summary "Approach"; abstract, observation (2)).
//
// Attention kernel (flash-attention forward, bf16 in / fp32 accumulate, D = 64 or 128,
// one instantiation each):
//  - a block has 4 waves of 32 query rows: gcd(G, 4) query heads of one KV head (grouped-
//    query attention: they read the same keys) times 4 / gcd(G, 4) row slices, so one K/V
//    tile copied to LDS serves up to four heads.  It walks 64-key tiles of the cache:
//    every key tile for retrieval heads up to the diagonal; only the sink tile(s) and
//    the window tiles for local heads (tiles outside the mask are never loaded).  Blocks
//    are ordered heaviest first (retrieval heads, last rows).
//  - S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K tile from LDS, Q^T held in registers
//    for the whole loop); the accumulator layout of S^T is exactly the B operand of
//    O^T = V^T P^T, so P never goes through LDS.
//  - online softmax in the exp2 domain with a lazy reference max (rescale only when
//    a row max grows by more than 2^8); masks are applied only on boundary tiles.
//  - K/V tiles are double-buffered in LDS; the next tiles are copied HBM -> LDS directly
//    (no registers; one scalar base plus a fixed per-lane offset per copy) while the
//    current tile is computed, and V^T operands are read with the transposing LDS read
//    (ds_read_b64_tr_b16), so V needs no explicit transpose.
//  - per tile, the rare branches (boundary mask, reference-max move) come first; the rest
//    is 32 MFMA slots pinned in order by scheduling barriers: the next tile's QK^T, each
//    slot carrying one pair of this tile's exponentials, then this tile's PV product,
//    carrying the next tile's row max.  The loop runs two tiles per trip so that LDS
//    buffer indices are constants and the two S accumulator sets swap roles without
//    register copies.
//  - the indexer-key projection runs as the last blocks of the same grid (64 tokens x one
//    retrieval KV head each), so it fills the attention's tail instead of a launch.
#include <cmath>
#include <numeric>
#include <type_traits>

#include "rtp_internal.hpp"

using namespace rtp;
using namespace rtp_dev;

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int RB = 1;                 // 32-row column blocks per wave
constexpr int NW = 4;                 // waves per block (two blocks per CU)
constexpr int kOpAhead = 2;           // LDS operand reads in flight ahead of their MFMA
constexpr int WR = 32 * RB;           // query rows per wave
constexpr int BN = 64;                // keys per tile
// LDS tiles are 64 rows x PD bf16 (2*PD-byte rows of PD/8 chunks of 16 bytes), unpadded
// (direct-to-LDS loads fill 1 KB contiguous runs), with the chunk index XOR-swizzled per
// row, differently for K and V, so that the 16 (ds_read_b128) or 32 (ds_read_b64_tr_b16)
// lanes the LDS serves together touch 256 distinct bytes:
//  - K is read as MFMA A operands: 16 consecutive rows, one chunk each.  PD = 128
//    (256-byte rows): c ^ (r & 15) puts them in 16 different chunk slots; PD = 64
//    (128-byte rows, two per 256 bytes): c ^ ((r >> 1) & 7) gives the 8 rows of each parity
//    8 different slots.
//  - V is read with the transposing read: per wave, rows 4h .. 4h+3 (h = 0, 1) x 4 chunks.
//    PD = 128: c ^ 4*(r & 3) spreads each row's 4 chunks over a different quarter of the
//    row; PD = 64: c ^ 4*((r >> 1) & 1) puts rows 4h and 4h+2 (same half of 256 bytes) in
//    different halves of their rows.
template <int PD>
__device__ __forceinline__ int swz_xk(int r) { return PD == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int PD>
__device__ __forceinline__ int swz_xv(int r) { return PD == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
template <int PD>
__device__ __forceinline__ int swz_k(int r, int c) { return r * PD + ((c ^ swz_xk<PD>(r)) << 3); }
template <int PD>
__device__ __forceinline__ int swz_v(int r, int c) { return r * PD + ((c ^ swz_xv<PD>(r)) << 3); }

// 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane i writes at the
// wave-uniform LDS byte address `lds` + 16*i.  Issued from inline asm so that the
// compiler's wait insertion does not treat it as an LDS store that every later LDS read
// must wait for (the compiler cannot tell that the two double-buffer halves are
// disjoint).  The instruction has no destination register; completion is awaited
// explicitly (vmcnt) before the barrier that publishes the tile.
__device__ __forceinline__ void g2lds_16(const void* gaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(gaddr)
               : "memory", "m0");
}
// Same copy with a wave-uniform global base (scalar registers) and a 32-bit per-lane
// byte offset: no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void g2lds_16s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8)); }   // vmcnt(0)

constexpr int kPreThreads = 64 * NW;

struct PrefArgs {
  const uint16_t* q;        // [C][Hq][D]
  const uint16_t* k;        // [Hkv][n_cap][D]
  const uint16_t* v;
  uint16_t* out;            // [C][Hq][D]
  int64_t c0;
  int C;
  int Hq, G;
  int64_t n_cap;
  int n_sinks, window;
  float scale_log2;
  int gb;                   // query heads per block (of one KV head): gcd(G, NW)
  int ngrp;                 // G / gb head groups per KV head
  int rows;                 // query rows per block: WR * NW / gb
  int nmb;                  // row blocks per chunk
  int n_ret, n_loc;         // retrieval / local KV heads
  HeadMap ret, loc;         // rank -> KV head
  int n_attn;               // attention blocks; the blocks after them project indexer keys
  int n_px;                 // projection blocks per retrieval KV head (64 tokens each)
  int Hkv, idx;             // KV heads, indexer dim
  const uint16_t* k_pre;    // [C][Hkv][D] pre-RoPE keys of the chunk
  const uint16_t* w_k;      // [Hkv_r][D][idx] (head stride w_stride)
  int64_t w_stride;
  uint16_t* k_idx;          // [Hkv_r][n_cap][idx]
};

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }


// Indexer keys of the chunk: k_idx[r][c0 + t][:] = bf16(k_pre[t][g(r)][:] . W_k_idx[r]).
// One wave per 16 tokens on v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 dims of
// k_pre (one 16-byte load per lane and step), B = W^T staged in LDS, one 16-column
// block per 16 indexer outputs (dims 4 and 8 use one block, zero-padded).
// These blocks run as the last blocks of the attention grid (block x of 64 tokens, retrieval
// rank r), in the attention's tail; `lds` is the block's K tile buffer, free in such blocks.
template <int IDX, int PD>
__device__ __forceinline__ void kidx_proj_block(const PrefArgs& a, int bx, int r, uint16_t* lds) {
  constexpr int NCB = IDX > 16 ? IDX / 16 : 1;                  // 16-column output blocks
  const uint16_t* __restrict__ k_pre = a.k_pre;
  const uint16_t* __restrict__ w_k = a.w_k;
  uint16_t* __restrict__ k_idx = a.k_idx;
  const int C = a.C, Hkv = a.Hkv;
  const int64_t c0 = a.c0, n_cap = a.n_cap, w_stride = a.w_stride;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = a.ret.kv[r];
  typedef uint16_t wrow_t[PD + 8];
  wrow_t* s_wt = reinterpret_cast<wrow_t*>(lds);                // W^T: [out][d], 16 * NCB rows
  for (int i = tid; i < PD * 16 * NCB; i += 256) {
    const int d = i / (16 * NCB), c = i % (16 * NCB);
    s_wt[c][d] = c < IDX ? w_k[int64_t(r) * w_stride + d * IDX + c] : uint16_t(0);
  }
  __syncthreads();
  const int t0 = (bx * 4 + wave) * 16;                         // first token of this wave
  const int row = lane & 15, kq = lane >> 4;
  const int tok = min(t0 + row, C - 1);
  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int st = 0; st < PD / 32; ++st) {
    const uint4 av = *reinterpret_cast<const uint4*>(k_pre + (int64_t(tok) * Hkv + g) * PD + 32 * st + 8 * kq);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const uint4 bv = *reinterpret_cast<const uint4*>(&s_wt[cb * 16 + row][32 * st + 8 * kq]);
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc[cb], 0, 0, 0);
    }
  }
  // D (16 x 16): lane holds output column (lane & 15), token rows 4*(lane>>4) + v
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + 4 * kq + v, col = cb * 16 + row;
      if (t < C && col < IDX) k_idx[(int64_t(r) * n_cap + c0 + t) * IDX + col] = f32_to_bf16(acc[cb][v]);
    }
}



typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) const void* glb_ptr_t;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t* lds_s4;

template <int PD>
__global__ __launch_bounds__(kPreThreads, 2) void k_prefill_attn(PrefArgs a) {
  static_assert(PD == 64 || PD == 128, "head dims");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hf = lane >> 5;
  __shared__ uint16_t s_k[2][BN * PD];
  __shared__ uint16_t s_v[2][BN * PD];

  if (blockIdx.x >= a.n_attn) {               // indexer-key projection block
    const int pb = blockIdx.x - a.n_attn, bx = pb % a.n_px, r = pb / a.n_px;
    switch (a.idx) {
      case 4: kidx_proj_block<4, PD>(a, bx, r, s_k[0]); break;
      case 8: kidx_proj_block<8, PD>(a, bx, r, s_k[0]); break;
      case 16: kidx_proj_block<16, PD>(a, bx, r, s_k[0]); break;
      default: kidx_proj_block<32, PD>(a, bx, r, s_k[0]); break;
    }
    return;
  }

  // ---- which KV head / head group / row block (heaviest first).  The block's waves are
  // gb query heads of one KV head x NW/gb row slices, so every K/V tile copied to LDS
  // serves gb heads.
  int idx = blockIdx.x;
  bool retr;
  int kvh, grp, mb;
  if (idx < a.n_ret * a.ngrp * a.nmb) {
    retr = true;
    const int per = a.n_ret * a.ngrp, i = idx % per;
    mb = a.nmb - 1 - idx / per;
    kvh = a.ret.kv[i / a.ngrp];
    grp = i % a.ngrp;
  } else {
    idx -= a.n_ret * a.ngrp * a.nmb;
    retr = false;
    const int per = a.n_loc * a.ngrp, i = idx % per;
    mb = a.nmb - 1 - idx / per;
    kvh = a.loc.kv[i / a.ngrp];
    grp = i % a.ngrp;
  }
  const int qh = kvh * a.G + grp * a.gb + wave % a.gb;         // this wave's query head
  const int rslice = wave / a.gb;                              // this wave's row slice
  const int64_t R0 = a.c0 + int64_t(mb) * a.rows;              // first row of the block
  const int64_t Rend = min<int64_t>(R0 + a.rows, a.c0 + a.C);  // one past the last valid row
  const int64_t Rl = Rend - 1;                                 // last valid row

  // ---- key tiles this block visits
  const int kt_last = int(Rl / BN);
  int n_sink_t = 0, kt_start = 0;
  if (!retr) {
    const int64_t wlo = max<int64_t>(0, R0 - a.window + 1);    // first window key of the first row
    kt_start = int(wlo / BN);
    const int st_end = (a.n_sinks + BN - 1) / BN;              // tiles holding sinks
    n_sink_t = min(st_end, kt_start);                          // those before the window tiles
  }
  const int n_tiles = n_sink_t + (kt_last - kt_start + 1);
  auto tile_of = [&](int n) { return n < n_sink_t ? n : kt_start + (n - n_sink_t); };

  const uint16_t* kbase = a.k + int64_t(kvh) * a.n_cap * PD;
  const uint16_t* vbase = a.v + int64_t(kvh) * a.n_cap * PD;

  // ---- Q^T operands: a wave owns 32 rows; lane holds row R0 + wave*32 + l32, dims
  // 16*ds + 8*hf .. +8 (all 128 dims of the row over the two wave halves)
  int64_t my_row[RB];
  bf16x8_t qop[RB][PD / 16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    my_row[rb] = R0 + rslice * WR + rb * 32 + l32;
    const int64_t qrow_c = min<int64_t>(my_row[rb] - a.c0, a.C - 1);   // chunk-relative, clamped
#pragma unroll
    for (int ds = 0; ds < PD / 16; ++ds)
      qop[rb][ds] = as_bf16x8(*reinterpret_cast<const uint4*>(a.q + (qrow_c * a.Hq + qh) * PD + 16 * ds + 8 * hf));
  }

  // ---- tile staging: the next tiles' K and V rows go from HBM straight to the other LDS
  // buffer while the current tile is computed.
  constexpr int KCH = BN * PD / 8;                            // 16-byte chunks per tile
  constexpr int KLD = KCH / kPreThreads;                      // copies per thread per tile (K and V each)
  constexpr int NWV = kPreThreads / 64;
  // V^T operand addresses.  ds_read_b64_tr_b16: within each 16-lane group, lane r names a
  // row of 4 bf16 and lane 4j+i receives element i of the rows named by lanes j, j+4, j+8,
  // j+12.  Lane r names V[key0 + r/4][d0 + 4*(r%4)], so lane l receives dims d0 + l%16 of
  // keys key0 .. key0+3: a slice of the V^T operand.  For the (32-dim block db, 16-key step
  // ks) operand, lane l's 8 elements are the keys 16*ks + 8*(e/4) + 4*(l/32) + e%4 (the key
  // order of the P^T operand); read t covers e = 4t .. 4t+3.
  const int tr_r = lane & 15, tr_dsub = (lane >> 4) & 1;
  auto vt_operand = [&](int buf, int db, int ks) -> bf16x8_t {
    short4_t h0, h1;
    const int d = 32 * db + 16 * tr_dsub + 4 * (tr_r & 3);
    const int key0 = 16 * ks + 4 * hf + (tr_r >> 2);
    h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(&s_v[buf][swz_v<PD>(key0, d >> 3) + (d & 7)]));
    h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(&s_v[buf][swz_v<PD>(key0 + 8, d >> 3) + (d & 7)]));
    short8_t r8;
    r8[0] = h0[0]; r8[1] = h0[1]; r8[2] = h0[2]; r8[3] = h0[3];
    r8[4] = h1[0]; r8[5] = h1[1]; r8[6] = h1[2]; r8[7] = h1[3];
    return __builtin_bit_cast(bf16x8_t, r8);
  };

  f32x16 oacc[RB][PD / 32];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < PD / 32; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[rb][db][v] = 0.0f;
  // Running reference max (log2 domain) starts finite: a row that has seen no visible
  // key yet gets exp2(-inf - m) = 0 everywhere and its first real max rescales by 0.
  constexpr float kNoMax = -1.0e30f;
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = kNoMax;
    l_run[rb] = 0.0f;
  }

  // S^T = K Q^T of one key tile; each K operand read from LDS serves every row block
  auto qk = [&](auto bufc, f32x16 (&sa)[RB][2]) {
    constexpr int buf = decltype(bufc)::value;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) sa[rb][kb][v] = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < PD / 16; ++ds) {
        const uint4 kv = *reinterpret_cast<const uint4*>(&s_k[buf][swz_k<PD>(kb * 32 + l32, 2 * ds + hf)]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sa[rb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qop[rb][ds], sa[rb][kb], 0, 0, 0);
      }
  };

  // Tile copies.  Wave w's i-th copy fills physical chunks (NW*i + w)*64 .. +63 of the
  // tile, i.e. the RPC rows RPC*NW*i + crow (crow = RPC*w + lane/CPR, RPC = 1 KB / row
  // bytes, CPR chunks per row); the swizzled chunk a lane fetches does not depend on i, so
  // a copy is one scalar base (the tile's first row, + NW KB per i) plus a fixed per-lane
  // byte offset.  Only a tile that runs past the chunk's last row (rows from c0 + C on
  // need not hold valid data yet) takes the clamped path: its rows from there on repeat
  // the last valid row, so they are finite; their scores are masked and their
  // probabilities are exactly 0.
  constexpr int CPR = PD / 8;                                 // 16-byte chunks per row
  constexpr int RPC = 64 / CPR;                               // rows per 1 KB wave copy
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int crow = RPC * wave + lane / CPR;
  const int cslot = lane % CPR;
  // the XOR terms depend only on crow: RPC*NW*i is a multiple of 16 (PD = 128) or 32 (PD = 64)
  const uint32_t koff = uint32_t(crow * PD + ((cslot ^ swz_xk<PD>(crow)) << 3)) * 2u;
  const uint32_t voff = uint32_t(crow * PD + ((cslot ^ swz_xv<PD>(crow)) << 3)) * 2u;
  static_assert(KLD * NWV * 64 == KCH && NWV == NW, "copy layout");
  const int64_t kv_end = a.c0 + a.C;          // cache rows below this are valid (<= n_cap)
  auto copy_tile = [&](const uint16_t* base, int kt, uint32_t off, uint16_t* lds_tile, bool is_k) {
    const int64_t k0 = int64_t(kt) * BN;
    const uint32_t lds0 = lds_addr(lds_tile) + uint32_t(wave_u) * 1024u;
    if (k0 + BN <= kv_end) {
      const char* g0 = reinterpret_cast<const char*>(base + k0 * PD);
#pragma unroll
      for (int i = 0; i < KLD; ++i) g2lds_16s(g0 + 1024 * NW * i, off, lds0 + 1024u * NW * i);
    } else {
#pragma unroll
      for (int i = 0; i < KLD; ++i) {
        const int row = RPC * NW * i + crow;
        const int c = is_k ? (cslot ^ swz_xk<PD>(crow)) : (cslot ^ swz_xv<PD>(crow));
        const int64_t kr = min<int64_t>(k0 + row, kv_end - 1);
        g2lds_16(base + kr * PD + c * 8, lds0 + 1024u * NW * i);
      }
    }
  };

  // row max of a tile's raw scores, both wave halves (the two halves hold the same rows,
  // different keys: one lane swap), in the log2 domain (the scale is positive)
  auto row_max = [&](const f32x16 (&sc)[RB][2], int rb) -> float {
    float t = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) t = fmaxf(t, sc[rb][kb][v]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
  };
  float tmax_carry[RB];          // row max of the S tile the next step starts from (unmasked)

  // one pipeline step: S(n) is in `cur`; copies K(n+2) -> buffer B and V(n+1) -> buffer
  // 1-B, then (when there is a next tile) computes S(n+1) = K(n+1) Q^T into `nxt` on the
  // MFMA pipe while the softmax of S(n) runs on the VALU, then O^T += V(n)^T P(n)^T from
  // buffer B.  The rare branches (boundary-tile mask, reference-max move) come first so
  // that the MFMA and VALU work of the step is one straight-line block the compiler can
  // interleave.
  auto step = [&](auto bc, auto has_next_c, int n, f32x16 (&cur)[RB][2], f32x16 (&nxt)[RB][2]) {
    constexpr int B = decltype(bc)::value;
    constexpr bool HAS_NEXT = decltype(has_next_c)::value;
    const int kt = tile_of(n);
    const int k0 = kt * BN;
    if (n + 2 < n_tiles) copy_tile(kbase, tile_of(n + 2), koff, s_k[B], true);
    if (HAS_NEXT) copy_tile(vbase, tile_of(n + 1), voff, s_v[1 - B], false);

    // masks apply only where some (row, key) pair of the tile is invisible
    bool full;
    if (retr) {
      full = (int64_t(k0) + BN - 1 <= R0);
    } else {
      full = (int64_t(k0) + BN - 1 <= R0) && (int64_t(k0) >= Rl - a.window + 1 || k0 + BN - 1 < a.n_sinks);
    }
    if (!full) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int rrel = int(my_row[rb] - k0);            // row relative to the tile's first key
        const int sink_lim = a.n_sinks - k0;              // keys below this index are sinks
        const int wlo = rrel - a.window;                  // window keys are > wlo
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kr = kb * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
            const bool vis = (kr <= rrel) & (retr | (kr < sink_lim) | (kr > wlo));   // no short-circuit branches
            cur[rb][kb][v] = vis ? cur[rb][kb][v] : -INFINITY;
          }
        tmax_carry[rb] = row_max(cur, rb);              // the carried max did not see the mask
      }
    }
    // row max on the raw scores (the scale is positive); the two wave halves hold the same
    // rows (different keys) and exchange their maxima with one lane swap.  The reference
    // max (log2 domain) moves only when a row max grows past it by more than 2^8.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float tmax = tmax_carry[rb];
      const bool grow = tmax > m_run[rb] + 8.0f;
      if (__ballot(grow)) {
        const float m_new = grow ? tmax : m_run[rb];
        const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < PD / 32; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[rb][db][v] *= alpha;
        m_run[rb] = m_new;
      }
    }

    // ---- straight-line part: QK of the next tile, softmax and PV of this one
    if constexpr (HAS_NEXT) {
      // 2*NQK MFMA slots (32 at PD = 128, 16 at PD = 64), pinned in this order by scheduling
      // barriers: QK^T(n+1) in slots 0..NQK-1 (alternating the two 32-key chains), each
      // carrying 16/NQK pairs of this tile's exponentials; PV(n) in the next NQK slots,
      // which also carry the next tile's row max (its chains finished by then).  K and V^T
      // operands are read kOpAhead slots ahead; left to itself the compiler reads each
      // operand one MFMA before its use.
      static_assert(RB == 1, "slot schedule assumes one row block per wave");
      constexpr int KB1 = 1 - B;
      constexpr int NQK = PD / 8;                 // QK^T MFMAs per tile: 2 chains x PD/16
      constexpr int NDB = PD / 32;                // 32-dim output blocks
      constexpr int NPV = 4 * NDB;                // PV MFMAs per tile: 4 key steps x NDB
      constexpr int EPS = 16 / NQK;               // exponential pairs per QK slot
      constexpr int T0 = PD == 128 ? 2 : 1;       // first PV slot folding chain 0 into the row max
      constexpr int T1 = NPV / 2;                 // first PV slot folding chain 1
      constexpr int VPP = 16 / (NPV - T1);        // values folded per slot
      static_assert(NPV == NQK && EPS * NQK == 16 && VPP * (NPV - T1) == 16, "slot schedule");
      bf16x8_t kop[NQK], vop[NPV];
      uint32_t pk[2][8];
      float psum = 0.0f;
      const float nm = -m_run[0];
      auto kread = [&](int s) {
        const int kbp = s & 1, ds = s >> 1;
        kop[s] = as_bf16x8(*reinterpret_cast<const uint4*>(&s_k[KB1][swz_k<PD>(kbp * 32 + l32, 2 * ds + hf)]));
      };
      auto vread = [&](int p) { vop[p] = vt_operand(B, p % NDB, p / NDB); };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) nxt[0][kb][v] = 0.0f;
#pragma unroll
      for (int s = 0; s < kOpAhead; ++s) kread(s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < NQK; ++s) {
        nxt[0][s & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[s], qop[0][s >> 1], nxt[0][s & 1], 0, 0, 0);
        if (s + kOpAhead < NQK) kread(s + kOpAhead);
        if (s >= NQK - kOpAhead) vread(s - (NQK - kOpAhead));
#pragma unroll
        for (int j = 0; j < EPS; ++j) {
          const int e = s * EPS + j, kb = e >> 3, v = 2 * (e & 7);
          const float p0 = __builtin_amdgcn_exp2f(fmaf(cur[0][kb][v], a.scale_log2, nm));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(cur[0][kb][v + 1], a.scale_log2, nm));
          pk[kb][e & 7] = pack_bf16x2(p0, p1);
          psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[kb][e & 7]),
                                                 __builtin_bit_cast(bf16x2_t, 0x3F803F80u), psum, false);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // PV slots; the next tile's row max rides along (its S chains finished in the last
      // two QK slots)
      float tm0 = -INFINITY, tm1 = -INFINITY;
#pragma unroll
      for (int p = 0; p < NPV; ++p) {
        const int ks = p / NDB, db = p % NDB, kb = ks >> 1, half = ks & 1;
        if (p + kOpAhead < NPV) vread(p + kOpAhead);
        const uint4 pb = make_uint4(pk[kb][4 * half], pk[kb][4 * half + 1], pk[kb][4 * half + 2], pk[kb][4 * half + 3]);
        oacc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[p], as_bf16x8(pb), oacc[0][db], 0, 0, 0);
        if (p >= T0 && p < T0 + 16 / VPP) {
#pragma unroll
          for (int j = 0; j < VPP; j += 2)
            tm0 = fmaxf(fmaxf(tm0, nxt[0][0][VPP * (p - T0) + j]), nxt[0][0][VPP * (p - T0) + j + 1]);
          asm volatile("" : "+v"(tm0));          // keep this partial max in its slot
        }
        if (p >= T1) {
#pragma unroll
          for (int j = 0; j < VPP; j += 2)
            tm1 = fmaxf(fmaxf(tm1, nxt[0][1][VPP * (p - T1) + j]), nxt[0][1][VPP * (p - T1) + j + 1]);
          asm volatile("" : "+v"(tm1));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      {
        const float t = fmaxf(tm0, tm1);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
        tmax_carry[0] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
      }
      l_run[0] += psum;
    } else {
    if constexpr (HAS_NEXT) qk(std::integral_constant<int, 1 - B>{}, nxt);
    if constexpr (HAS_NEXT) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) tmax_carry[rb] = row_max(nxt, rb);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t pk[RB][8];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float nm = -m_run[rb];
        float psum = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(cur[rb][kb][v], a.scale_log2, nm));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(cur[rb][kb][v + 1], a.scale_log2, nm));
          pk[rb][v >> 1] = pack_bf16x2(p0, p1);
          // row sum of the bf16 probabilities the PV product uses (one dot2 per pair)
          psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[rb][v >> 1]),
                                                 __builtin_bit_cast(bf16x2_t, 0x3F803F80u), psum, false);
        }
        l_run[rb] += psum;
      }
      // O^T += V^T P^T over this 32-key half: each V^T operand read serves every row block
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ks = 2 * kb + half;
#pragma unroll
        for (int db = 0; db < PD / 32; ++db) {
          const bf16x8_t vv = vt_operand(B, db, ks);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const uint4 pb = make_uint4(pk[rb][4 * half], pk[rb][4 * half + 1], pk[rb][4 * half + 2], pk[rb][4 * half + 3]);
            oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, as_bf16x8(pb), oacc[rb][db], 0, 0, 0);
          }
        }
      }
    }
    }
    wait_vm0();                 // this wave's copies of K(n+2) and V(n+1) have landed
    __syncthreads();            // ... and everyone's; K(n+1) and V(n) buffers are free again
  };

  f32x16 sacc[RB][2], snext[RB][2];
  copy_tile(kbase, tile_of(0), koff, s_k[0], true);
  copy_tile(vbase, tile_of(0), voff, s_v[0], false);
  if (n_tiles > 1) copy_tile(kbase, tile_of(1), koff, s_k[1], true);
  wait_vm0();
  __syncthreads();
  qk(std::integral_constant<int, 0>{}, sacc);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) tmax_carry[rb] = row_max(sacc, rb);
  __syncthreads();              // K(0) is consumed: its buffer takes K(2)

  // two steps per trip so that the buffer index is a constant and S alternates between
  // the two accumulator sets without copies; the last step (no next tile) is peeled
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  int n = 0;
  for (; n + 2 < n_tiles; n += 2) {
    step(I0{}, T{}, n, sacc, snext);
    step(I1{}, T{}, n + 1, snext, sacc);
  }
  if (n + 1 < n_tiles) {
    step(I0{}, T{}, n, sacc, snext);
    step(I1{}, F{}, n + 1, snext, sacc);
  } else {
    step(I0{}, F{}, n, sacc, snext);
  }

  // ---- normalise and store: lane holds row my_row[rb], dims db*32 + 8*(v/4) + 4*hf + (v%4)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float lt = l_run[rb] + __shfl_xor(l_run[rb], 32, 64);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (my_row[rb] < Rend) {
      uint16_t* op = a.out + ((my_row[rb] - a.c0) * a.Hq + qh) * PD;
#pragma unroll
      for (int db = 0; db < PD / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint2 w;
          w.x = pack_bf16x2(oacc[rb][db][4 * g4] * inv, oacc[rb][db][4 * g4 + 1] * inv);
          w.y = pack_bf16x2(oacc[rb][db][4 * g4 + 2] * inv, oacc[rb][db][4 * g4 + 3] * inv);
          *reinterpret_cast<uint2*>(op + db * 32 + 8 * g4 + 4 * hf) = w;
        }
    }
  }
}

}  // namespace

namespace rtp {
size_t prefill_ws_bytes(const Layer& L, int64_t C) {
  (void)L;
  (void)C;
  return 256;   // the prefill kernels use no scratch memory
}
}  // namespace rtp

extern "C" rtp_status rtp_prefill_attn(const rtp_layer_desc* desc, int64_t c0, int32_t C, const uint16_t* q,
                                       const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_pre,
                                       const uint16_t* w_k_idx, int64_t w_head_stride, uint16_t* k_idx_cache,
                                       float sm_scale, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  TraceRange trace_("rtp_prefill_attn");
  (void)ws;
  (void)ws_bytes;
  Layer L;
  rtp_status st = check_desc(desc, &L);
  if (st != RTP_OK) return st;
  if (L.B != 1) return fail(RTP_EINVAL, "rtp_prefill_attn: batch must be 1 (got %d)", L.B);
  if (C < 1) return fail(RTP_EINVAL, "rtp_prefill_attn: C must be >= 1 (got %d)", C);
  if (c0 < 0 || c0 + C > L.n_cap)
    return fail(RTP_EINVAL, "rtp_prefill_attn: need 0 <= c0 and c0 + C <= n_cap (c0=%lld, C=%d, n_cap=%lld)",
                (long long)c0, C, (long long)L.n_cap);

  if (L.kv_layout != RTP_KV_FULL)
    return fail(RTP_EUNSUPPORTED, "rtp_prefill_attn: the chunk needs the full cache layout (RTP_KV_FULL)");
  if (!q || !k_cache || !v_cache || !out) return fail(RTP_EINVAL, "rtp_prefill_attn: NULL tensor pointer");
  if (L.n_ret > 0 && (!k_pre || !w_k_idx || !k_idx_cache))
    return fail(RTP_EINVAL, "rtp_prefill_attn: NULL indexer pointer");
  if (w_head_stride < 0) return fail(RTP_EINVAL, "w_head_stride must be >= 0");
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return fail(RTP_EINVAL, "rtp_prefill_attn: sm_scale must be finite and > 0");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      (k_pre && !aligned(k_pre, 16)) || (k_idx_cache && !aligned(k_idx_cache, 2)))
    return fail(RTP_EINVAL, "rtp_prefill_attn: tensors must be 16-byte aligned");
  if ((st = enqueue_gate("rtp_prefill_attn")) != RTP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PrefArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.c0 = c0;
  a.C = C;
  a.Hq = L.Hq;
  a.G = L.G;
  a.n_cap = L.n_cap;
  a.n_sinks = L.n_sinks;
  a.window = L.window;
  a.scale_log2 = sm_scale * kLog2e;
  a.gb = std::gcd(L.G, NW);
  a.ngrp = L.G / a.gb;
  a.rows = WR * NW / a.gb;
  a.nmb = (C + a.rows - 1) / a.rows;
  a.n_ret = L.n_ret;
  a.n_loc = L.n_loc;
  a.ret = ret_map(L);
  a.loc = loc_map(L);
  a.n_attn = a.nmb * L.Hkv * a.ngrp;
  a.n_px = (C + 63) / 64;
  a.Hkv = L.Hkv;
  a.idx = L.idx;
  a.k_pre = k_pre;
  a.w_k = w_k_idx;
  a.w_stride = w_head_stride;
  a.k_idx = k_idx_cache;
  const int n_proj = L.n_ret > 0 ? a.n_px * L.n_ret : 0;
  if (L.D == 128)
    hipLaunchKernelGGL(k_prefill_attn<128>, dim3(a.n_attn + n_proj), dim3(kPreThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_prefill_attn<64>, dim3(a.n_attn + n_proj), dim3(kPreThreads), 0, s, a);
  return check_launch("k_prefill_attn");
}
