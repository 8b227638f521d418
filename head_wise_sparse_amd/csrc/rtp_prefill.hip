// rtp_prefill_attn: one causal prefill chunk of one sequence.
//
//  * retrieval heads: dense causal attention (research-map summary, "Limitations":
//    retrieval heads keep dense attention in prefill);
//  * local heads: causal attention over the sink tokens plus a sliding window
//    (summary, "Approach");
//  * the chunk's 16-dim indexer keys, bf16(k_pre . W_k_idx), for every retrieval KV
//    head (pre-RoPE projection, summary "Approach"; abstract, observation (2)).
//
// Attention kernel (flash-attention forward, bf16 in / fp32 accumulate, D = 128):
//  - a block owns 128 query rows of one head (4 waves x 32 rows) and walks 64-key
//    tiles of the cache: every key tile for retrieval heads up to the diagonal; only
//    the sink tile(s) and the window tiles for local heads (tiles outside the mask are
//    never loaded).  Blocks are ordered heaviest first (retrieval heads, last rows).
//  - S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K tile from LDS, Q^T held in registers
//    for the whole loop); the accumulator layout of S^T is exactly the B operand of
//    O^T = V^T P^T, so P never goes through LDS.
//  - V^T is staged in LDS: each thread loads 4 keys x 8 dims, transposes them in
//    registers and writes 8-byte runs; keys are stored in the order the P^T operand
//    holds them, so every MFMA operand read is one 16-byte ds_read.
//  - online softmax in the exp2 domain with a lazy reference max (rescale only when
//    a row max grows by more than 2^8); masks are applied only on boundary tiles.
//  - K/V tiles are double-buffered in LDS and the next tile's global loads are in
//    flight while the current tile is computed.
#include <cmath>

#include "rtp_internal.hpp"

using namespace rtp;
using namespace rtp_dev;

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int PD = 128;               // head dim
constexpr int BM = 128;               // query rows per block
constexpr int BN = 64;                // keys per tile
constexpr int KP = PD + 8;            // K tile row pitch (bf16 elements): 272 bytes
constexpr int VP = BN + 8;            // V^T tile row pitch (bf16 elements): 144 bytes
constexpr int kPreThreads = 256;

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
  int nmb;                  // row blocks per head
  int n_ret_q, n_loc_q;     // retrieval / local query heads
  HeadMap ret, loc;         // rank -> KV head
};

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

// position of key kl (multiple of 4, inside a 64-key tile) in the V^T tile row: within
// each 16-key group, keys 4h..4h+3 and 8+4h..8+4h+3 sit in slots 8h .. 8h+7
__device__ __forceinline__ int vt_pos(int kl) {
  const int q4 = (kl & 15) >> 2;
  return (kl & ~15) + 8 * (q4 & 1) + 4 * (q4 >> 1);
}

__global__ __launch_bounds__(kPreThreads, 2) void k_prefill_attn(PrefArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hf = lane >> 5;

  // ---- which head / row block (heaviest first)
  int idx = blockIdx.x;
  bool retr;
  int qh;                     // global query head
  int mb;
  if (idx < a.n_ret_q * a.nmb) {
    retr = true;
    const int i = idx % a.n_ret_q;
    mb = a.nmb - 1 - idx / a.n_ret_q;
    qh = a.ret.kv[i / a.G] * a.G + i % a.G;
  } else {
    idx -= a.n_ret_q * a.nmb;
    retr = false;
    const int i = idx % a.n_loc_q;
    mb = a.nmb - 1 - idx / a.n_loc_q;
    qh = a.loc.kv[i / a.G] * a.G + i % a.G;
  }
  const int kvh = qh / a.G;
  const int64_t R0 = a.c0 + int64_t(mb) * BM;                  // first row of the block
  const int64_t Rend = min<int64_t>(R0 + BM, a.c0 + a.C);      // one past the last valid row
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

  __shared__ uint16_t s_k[2][BN * KP];
  __shared__ uint16_t s_vt[2][PD * VP];

  const uint16_t* kbase = a.k + int64_t(kvh) * a.n_cap * PD;
  const uint16_t* vbase = a.v + int64_t(kvh) * a.n_cap * PD;

  // ---- Q^T operand: lane holds q row (wave*32 + l32), dims 16*ds + 8*hf .. +8
  const int64_t my_row = R0 + wave * 32 + l32;                 // absolute row of this lane's column
  const int64_t qrow_c = min<int64_t>(my_row - a.c0, a.C - 1); // chunk-relative, clamped
  bf16x8_t qop[PD / 16];
#pragma unroll
  for (int ds = 0; ds < PD / 16; ++ds)
    qop[ds] = as_bf16x8(*reinterpret_cast<const uint4*>(a.q + (qrow_c * a.Hq + qh) * PD + 16 * ds + 8 * hf));

  // ---- tile staging: global -> registers -> LDS
  uint4 kreg[4], vreg[4];
  auto load_tile = [&](int kt) {
    const int64_t k0 = int64_t(kt) * BN;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + kPreThreads * i;
      const int key = u >> 4, d8 = u & 15;
      const int64_t kr = min<int64_t>(k0 + key, a.n_cap - 1);
      kreg[i] = *reinterpret_cast<const uint4*>(kbase + kr * PD + d8 * 8);
    }
    const int kg = tid >> 4, d8 = tid & 15;                    // keys 4kg..4kg+3, dims 8*d8..+8
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kr = min<int64_t>(k0 + 4 * kg + j, a.n_cap - 1);
      vreg[j] = *reinterpret_cast<const uint4*>(vbase + kr * PD + d8 * 8);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + kPreThreads * i;
      const int key = u >> 4, d8 = u & 15;
      *reinterpret_cast<uint4*>(&s_k[buf][key * KP + d8 * 8]) = kreg[i];
    }
    const int kg = tid >> 4, d8 = tid & 15;
    const int pos = vt_pos(4 * kg);
    auto word = [&](int j, int e2) -> uint32_t {
      return e2 == 0 ? vreg[j].x : (e2 == 1 ? vreg[j].y : (e2 == 2 ? vreg[j].z : vreg[j].w));
    };
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {          // dims 8*d8 + 2*e2 (low halves) and +1 (high halves)
      const uint32_t w0 = word(0, e2), w1 = word(1, e2), w2 = word(2, e2), w3 = word(3, e2);
      uint2 lo, hi;
      lo.x = (w0 & 0xFFFFu) | (w1 << 16);
      lo.y = (w2 & 0xFFFFu) | (w3 << 16);
      hi.x = (w0 >> 16) | (w1 & 0xFFFF0000u);
      hi.y = (w2 >> 16) | (w3 & 0xFFFF0000u);
      *reinterpret_cast<uint2*>(&s_vt[buf][(d8 * 8 + 2 * e2) * VP + pos]) = lo;
      *reinterpret_cast<uint2*>(&s_vt[buf][(d8 * 8 + 2 * e2 + 1) * VP + pos]) = hi;
    }
  };

  f32x16 oacc[PD / 32];
#pragma unroll
  for (int db = 0; db < PD / 32; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[db][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  load_tile(tile_of(0));
  store_tile(0);
  __syncthreads();

  for (int n = 0; n < n_tiles; ++n) {
    const int buf = n & 1;
    const int kt = tile_of(n);
    const int64_t k0 = int64_t(kt) * BN;
    if (n + 1 < n_tiles) load_tile(tile_of(n + 1));

    // S^T = K Q^T : two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.0f;
#pragma unroll
      for (int ds = 0; ds < PD / 16; ++ds) {
        const uint4 kv = *reinterpret_cast<const uint4*>(&s_k[buf][(kb * 32 + l32) * KP + 16 * ds + 8 * hf]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qop[ds], sacc[kb], 0, 0, 0);
      }
    }

    // mask (boundary tiles only): key = k0 + kb*32 + 8*(v/4) + 4*hf + v%4, row = my_row
    bool full;
    if (retr) {
      full = (k0 + BN - 1 <= R0);
    } else {
      full = (k0 + BN - 1 <= R0) && (k0 >= Rl - a.window + 1 || k0 + BN - 1 < a.n_sinks);
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = sacc[kb][v] * a.scale_log2;
        if (!full) {
          const int64_t key = k0 + kb * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
          bool vis = key <= my_row;
          if (!retr) vis = vis && (key < a.n_sinks || key > my_row - a.window);
          x = vis ? x : -INFINITY;
        }
        sacc[kb][v] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));             // both halves hold the same row
    // lazy reference max: move it only when the row max grows past 2^8 of headroom
    const bool grow = tmax > m_run + 8.0f;
    if (__ballot(grow)) {
      const float m_new = grow ? tmax : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < PD / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
      m_run = m_new;
    }
    const bool live = m_run != -INFINITY;
    uint32_t pk[2][8];
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float p0 = live ? __builtin_amdgcn_exp2f(sacc[kb][v] - m_run) : 0.0f;
        const float p1 = live ? __builtin_amdgcn_exp2f(sacc[kb][v + 1] - m_run) : 0.0f;
        psum += p0 + p1;
        pk[kb][v >> 1] = pack_bf16x2(p0, p1);
      }
    l_run += psum;

    // O^T += V^T P^T : four 32-dim blocks x four 16-key steps
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = ks >> 1, half = ks & 1;
      const uint4 pb = make_uint4(pk[kb][4 * half], pk[kb][4 * half + 1], pk[kb][4 * half + 2], pk[kb][4 * half + 3]);
#pragma unroll
      for (int db = 0; db < PD / 32; ++db) {
        const uint4 vv = *reinterpret_cast<const uint4*>(&s_vt[buf][(db * 32 + l32) * VP + 16 * ks + 8 * hf]);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), as_bf16x8(pb), oacc[db], 0, 0, 0);
      }
    }

    if (n + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: lane holds row my_row, dims db*32 + 8*(v/4) + 4*hf + (v%4)
  const float lt = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (my_row < Rend) {
    uint16_t* op = a.out + ((my_row - a.c0) * a.Hq + qh) * PD;
#pragma unroll
    for (int db = 0; db < PD / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        uint2 w;
        w.x = pack_bf16x2(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv);
        w.y = pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + db * 32 + 8 * g4 + 4 * hf) = w;
      }
  }
}

// Indexer keys of the chunk: k_idx[r][c0 + t][:] = bf16(k_pre[t][g(r)][:] . W_k_idx[r]).
// One wave per 16 tokens on v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 dims of
// k_pre (one 16-byte load per lane and step), B = W^T staged in LDS.
__global__ __launch_bounds__(256) void k_kidx_proj(const uint16_t* __restrict__ k_pre,
                                                   const uint16_t* __restrict__ w_k, int64_t w_stride,
                                                   uint16_t* __restrict__ k_idx, int64_t c0, int C, int Hkv,
                                                   int64_t n_cap, HeadMap ret) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = blockIdx.y;
  const int g = ret.kv[r];
  __shared__ uint16_t s_wt[kIdxDim][PD + 8];                   // W^T: [out][d]
  for (int i = tid; i < PD * kIdxDim; i += 256) {
    const int d = i / kIdxDim, c = i % kIdxDim;
    s_wt[c][d] = w_k[int64_t(r) * w_stride + i];
  }
  __syncthreads();
  const int t0 = (blockIdx.x * 4 + wave) * 16;                 // first token of this wave
  const int row = lane & 15, kq = lane >> 4;
  const int tok = min(t0 + row, C - 1);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int st = 0; st < PD / 32; ++st) {
    const uint4 av = *reinterpret_cast<const uint4*>(k_pre + (int64_t(tok) * Hkv + g) * PD + 32 * st + 8 * kq);
    const uint4 bv = *reinterpret_cast<const uint4*>(&s_wt[row][32 * st + 8 * kq]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc, 0, 0, 0);
  }
  // D (16 x 16): lane holds output column (lane & 15), token rows 4*(lane>>4) + v
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = t0 + 4 * kq + v;
    if (t < C) k_idx[(int64_t(r) * n_cap + c0 + t) * kIdxDim + row] = f32_to_bf16(acc[v]);
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
  if (L.D != PD) return fail(RTP_EUNSUPPORTED, "rtp_prefill_attn: head_dim must be 128 (got %d)", L.D);
  if (!q || !k_cache || !v_cache || !out) return fail(RTP_EINVAL, "rtp_prefill_attn: NULL tensor pointer");
  if (L.n_ret > 0 && (!k_pre || !w_k_idx || !k_idx_cache))
    return fail(RTP_EINVAL, "rtp_prefill_attn: NULL indexer pointer");
  if (w_head_stride < 0) return fail(RTP_EINVAL, "w_head_stride must be >= 0");
  if (!std::isfinite(sm_scale)) return fail(RTP_EINVAL, "rtp_prefill_attn: sm_scale must be finite");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      (k_pre && !aligned(k_pre, 16)) || (k_idx_cache && !aligned(k_idx_cache, 2)))
    return fail(RTP_EINVAL, "rtp_prefill_attn: tensors must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (L.n_ret > 0) {
    hipLaunchKernelGGL(k_kidx_proj, dim3((C + 63) / 64, L.n_ret), dim3(256), 0, s, k_pre, w_k_idx, w_head_stride,
                       k_idx_cache, c0, C, L.Hkv, L.n_cap, ret_map(L));
    if ((st = check_launch("k_kidx_proj")) != RTP_OK) return st;
  }
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
  a.nmb = (C + BM - 1) / BM;
  a.n_ret_q = L.n_ret * L.G;
  a.n_loc_q = L.n_loc * L.G;
  a.ret = ret_map(L);
  a.loc = loc_map(L);
  hipLaunchKernelGGL(k_prefill_attn, dim3(a.nmb * L.Hq), dim3(kPreThreads), 0, s, a);
  return check_launch("k_prefill_attn");
}
