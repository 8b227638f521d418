"""Seeded synthetic inputs for head-wise sparse attention (decode and chunked prefill).

This module only *draws inputs*.  It holds none of the method's arithmetic
(no indexer scoring, no top-p rule, no masking, no attention): the oracle under
``oracle/`` and the HIP library both consume the arrays produced here, and
neither imports the other.

Why synthetic: the pages evaluate on LongBench, RULER and reasoning tasks with
trained Qwen3 weights (research-map summary page, sections "Key results" and
"Experimental setup"); neither the data nor the weights exist here.  The
workloads below keep the attention shapes of a Qwen3-8B-like layer (32 query
heads, 8 KV heads, head dim 128), the context lengths of the pages' speed points
(32K and 1M, section "Key results"), and planted "needle" indexer keys so that the
indexer's softmax mass is peaked the way retrieval heads are (abstract,
observation (2)).

Conventions (all arrays are numpy; bf16 tensors are carried as ``uint16`` raw
bits, so they can be handed to torch with ``.view(torch.bfloat16)``):

* Every tensor comes from its own substream
  ``default_rng(SeedSequence([BASE_SEED, config_id, tensor_id, a, b]))``; the
  oracle side and the GPU side regenerate bit-identical inputs.
* Draws are float32, then rounded to bf16 round-to-nearest-even.
* RoPE ("rotate half", inverse frequency ``1e6 ** (-2i/D)``, position = token
  index) is applied here, by the harness, before anything crosses the library
  boundary: the cache holds post-RoPE keys; the indexer sees pre-RoPE q and the
  pre-RoPE key projection (``k_idx``).
* Decode: the cache holds ``N`` tokens; the query sits at position ``N-1``.
* Needles: a needle token's indexer key is ``4 x mean(q_idx)`` over the query
  heads of its GQA group (for a group of one head this is exactly 4x the query
  indexer vector), where ``q_idx = q_pre . W_q_idx`` is computed here in fp64
  for input construction only.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

BASE_SEED = 0
ROPE_BASE = 1.0e6
IDX_DIM = 16

# tensor ids for the seed substreams
T_Q, T_K, T_V, T_WQ, T_WK, T_NEEDLE, T_QSCALE = 1, 2, 3, 4, 5, 6, 7


# ----------------------------------------------------------------------------- bf16 helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cid: int, tid: int, a: int = 0, b: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([BASE_SEED, cid, tid, a, b]))


_ROPE_CACHE: Dict[Tuple[int, int, int], Tuple[np.ndarray, np.ndarray]] = {}


def _rope_tables(positions: np.ndarray, d: int) -> Tuple[np.ndarray, np.ndarray]:
    """float32 cos/sin tables [n][D/2] (angles computed in float64)."""
    contiguous = positions.size > 1 and positions[-1] - positions[0] == positions.size - 1 \
        and np.all(np.diff(positions) == 1)
    key = (int(positions[0]), int(positions.size), d) if contiguous else None
    if key is not None and key in _ROPE_CACHE:
        return _ROPE_CACHE[key]
    half = d // 2
    inv_freq = ROPE_BASE ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = positions.astype(np.float64)[:, None] * inv_freq[None, :]
    tab = (np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32))
    if key is not None:
        if len(_ROPE_CACHE) > 4:
            _ROPE_CACHE.clear()
        _ROPE_CACHE[key] = tab
    return tab


def _rope_bf16(x_bits: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE (float32 arithmetic) on bf16 rows [n][D] at the given positions -> bf16 bits."""
    x = bf16_bits_to_f32(x_bits)
    d = x.shape[-1]
    half = d // 2
    cos, sin = _rope_tables(np.asarray(positions), d)
    x1, x2 = x[..., :half], x[..., half:]
    y = np.empty_like(x)
    y[..., :half] = x1 * cos - x2 * sin
    y[..., half:] = x2 * cos + x1 * sin
    return f32_to_bf16_bits(y)


def _normal_bf16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return f32_to_bf16_bits(x)


# ----------------------------------------------------------------------------- configurations
@dataclass(frozen=True)
class DecodeConfig:
    """One decode step of one attention layer."""
    cid: int
    name: str
    batch: int
    n_ctx: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    retrieval_kv: Tuple[int, ...]
    top_p: float
    n_sinks: int
    window: int
    n_needles: int
    lognormal_qscale: bool
    idx_dim: int = IDX_DIM      # indexer dimension (16 on the pages' design; 4 / 8 / 32 for the ablation)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def kv_role(self) -> np.ndarray:
        r = np.zeros(self.n_kv_heads, np.uint8)
        r[list(self.retrieval_kv)] = 1
        return r

    @property
    def n_kv_r(self) -> int:
        return len(self.retrieval_kv)


@dataclass(frozen=True)
class PrefillConfig:
    """Causal chunked prefill of one sequence through one attention layer."""
    cid: int
    name: str
    seq_len: int
    chunk: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    retrieval_kv: Tuple[int, ...]
    n_sinks: int
    window: int
    rows_per_head: int          # query rows per head the oracle checks
    idx_dim: int = IDX_DIM

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def kv_role(self) -> np.ndarray:
        r = np.zeros(self.n_kv_heads, np.uint8)
        r[list(self.retrieval_kv)] = 1
        return r

    @property
    def n_kv_r(self) -> int:
        return len(self.retrieval_kv)

    @property
    def n_chunks(self) -> int:
        return (self.seq_len + self.chunk - 1) // self.chunk


K32, K128, M1 = 32768, 131072, 1048576

CONFIGS: Dict[str, object] = {
    # tiny decode step: 4 q heads, 2 KV heads, d64; KV0 retrieval p=0.9, KV1 local S4 W256
    "decode_tiny_2k": DecodeConfig(0, "decode_tiny_2k", 1, 2048, 4, 2, 64, (0,), 0.9, 4, 256, 8, False),
    # Qwen3-8B-like layer, batch 8, 32K context
    "decode_b8_32k": DecodeConfig(1, "decode_b8_32k", 8, K32, 32, 8, 128, (0, 3), 0.95, 4, 2048, 64, True),
    # batch 4, 128K context (p swept over 0.9 / 0.95 / 0.99 by the caller)
    "decode_b4_128k": DecodeConfig(2, "decode_b4_128k", 4, K128, 32, 8, 128, (0, 3), 0.95, 4, 4096, 256, True),
    # 32K-token causal prefill in 4K chunks
    "prefill_32k": PrefillConfig(3, "prefill_32k", K32, 4096, 32, 8, 128, (0, 3), 4, 4096, 64),
    # 1M context: (a) one decode step, (b) prefill in 16K chunks
    "decode_b1_1m": DecodeConfig(4, "decode_b1_1m", 1, M1, 32, 8, 128, (0, 3), 0.95, 4, 8192, 1024, True),
    "prefill_1m": PrefillConfig(5, "prefill_1m", M1, 16384, 32, 8, 128, (0, 3), 4, 8192, 32),
}


def scaled_decode(cfg: DecodeConfig, **over) -> DecodeConfig:
    """A copy of a decode configuration with some fields replaced (e.g. smaller n_ctx)."""
    d = {k: getattr(cfg, k) for k in cfg.__dataclass_fields__}
    d.update(over)
    return DecodeConfig(**d)


def scaled_prefill(cfg: PrefillConfig, **over) -> PrefillConfig:
    d = {k: getattr(cfg, k) for k in cfg.__dataclass_fields__}
    d.update(over)
    return PrefillConfig(**d)


# ----------------------------------------------------------------------------- decode inputs
@dataclass
class DecodeInputs:
    cfg: DecodeConfig
    n_cap: int
    q_pre: np.ndarray      # [B][Hq][D] bf16 bits, pre-RoPE (indexer input)
    q: np.ndarray          # [B][Hq][D] bf16 bits, post-RoPE at position N-1
    k: np.ndarray          # [B][Hkv][n_cap][D] bf16 bits, post-RoPE
    v: np.ndarray          # [B][Hkv][n_cap][D] bf16 bits
    k_idx: np.ndarray      # [B][Hkv_r][n_cap][16] bf16 bits (pre-RoPE key projection; needles planted)
    w_q_idx: np.ndarray    # [Hq_r][D][16] bf16 bits
    w_k_idx: np.ndarray    # [Hkv_r][D][16] bf16 bits
    kv_role: np.ndarray    # [Hkv] uint8, 1 = retrieval
    needle_pos: np.ndarray  # [B][Hkv_r][n_needles] int64
    q_scale: np.ndarray    # [B][Hq] float32 per-head query scale (1 when not lognormal)
    extra: dict = field(default_factory=dict)


def make_decode_inputs(cfg: DecodeConfig, n_cap: Optional[int] = None,
                       zero_query_heads: Tuple[int, ...] = ()) -> DecodeInputs:
    """Draw one decode step's inputs.  Rows [n_ctx, n_cap) of the caches are zero.

    ``zero_query_heads`` forces q (both pre- and post-RoPE) of the listed global
    query heads to zero, for closed-form edge cases.
    """
    B, N, Hq, Hkv, D = cfg.batch, cfg.n_ctx, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = cfg.group
    ncap = N if n_cap is None else int(n_cap)
    assert ncap >= N
    ret = list(cfg.retrieval_kv)
    Hkv_r, Hq_r = len(ret), len(ret) * G
    cid = cfg.cid

    I = cfg.idx_dim
    w_q = np.stack([_normal_bf16(_rng(cid, T_WQ, 0, i), (D, I), 1.0 / np.sqrt(D)) for i in range(Hq_r)]) \
        if Hq_r else np.zeros((0, D, I), np.uint16)
    w_k = np.stack([_normal_bf16(_rng(cid, T_WK, 0, i), (D, I), 1.0 / np.sqrt(D)) for i in range(Hkv_r)]) \
        if Hkv_r else np.zeros((0, D, I), np.uint16)

    q_scale = np.ones((B, Hq), np.float32)
    if cfg.lognormal_qscale:
        for b in range(B):
            q_scale[b] = _rng(cid, T_QSCALE, b, 0).lognormal(0.0, 1.0, Hq).astype(np.float32)
    q_pre = np.empty((B, Hq, D), np.uint16)
    for b in range(B):
        for h in range(Hq):
            x = _rng(cid, T_Q, b, h).standard_normal(D, dtype=np.float32) * q_scale[b, h]
            if h in zero_query_heads:
                x[:] = 0
            q_pre[b, h] = f32_to_bf16_bits(x)
    q = _rope_bf16(q_pre.reshape(B * Hq, D), np.full(B * Hq, N - 1)).reshape(B, Hq, D)

    k = np.zeros((B, Hkv, ncap, D), np.uint16)
    v = np.zeros((B, Hkv, ncap, D), np.uint16)
    k_idx = np.zeros((B, Hkv_r, ncap, I), np.uint16)
    n_needles = min(cfg.n_needles, N)
    needle_pos = np.zeros((B, Hkv_r, n_needles), np.int64)
    pos = np.arange(N)
    wq64 = bf16_bits_to_f32(w_q).astype(np.float64)
    wk64 = bf16_bits_to_f32(w_k).astype(np.float64)
    _rope_tables(pos, D)                       # fill the table cache once

    def one(bg):
        b, g = bg
        k_pre = _normal_bf16(_rng(cid, T_K, b, g), (N, D))
        k[b, g, :N] = _rope_bf16(k_pre, pos)
        v[b, g, :N] = _normal_bf16(_rng(cid, T_V, b, g), (N, D))
        if g in ret:
            r = ret.index(g)
            # products by numpy's own loops, not BLAS: BLAS called from several of these
            # worker threads at once has returned differing results from run to run
            proj = np.einsum("nd,di->ni", bf16_bits_to_f32(k_pre).astype(np.float64), wk64[r], optimize=False)
            k_idx[b, r, :N] = f32_to_bf16_bits(proj.astype(np.float32))
            if n_needles:
                npos = np.sort(_rng(cid, T_NEEDLE, b, r).choice(N, size=n_needles, replace=False))
                needle_pos[b, r] = npos
                qi = [np.einsum("d,di->i", bf16_bits_to_f32(q_pre[b, g * G + t]).astype(np.float64),
                                wq64[r * G + t], optimize=False) for t in range(G)]
                needle = 4.0 * np.mean(np.stack(qi), axis=0)
                k_idx[b, r, npos] = f32_to_bf16_bits(needle.astype(np.float32))[None, :]

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(one, [(b, g) for b in range(B) for g in range(Hkv)]))
    return DecodeInputs(cfg, ncap, q_pre, q, k, v, k_idx, w_q, w_k, cfg.kv_role, needle_pos, q_scale)


# ----------------------------------------------------------------------------- prefill inputs
class PrefillInputs:
    """Lazily drawn chunked-prefill inputs.

    Every chunk's q / pre-RoPE k / v come from per-(chunk, head) substreams, so a
    single chunk (or a few sampled rows) can be regenerated without the rest.
    """

    def __init__(self, cfg: PrefillConfig):
        self.cfg = cfg
        D, Hkv_r = cfg.head_dim, cfg.n_kv_r
        self.w_k_idx = np.stack([_normal_bf16(_rng(cfg.cid, T_WK, 0, i), (D, cfg.idx_dim), 1.0 / np.sqrt(D))
                                 for i in range(Hkv_r)])
        self.kv_role = cfg.kv_role

    def chunk_bounds(self, c: int) -> Tuple[int, int]:
        c0 = c * self.cfg.chunk
        return c0, min(self.cfg.seq_len, c0 + self.cfg.chunk)

    def q_chunk(self, c: int, heads=None) -> np.ndarray:
        """[C][Hq][D] bf16 bits (post-RoPE) for chunk c."""
        cfg = self.cfg
        c0, c1 = self.chunk_bounds(c)
        C = c1 - c0
        heads = range(cfg.n_q_heads) if heads is None else heads
        out = np.zeros((C, cfg.n_q_heads, cfg.head_dim), np.uint16)
        for h in heads:
            out[:, h] = self.q_head(c, h)
        return out

    def q_head(self, c: int, h: int) -> np.ndarray:
        """[C][D] bf16 bits (post-RoPE): query head h of chunk c (the same values as q_chunk)."""
        cfg = self.cfg
        c0, c1 = self.chunk_bounds(c)
        return _rope_bf16(_normal_bf16(_rng(cfg.cid, T_Q, c, h), (c1 - c0, cfg.head_dim)), np.arange(c0, c1))

    def k_pre_chunk(self, c: int) -> np.ndarray:
        """[C][Hkv][D] bf16 bits, pre-RoPE keys of chunk c."""
        cfg = self.cfg
        c0, c1 = self.chunk_bounds(c)
        out = np.empty((c1 - c0, cfg.n_kv_heads, cfg.head_dim), np.uint16)
        for g in range(cfg.n_kv_heads):
            out[:, g] = _normal_bf16(_rng(cfg.cid, T_K, c, g), (c1 - c0, cfg.head_dim))
        return out

    def k_chunk(self, c: int, k_pre: Optional[np.ndarray] = None) -> np.ndarray:
        """[Hkv][C][D] bf16 bits, post-RoPE keys of chunk c (cache layout)."""
        kp = self.k_pre_chunk(c) if k_pre is None else k_pre
        c0, c1 = self.chunk_bounds(c)
        pos = np.arange(c0, c1)
        return np.stack([_rope_bf16(kp[:, g], pos) for g in range(self.cfg.n_kv_heads)])

    def v_chunk(self, c: int) -> np.ndarray:
        """[Hkv][C][D] bf16 bits."""
        cfg = self.cfg
        c0, c1 = self.chunk_bounds(c)
        return np.stack([_normal_bf16(_rng(cfg.cid, T_V, c, g), (c1 - c0, cfg.head_dim))
                         for g in range(cfg.n_kv_heads)])

    def full_kv(self) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """(k [Hkv][T][D], v [Hkv][T][D], k_pre [T][Hkv][D]) for the whole sequence."""
        ks, vs, kps = [], [], []
        for c in range(self.cfg.n_chunks):
            kp = self.k_pre_chunk(c)
            kps.append(kp)
            ks.append(self.k_chunk(c, kp))
            vs.append(self.v_chunk(c))
        return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1), np.concatenate(kps, axis=0)

    def sample_rows(self, head: int) -> np.ndarray:
        """Seeded query rows checked for one head: the first and last row, then random rows."""
        cfg = self.cfg
        rng = _rng(cfg.cid, 100, head, 0)
        n = cfg.rows_per_head
        fixed = np.unique([0, cfg.seq_len - 1, min(cfg.seq_len - 1, cfg.window),
                           min(cfg.seq_len - 1, cfg.chunk)])[:n]
        pool = np.setdiff1d(np.arange(cfg.seq_len), fixed)
        rest = rng.choice(pool, size=min(pool.size, max(0, n - fixed.size)), replace=False)
        return np.sort(np.concatenate([fixed, rest])).astype(np.int64)
