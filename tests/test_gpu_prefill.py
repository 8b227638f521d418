"""GPU parity of the prefill path (rtp_prefill_attn) against the fp64 oracle.

The cache holds the whole sequence's post-RoPE keys and values up front; causality
means chunk c only reads keys below its last row, exactly as if the chunks had been
appended one by one.  Small cases check every row; the 32K and 1M configurations
check the oracle's seeded sample rows of every head (first, last, window- and
chunk-boundary rows included) and the full indexer-key projection.
"""
import math

import numpy as np
import pytest

from head_wise_sparse_amd import rtp
from head_wise_sparse_amd import workloads as W
from oracle import rtp_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu


def _run_prefill(cfg, pi, k, v, kp, keep_rows=None):
    """Run every chunk; returns (out bf16 bits, k_idx bits).  `out` is [T][Hq][D], or, when
    `keep_rows` is given, a dict row -> [Hq][D] holding only those rows."""
    import torch
    T, Hq, D = cfg.seq_len, cfg.n_q_heads, cfg.head_dim
    L = rtp.Layer(1, Hq, cfg.n_kv_heads, D, T, cfg.kv_role.tolist(), cfg.n_sinks, cfg.window, idx_dim=cfg.idx_dim)
    I = cfg.idx_dim
    kd, vd = P.dev(k), P.dev(v)
    w = P.dev(pi.w_k_idx)
    kidx = torch.zeros(cfg.n_kv_r * T * I, dtype=torch.bfloat16, device="cuda")
    out = np.zeros((T, Hq, D), np.uint16) if keep_rows is None else {}
    ws = rtp.workspace(L, cfg.chunk, rtp.CALL_PREFILL)
    for c in range(cfg.n_chunks):
        c0, c1 = pi.chunk_bounds(c)
        q = P.dev(pi.q_chunk(c))
        o = torch.empty((c1 - c0) * Hq * D, dtype=torch.bfloat16, device="cuda")
        rtp.rtp_prefill_attn(L, c0, c1 - c0, q, kd, vd, P.dev(kp[c0:c1]), w, D * I, kidx, 1 / math.sqrt(D), o,
                             ws)
        torch.cuda.synchronize()
        ob = rtp.from_device_bf16(o).reshape(c1 - c0, Hq, D)
        if keep_rows is None:
            out[c0:c1] = ob
        else:
            for r in keep_rows:
                if c0 <= r < c1:
                    out[int(r)] = ob[r - c0]
    return out, rtp.from_device_bf16(kidx).reshape(cfg.n_kv_r, T, I)


def _check_rows(cfg, pi, k, v, out, rows_of_head):
    G = cfg.group
    worst = 0.0
    for h in range(cfg.n_q_heads):
        g = h // G
        rows = rows_of_head(h)
        qs = {}
        for r in rows:
            c = r // cfg.chunk
            if c not in qs:
                qs[c] = pi.q_head(c, h)
        q_rows = np.stack([qs[r // cfg.chunk][r - (r // cfg.chunk) * cfg.chunk] for r in rows])
        ref = O.prefill_rows(q_rows, rows, k[g], v[g], bool(cfg.kv_role[g]), cfg.n_sinks, cfg.window)
        got = out[rows, h] if isinstance(out, np.ndarray) else np.stack([out[int(r)][h] for r in rows])
        e, _ = P.check_outputs(got, ref, f"head {h} ({'retrieval' if cfg.kv_role[g] else 'local'})")
        worst = max(worst, e)
    return worst


def _check_kidx(cfg, pi, kp, kidx):
    """The stored bf16 keys must be the oracle's (bf16 of the fp64 projection) except where the
    kernel's fp32 accumulation lands on the other side of a rounding boundary: then the value
    is within one bf16 ulp of the exact projection plus the fp32 dot-product error bound
    (128 terms: 1e-6 of the sum of |terms|, generous), which matters only under cancellation."""
    ref = O.prefill_kidx(kp, pi.w_k_idx, cfg.kv_role)
    ret = [g for g in range(cfg.n_kv_heads) if cfg.kv_role[g]]
    same = 0
    for r, g in enumerate(ret):
        a = O.bf16_to_f64(kp[:, g])
        w = O.bf16_to_f64(pi.w_k_idx[r])
        exact = a @ w
        terms = np.abs(a) @ np.abs(w)
        got = O.bf16_to_f64(kidx[r])
        allow = P.bf16_ulp(exact) + 1e-6 * terms
        err = np.abs(got - exact)
        if (err > allow).any():
            t, c = np.argwhere(err > allow)[0]
            raise AssertionError(f"indexer key (r={r}, t={t}, c={c}): gpu {got[t, c]} exact {exact[t, c]}")
        same += int((kidx[r] == ref[r]).sum())
    assert same >= 0.99 * ref.size


@pytest.mark.parametrize("over", [
    dict(seq_len=700, chunk=256, window=100, n_sinks=4),          # ragged chunks, window crosses tiles
    dict(seq_len=513, chunk=513, window=4096, n_sinks=4),         # window covers everything: causal
    dict(seq_len=640, chunk=192, window=1, n_sinks=0),            # query token only
    dict(seq_len=600, chunk=128, window=70, n_sinks=0),           # no sinks: first rows see few keys
    dict(seq_len=900, chunk=300, window=130, n_sinks=77),         # sinks span two key tiles
    dict(seq_len=150, chunk=17, window=40, n_sinks=3),            # chunks shorter than one 32-row block
    dict(seq_len=40, chunk=1, window=9, n_sinks=2),               # one row per chunk
    dict(seq_len=520, chunk=260, window=100, n_sinks=4, idx_dim=4),   # indexer dims of the ablation
    dict(seq_len=520, chunk=260, window=100, n_sinks=4, idx_dim=8),
    dict(seq_len=520, chunk=260, window=100, n_sinks=4, idx_dim=32),
])
def test_prefill_small_all_rows(over):
    P.require_gpu()
    cfg = W.scaled_prefill(W.CONFIGS["prefill_32k"], rows_per_head=4, **over)
    pi = W.PrefillInputs(cfg)
    k, v, kp = pi.full_kv()
    out, kidx = _run_prefill(cfg, pi, k, v, kp)
    heads = [0, 1, 4, 13, 31]
    # every row of a few heads of each kind
    G = cfg.group
    for h in heads:
        g = h // G
        rows = np.arange(cfg.seq_len)
        q_rows = np.concatenate([pi.q_head(c, h) for c in range(cfg.n_chunks)])
        ref = O.prefill_rows(q_rows, rows, k[g], v[g], bool(cfg.kv_role[g]), cfg.n_sinks, cfg.window)
        P.check_outputs(out[:, h], ref, f"head {h}")
    _check_kidx(cfg, pi, kp, kidx)


@pytest.mark.parametrize("hq,hkv,retr", [
    (8, 8, (0, 3)),        # one query head per KV head: a block takes 4 row slices of one head
    (16, 8, (1, 6)),       # two per KV head: 2 heads x 2 row slices
    (64, 8, (0, 3)),       # eight per KV head: two head groups of 4 per KV head
])
def test_prefill_query_group_sizes(hq, hkv, retr):
    P.require_gpu()
    cfg = W.scaled_prefill(W.CONFIGS["prefill_32k"], seq_len=700, chunk=256, window=100, n_sinks=4,
                           rows_per_head=4, n_q_heads=hq, n_kv_heads=hkv, retrieval_kv=retr)
    pi = W.PrefillInputs(cfg)
    k, v, kp = pi.full_kv()
    out, kidx = _run_prefill(cfg, pi, k, v, kp)
    G = cfg.group
    for h in sorted({0, 1, G - 1, G, hq // 2 + 1, hq - 1} & set(range(hq))):
        g = h // G
        rows = np.arange(cfg.seq_len)
        q_rows = np.concatenate([pi.q_head(c, h) for c in range(cfg.n_chunks)])
        ref = O.prefill_rows(q_rows, rows, k[g], v[g], bool(cfg.kv_role[g]), cfg.n_sinks, cfg.window)
        P.check_outputs(out[:, h], ref, f"head {h} (G={G})")
    _check_kidx(cfg, pi, kp, kidx)


@pytest.mark.parametrize("over", [
    dict(seq_len=700, chunk=256, window=100, n_sinks=4),                       # G = 4, ragged chunks
    dict(seq_len=900, chunk=300, window=130, n_sinks=77),                      # sinks span two key tiles
    dict(seq_len=40, chunk=1, window=9, n_sinks=2),                            # one row per chunk
    dict(seq_len=513, chunk=513, window=4096, n_sinks=4),                      # window covers everything
    dict(seq_len=600, chunk=200, window=70, n_sinks=3, n_q_heads=8),           # G = 1
    dict(seq_len=600, chunk=200, window=70, n_sinks=3, n_q_heads=16),          # G = 2
    dict(seq_len=520, chunk=260, window=100, n_sinks=4, idx_dim=32),           # two indexer column blocks
])
def test_prefill_head_dim_64(over):
    """Head dimension 64 (its own tile layout and slot schedule): every row of several heads
    of each kind, and the indexer keys."""
    P.require_gpu()
    cfg = W.scaled_prefill(W.CONFIGS["prefill_32k"], rows_per_head=4, head_dim=64, **over)
    pi = W.PrefillInputs(cfg)
    k, v, kp = pi.full_kv()
    out, kidx = _run_prefill(cfg, pi, k, v, kp)
    G, Hq = cfg.group, cfg.n_q_heads
    for h in sorted({0, 1, G - 1, G, 3 * G, Hq // 2 + 1, Hq - 1} & set(range(Hq))):
        g = h // G
        rows = np.arange(cfg.seq_len)
        q_rows = np.concatenate([pi.q_head(c, h) for c in range(cfg.n_chunks)])
        ref = O.prefill_rows(q_rows, rows, k[g], v[g], bool(cfg.kv_role[g]), cfg.n_sinks, cfg.window)
        P.check_outputs(out[:, h], ref, f"head {h} (D=64, G={G})")
    _check_kidx(cfg, pi, kp, kidx)


@pytest.mark.parametrize("retr", [(0, 3), (0, 1, 2, 3, 4, 5, 6, 7)])
def test_prefill_ignores_rows_past_the_chunk(retr):
    """Cache rows at or past c0 + C are not valid yet (the contract): fill them with NaN and
    the chunk's outputs must still match the oracle (a key tile that crosses the chunk's end
    must not let those rows into the sums, not even as 0 * NaN)."""
    P.require_gpu()
    import torch
    cfg = W.scaled_prefill(W.CONFIGS["prefill_32k"], seq_len=700, chunk=300, window=100, n_sinks=4,
                           rows_per_head=4, retrieval_kv=retr)
    pi = W.PrefillInputs(cfg)
    k, v, kp = pi.full_kv()
    T, Hq, D, G = cfg.seq_len, cfg.n_q_heads, cfg.head_dim, cfg.group
    L = rtp.Layer(1, Hq, cfg.n_kv_heads, D, T, cfg.kv_role.tolist(), cfg.n_sinks, cfg.window, idx_dim=cfg.idx_dim)
    I = cfg.idx_dim
    w = P.dev(pi.w_k_idx)
    kidx = torch.zeros(cfg.n_kv_r * T * I, dtype=torch.bfloat16, device="cuda")
    ws = rtp.workspace(L, cfg.chunk, rtp.CALL_PREFILL)
    nan = np.uint16(0x7FC0)
    for c in range(cfg.n_chunks):
        c0, c1 = pi.chunk_bounds(c)
        kn, vn = k.copy(), v.copy()
        kn[:, c1:] = nan
        vn[:, c1:] = nan
        q = P.dev(pi.q_chunk(c))
        o = torch.empty((c1 - c0) * Hq * D, dtype=torch.bfloat16, device="cuda")
        rtp.rtp_prefill_attn(L, c0, c1 - c0, q, P.dev(kn), P.dev(vn), P.dev(kp[c0:c1]), w, D * I, kidx,
                             1 / math.sqrt(D), o, ws)
        torch.cuda.synchronize()
        ob = rtp.from_device_bf16(o).reshape(c1 - c0, Hq, D)
        for h in (0, 1, G, Hq - 1):
            g = h // G
            rows = np.arange(c0, c1)
            ref = O.prefill_rows(pi.q_head(c, h), rows, k[g], v[g], bool(cfg.kv_role[g]),
                                 cfg.n_sinks, cfg.window)
            P.check_outputs(ob[:, h], ref, f"chunk {c} head {h}")


def test_prefill_all_local_heads():
    """No retrieval head: no indexer-key work, the indexer pointers may be NULL."""
    P.require_gpu()
    import torch
    cfg = W.scaled_prefill(W.CONFIGS["prefill_32k"], seq_len=600, chunk=256, window=70, n_sinks=5, rows_per_head=4)
    pi = W.PrefillInputs(cfg)
    k, v, _ = pi.full_kv()
    T, Hq, D, G = cfg.seq_len, cfg.n_q_heads, cfg.head_dim, cfg.group
    L = rtp.Layer(1, Hq, cfg.n_kv_heads, D, T, [0] * cfg.n_kv_heads, cfg.n_sinks, cfg.window, idx_dim=cfg.idx_dim)
    ws = rtp.workspace(L, cfg.chunk, rtp.CALL_PREFILL)
    kd, vd = P.dev(k), P.dev(v)
    for c in range(cfg.n_chunks):
        c0, c1 = pi.chunk_bounds(c)
        o = torch.empty((c1 - c0) * Hq * D, dtype=torch.bfloat16, device="cuda")
        rtp.rtp_prefill_attn(L, c0, c1 - c0, P.dev(pi.q_chunk(c)), kd, vd, None, None, 0, None, 1 / math.sqrt(D), o, ws)
        torch.cuda.synchronize()
        ob = rtp.from_device_bf16(o).reshape(c1 - c0, Hq, D)
        for h in (0, G + 1, Hq - 1):
            ref = O.prefill_rows(pi.q_head(c, h), np.arange(c0, c1), k[h // G], v[h // G], False,
                                 cfg.n_sinks, cfg.window)
            P.check_outputs(ob[:, h], ref, f"chunk {c} head {h}")


def test_prefill_32k_sampled_rows():
    P.require_gpu()
    cfg = W.CONFIGS["prefill_32k"]
    pi = W.PrefillInputs(cfg)
    k, v, kp = pi.full_kv()
    out, kidx = _run_prefill(cfg, pi, k, v, kp)
    worst = _check_rows(cfg, pi, k, v, out, pi.sample_rows)
    _check_kidx(cfg, pi, kp, kidx)
    print(f"\nprefill 32K: worst |gpu - oracle| on sampled rows {worst:.3e}")


def test_prefill_is_deterministic():
    P.require_gpu()
    cfg = W.scaled_prefill(W.CONFIGS["prefill_32k"], seq_len=2048, chunk=1024, rows_per_head=4)
    pi = W.PrefillInputs(cfg)
    k, v, kp = pi.full_kv()
    a, ka = _run_prefill(cfg, pi, k, v, kp)
    b, kb = _run_prefill(cfg, pi, k, v, kp)
    assert np.array_equal(a, b) and np.array_equal(ka, kb)


@pytest.mark.slow
@pytest.mark.timeout(900)         # 64 chunks on the GPU plus the oracle's rows over 1M keys on the host
def test_prefill_1m_sampled_rows():
    P.require_gpu()
    cfg = W.CONFIGS["prefill_1m"]
    pi = W.PrefillInputs(cfg)
    k, v, kp = pi.full_kv()
    keep = np.unique(np.concatenate([pi.sample_rows(h) for h in range(cfg.n_q_heads)]))
    out, kidx = _run_prefill(cfg, pi, k, v, kp, keep_rows=keep)
    worst = _check_rows(cfg, pi, k, v, out, pi.sample_rows)
    _check_kidx(cfg, pi, kp, kidx)
    print(f"\nprefill 1M: worst |gpu - oracle| on sampled rows {worst:.3e}")
