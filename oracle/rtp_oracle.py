"""Plain fp64 CPU oracle for RTPurbo's head-wise sparse attention (test infrastructure).

THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it.  It shares no code with the HIP library: the only thing the
two sides have in common is the seeded input arrays, which the callers hand in.

Source: "Full Attention Strikes Back: Transferring Full Attention into Sparse
within Hundred Training Steps" (arXiv 2605.16928, method RTPurbo), as printed on
its abstract pages (OpenAlex record / podcast episode page) and the atlas.scime.ai
research-map summary.  The pages give no equations, so every step below is the
plainest reading of their prose; each function names the passage it follows.

Everything is computed in fp64 from the bf16 inputs (upcast exactly).  The only
rounding the oracle performs on purpose is the bf16 store of the prefill indexer
keys (the cache holds bf16).

Pins (tests/test_oracle_pins.py): brute-force minimal top-p sets on tiny rows,
hand-worked golden rows (tests/golden/), p=1 and window>=N reduce to dense
attention checked against torch's float64 scaled_dot_product_attention, q=0
reduces to the mean of V over exactly the attended set, bilinearity and
position-independence of indexer scores, torch's float32->bfloat16 RNE cast for
the bf16 store, and the recall statistic on a hand-worked three-key case (its
softmax scale included) and the all-tokens case.  Recall is computed but not
reported by the benchmark.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

IDX_DIM = 16


# ----------------------------------------------------------------------------- bf16 conversion
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 raw bits (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 straight to bf16 (round half to even), returned as raw uint16 bits.

    Written from the format's definition: a normal bf16 value is m * 2**e with an
    8-bit significand, so the value is frexp's mantissa scaled to 8 bits and
    rounded half-to-even (numpy's rint), with no intermediate float32 rounding.
    Zeros keep their sign; the cases here never reach the subnormal range.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0)                    # 8 significant bits, ties to even
    y = np.ldexp(r, e - 8)                    # exact in float64
    nz = x != 0
    if np.any(nz & (np.abs(y) < 2.0 ** -126)):
        raise ValueError("bf16 subnormal range not supported by the oracle")
    y32 = y.astype(np.float32)                # exact: y has <= 8 significant bits
    return (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------- indexer (decode)
def indexer_query(q_pre: np.ndarray, w_q_idx: np.ndarray) -> np.ndarray:
    """16-dim query indexer vector from the *pre-RoPE* query of one head.

    Abstract, observation (2): long-range retrieval lives in a low-dimensional
    subspace, reached with a 16-dimensional indexer; research-map summary,
    "Approach": the selector is a low-dimensional *pre-RoPE* projection.
    q_pre: [D] (bf16 values), w_q_idx: [D][16] -> [16] fp64, not rounded.
    """
    return np.asarray(q_pre, np.float64) @ np.asarray(w_q_idx, np.float64)


def indexer_scores(q_idx: np.ndarray, k_idx: np.ndarray, idx_scale: float = 1.0) -> np.ndarray:
    """Indexer score of every cached token: s_j = idx_scale * <q_idx, k_idx_j>.

    k_idx: [N][16] stored (bf16) pre-RoPE key projections.  No position enters.
    """
    return float(idx_scale) * (np.asarray(k_idx, np.float64) @ np.asarray(q_idx, np.float64))


def softmax_mass(scores: np.ndarray) -> np.ndarray:
    """Softmax of the indexer scores: pi_j = exp(s_j - max s) / sum_k exp(s_k - max s)."""
    s = np.asarray(scores, np.float64)
    w = np.exp(s - s.max())
    return w / math.fsum(w.tolist()) if w.size < 4096 else w / w.sum(dtype=np.float64)


def topp_select(scores: np.ndarray, p: float) -> Tuple[np.ndarray, Dict[str, np.ndarray]]:
    """Query-adaptive top-p token set (abstract, observation (3); summary, "Approach").

    Tokens are ranked by score, highest first, equal scores by lower index first.
    The set is the shortest prefix of that ranking whose softmax mass reaches p.
    p >= 1 keeps every token (cumulative floating-point sums need not reach 1.0).

    Returns (selected indices ascending, info) where info holds the ranking
    ``order``, the per-rank masses ``pi_sorted``, the cumulative masses ``cum``
    (cum[k] = mass of the first k+1 ranked tokens) and ``k`` = |S|.
    """
    s = np.asarray(scores, np.float64)
    n = s.size
    if not (p > 0.0):
        raise ValueError("top-p threshold must be > 0")
    idx = np.arange(n)
    order = np.lexsort((idx, -s))                       # score desc, then index asc
    pi = softmax_mass(s)[order]
    cum = np.cumsum(pi)
    if p >= 1.0:
        k = n
    else:
        k = int(np.searchsorted(cum, p, side="left")) + 1   # first rank with cum >= p
        k = min(k, n)
    sel = np.sort(order[:k])
    return sel, {"order": order, "pi_sorted": pi, "cum": cum, "k": np.int64(k)}


def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """Fixed-budget selection, the static rule the abstract contrasts with top-p: the k
    tokens that rank first by (score descending, index ascending), in increasing index
    order; k >= N keeps all N.  (Research-map summary, "Key results": top-k is the
    fixed-budget baseline the adaptive rule is compared against.)"""
    s = np.asarray(scores, np.float64)
    order = np.lexsort((np.arange(s.size), -s))
    return np.sort(order[:min(int(k), s.size)])


# ----------------------------------------------------------------------------- local heads
def local_set(n_ctx: int, n_sinks: int, window: int) -> np.ndarray:
    """Sink + sliding-window token set of a local head (summary, "Approach").

    The query is the last cached token (position n_ctx-1).  Sinks are the first
    ``n_sinks`` tokens; the window is the last ``window`` tokens and includes the
    query's own token.  The union never counts a token twice.
    """
    sinks = np.arange(min(n_sinks, n_ctx))
    win = np.arange(max(0, n_ctx - window), n_ctx)
    return np.union1d(sinks, win)


# ----------------------------------------------------------------------------- attention
def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray, sm_scale: float) -> np.ndarray:
    """Softmax attention of one query row over the listed cached tokens only.

    o = sum_{j in idx} softmax_j(sm_scale * q.k_j) v_j.  q: [D]; k, v: [N][D].
    """
    idx = np.asarray(idx)
    if idx.size == 0:
        raise ValueError("empty attention set")
    kk = np.asarray(k, np.float64)[idx]
    vv = np.asarray(v, np.float64)[idx]
    logits = sm_scale * (kk @ np.asarray(q, np.float64))
    a = np.exp(logits - logits.max())
    a /= a.sum()
    return a @ vv


def attention_recall(q: np.ndarray, k: np.ndarray, v_unused, n_ctx: int, sel: np.ndarray,
                     sm_scale: float) -> float:
    """Attention-mass recall of a selected set (summary, "Experimental setup", metrics):
    the share of the full-context attention softmax that falls on the selected tokens."""
    kk = np.asarray(k, np.float64)[:n_ctx]
    logits = sm_scale * (kk @ np.asarray(q, np.float64))
    a = np.exp(logits - logits.max())
    a /= a.sum()
    return float(a[np.asarray(sel)].sum())


# ----------------------------------------------------------------------------- one decode step
def decode_step(q_pre, q, k, v, k_idx, w_q_idx, kv_role, n_ctx: int, top_p, n_sinks: int, window: int,
                sm_scale: Optional[float] = None, idx_scale: float = 1.0, w_shared: bool = False,
                with_recall: bool = False, batch_rows: Optional[Sequence[int]] = None) -> Dict[str, object]:
    """One decode step of one layer, every head (abstract: full KV kept only for
    retrieval heads, which use the token indexer; summary "Approach": local heads
    use sinks plus a sliding window).

    Arrays are bf16 raw bits in the library layouts:
      q_pre, q: [B][Hq][D]; k, v: [B][Hkv][n_cap][D]; k_idx: [B][Hkv_r][n_cap][16];
      w_q_idx: [Hq_r][D][16] (or [1][D][16] when ``w_shared``); kv_role: [Hkv].
    ``top_p`` is a float or a per-retrieval-query-head sequence [Hq_r].
    Retrieval query head h = g*G + t with retrieval rank r has compact index r*G + t.

    Returns a dict with ``out`` [B][Hq][D] fp64 and, per retrieval row
    (b, compact index), ``scores``, ``sel``, ``info`` (and ``recall``).
    """
    q_pre, q = np.asarray(q_pre), np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    roles = np.asarray(kv_role)
    ret = [g for g in range(Hkv) if roles[g]]
    Hq_r = len(ret) * G
    p_of = (lambda i: float(top_p)) if np.isscalar(top_p) else (lambda i: float(top_p[i]))
    out = np.zeros((B, Hq, D), np.float64)
    scores, sels, infos, recalls = {}, {}, {}, {}
    lset = local_set(n_ctx, n_sinks, window)
    rows = range(B) if batch_rows is None else batch_rows
    for b in rows:
        for g in range(Hkv):
            kb = bf16_to_f64(k[b, g, :n_ctx])
            vb = bf16_to_f64(v[b, g, :n_ctx])
            for t in range(G):
                h = g * G + t
                qh = bf16_to_f64(q[b, h])
                if roles[g]:
                    r = ret.index(g)
                    ci = r * G + t
                    wq = bf16_to_f64(w_q_idx[0 if w_shared else ci])
                    qi = indexer_query(bf16_to_f64(q_pre[b, h]), wq)
                    s = indexer_scores(qi, bf16_to_f64(k_idx[b, r, :n_ctx]), idx_scale)
                    sel, info = topp_select(s, p_of(ci))
                    out[b, h] = attend(qh, kb, vb, sel, sm_scale)
                    scores[(b, ci)] = s
                    sels[(b, ci)] = sel
                    infos[(b, ci)] = info
                    if with_recall:
                        recalls[(b, ci)] = attention_recall(qh, kb, None, n_ctx, sel, sm_scale)
                else:
                    out[b, h] = attend(qh, kb, vb, lset, sm_scale)
    return {"out": out, "scores": scores, "sel": sels, "info": infos, "recall": recalls,
            "local_set": lset, "Hq_r": Hq_r}


# ----------------------------------------------------------------------------- prefill
def prefill_kidx(k_pre: np.ndarray, w_k_idx: np.ndarray, kv_role) -> np.ndarray:
    """Indexer keys written by a prefill chunk: bf16(k_pre . W_k_idx) for every
    retrieval KV head (pre-RoPE projection, summary "Approach"; the cache keeps
    the per-token 16-dim keys of retrieval heads, abstract).

    k_pre: [C][Hkv][D] bf16 bits; w_k_idx: [Hkv_r][D][I] -> [Hkv_r][C][I] bf16 bits (I = 16 on
    the pages' design; the same projection for the other indexer dimensions).
    """
    roles = np.asarray(kv_role)
    ret = [g for g in range(len(roles)) if roles[g]]
    out = []
    for r, g in enumerate(ret):
        proj = bf16_to_f64(k_pre[:, g]) @ bf16_to_f64(w_k_idx[r])
        out.append(f64_to_bf16(proj))
    return np.stack(out) if out else np.zeros((0, k_pre.shape[0], np.shape(w_k_idx)[-1]), np.uint16)


def prefill_row_set(i: int, retrieval: bool, n_sinks: int, window: int) -> np.ndarray:
    """Keys seen by prefill query row i.  Retrieval heads stay dense and causal in
    prefill (summary, "Limitations"); local heads see sinks + window, causally."""
    if retrieval:
        return np.arange(i + 1)
    return local_set(i + 1, n_sinks, window)


def prefill_rows(q_rows: np.ndarray, rows: Sequence[int], k: np.ndarray, v: np.ndarray, retrieval: bool,
                 n_sinks: int, window: int, sm_scale: Optional[float] = None) -> np.ndarray:
    """Prefill output of one query head at absolute rows ``rows``.

    q_rows: [len(rows)][D] bf16 bits; k, v: [T][D] bf16 bits (this head's KV head).
    """
    D = q_rows.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    kk, vv = bf16_to_f64(k), bf16_to_f64(v)
    return np.stack([attend(bf16_to_f64(q_rows[n]), kk, vv,
                            prefill_row_set(int(i), retrieval, n_sinks, window), sm_scale)
                     for n, i in enumerate(rows)])


# ----------------------------------------------------------------------------- set comparison rule
def exempt_ranks(info: Dict[str, np.ndarray], p: float, tol: float = 1e-4) -> np.ndarray:
    """Ranks whose mass interval [cum_{k-1}, cum_k] meets [p - tol, p + tol].

    Selected sets are compared outside these tokens: a token that sits on the
    p boundary within the tolerance may be in or out.
    """
    cum = info["cum"]
    lo = np.concatenate([[0.0], cum[:-1]])
    return np.nonzero((cum >= p - tol) & (lo <= p + tol))[0]


def set_mass(info: Dict[str, np.ndarray], sel: np.ndarray) -> float:
    """fp64 softmax mass of an arbitrary index set under the row's score distribution."""
    order, pi = info["order"], info["pi_sorted"]
    mass = np.zeros(order.size)
    mass[order] = pi
    return float(mass[np.asarray(sel, dtype=np.int64)].sum())
