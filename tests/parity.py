"""Shared pieces of the GPU parity tests: moving generator inputs to the device,
running the library's calls, and the comparison rules.

Comparison rules (the tolerances the decode path is held to):
  * indexer scores: |gpu - oracle| <= 1e-4 * sum_c |q_idx_c * k_idx_c|, i.e. 1e-4
    relative to the magnitude of the dot product's terms (a plain per-element
    relative error is meaningless for scores near 0);
  * selected sets: identical, except tokens whose oracle cumulative-mass interval
    touches [p - 1e-4, p + 1e-4], and -- when the GPU scored the tokens itself --
    tokens whose oracle score lies within the fp32 scoring error bound of the
    boundary token's score (their order can legitimately flip); the GPU set's
    fp64 mass must reach p - 1e-4;
  * attention outputs: max-abs 1e-2 plus half a bf16 ulp of the reference value
    (the output is stored in bf16), and relative L2 <= 5e-3 per output row.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np
import pytest

from head_wise_sparse_amd import rtp
from oracle import rtp_oracle as O

SCORE_RTOL = 1e-4
MASS_TOL = 1e-4
OUT_ATOL = 1e-2
OUT_RL2 = 5e-3
# fp32 scoring error bound, relative to sum_c |q_idx_c k_c|: q_idx is a 128-term fp32
# dot product and the score a 16-term one; 2*(128+16)*2^-24 ~ 1.7e-5, rounded up.
FP32_SCORE_SLACK = 2e-5


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    if not __import__("os").path.exists(rtp.LIB_PATH):
        pytest.fail("librtp.so missing on a GPU machine: build it first (no fallback exists)")


def dev(bits: np.ndarray):
    return rtp.to_device_bf16(bits)


def layer_for(cfg, n_cap=None) -> rtp.Layer:
    return rtp.Layer(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                     cfg.n_ctx if n_cap is None else n_cap, cfg.kv_role.tolist(), cfg.n_sinks, cfg.window,
                     idx_dim=cfg.idx_dim)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.frexp(np.where(ax > 0, ax, 1.0))[1]
    return np.ldexp(1.0, e - 8)


def check_outputs(gpu_bits: np.ndarray, ref: np.ndarray, what: str = ""):
    g = O.bf16_to_f64(gpu_bits).reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: {int((~np.isfinite(g)).sum())} non-finite outputs"
    err = np.abs(g - ref)
    allow = OUT_ATOL + 0.5 * bf16_ulp(ref)
    bad = err > allow
    assert not bad.any(), f"{what}: {bad.sum()} outputs beyond max-abs tolerance, worst {err.max():.3e}"
    g2 = g.reshape(-1, ref.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    num = np.linalg.norm(g2 - r2, axis=1)
    den = np.maximum(np.linalg.norm(r2, axis=1), 1e-30)
    rl2 = num / den
    assert (rl2 <= OUT_RL2).all(), f"{what}: relative L2 {rl2.max():.3e} > {OUT_RL2}"
    return float(err.max()), float(rl2.max())


def check_set(gpu_sel: np.ndarray, info: Dict[str, np.ndarray], p: float, scores64: np.ndarray = None,
              slack: np.ndarray = None) -> Tuple[bool, int]:
    """Compare one selected set with the oracle's.  Returns (identical, n_exempt_differences)."""
    order = info["order"]
    k = int(info["k"])
    ora = np.sort(order[:k])
    gpu = np.asarray(gpu_sel, np.int64)
    assert np.all(np.diff(gpu) > 0), "selected indices must be strictly increasing"
    if p >= 1.0:
        assert np.array_equal(gpu, np.arange(order.size))
        return True, 0
    diff = np.setxor1d(gpu, ora)
    if diff.size == 0:
        return True, 0
    exempt = set(order[O.exempt_ranks(info, p, MASS_TOL)].tolist())
    if scores64 is not None:
        b = order[k - 1]
        near = np.abs(scores64 - scores64[b]) <= slack + slack[b]
        exempt |= set(np.nonzero(near)[0].tolist())
    stray = [int(j) for j in diff if int(j) not in exempt]
    assert not stray, f"tokens {stray[:10]} differ from the oracle set and are not on the p boundary"
    assert O.set_mass(info, gpu) >= p - MASS_TOL
    return False, int(diff.size)


def check_prefix(gpu_sel: np.ndarray, scores32: np.ndarray, what: str = ""):
    """The selected set must be the first |S| tokens of the (score descending, index ascending)
    order of the very fp32 scores the kernel ranked (-0 and +0 tie).  The mass arithmetic only
    decides |S|; which tokens fill it, ties included, is exact integer/fp32 comparison work,
    so this holds bit for bit wherever the mass boundary falls."""
    sel = np.asarray(gpu_sel, np.int64)
    if sel.size == 0:
        return
    s = np.asarray(scores32, np.float32) + np.float32(0.0)
    t = s[sel].min()
    above = np.flatnonzero(s > t)
    tied = np.flatnonzero(s == t)
    n_t = sel.size - above.size
    assert 1 <= n_t <= tied.size, f"{what}: the set is not a prefix of the score order"
    want = np.sort(np.concatenate([above, tied[:n_t]]))
    assert np.array_equal(sel, want), f"{what}: the set is not the first {sel.size} tokens of the score order " \
        f"(ties are taken lowest index first)"


def sel_zero_bytes(L, n_ctx) -> int:
    """Bytes at the start of the selection region that every call leaves zero: all of it but
    the trailing digit tables (B * Hq_r * ceil(n_cap / RTP_SEL_RANGE) * 2 KiB), which calls
    write whole before they read them and leave as they are."""
    from head_wise_sparse_amd import rtp
    tables = L.batch * L.n_kv_r * L.group * (-(-L.n_cap // rtp.SEL_RANGE)) * 2048
    return rtp.rtp_workspace_bytes(L, n_ctx, rtp.CALL_TOPP_SELECT) - tables


class DeviceDecode:
    """Generator inputs of one decode configuration, resident on the GPU."""

    def __init__(self, x):
        import torch
        self.x = x
        self.q_pre = dev(x.q_pre)
        self.q = dev(x.q)
        self.k = dev(x.k)
        self.v = dev(x.v)
        self.k_idx = dev(x.k_idx)
        self.w_q_idx = dev(x.w_q_idx)
        torch.cuda.synchronize()


def score_scale(x, b: int, ci: int, r: int, n_ctx: int) -> np.ndarray:
    """sum_c |q_idx_c * k_idx_{j,c}| for every token of one retrieval row (fp64)."""
    G = x.cfg.group
    g = x.cfg.retrieval_kv[r]
    qi = O.indexer_query(O.bf16_to_f64(x.q_pre[b, g * G + ci % G]), O.bf16_to_f64(x.w_q_idx[ci]))
    return np.abs(O.bf16_to_f64(x.k_idx[b, r, :n_ctx])) @ np.abs(qi)


def check_retrieval_row(g_row: np.ndarray, x, b: int, h: int, gpu_sel: np.ndarray, n_ctx: int, same: bool,
                        ora_out_row: np.ndarray, what: str = ""):
    """Output of one retrieval query row.  When the GPU set equals the oracle's, against the
    oracle's output; otherwise against the oracle's attention over the GPU's own set (the set
    itself is judged by check_set), so that every row's gather and merge are checked."""
    if same:
        return check_outputs(g_row[None], ora_out_row[None], what)
    G = x.cfg.group
    D = x.cfg.head_dim
    sel = np.asarray(gpu_sel, np.int64)
    if sel.size == 0:
        assert np.all(O.bf16_to_f64(g_row) == 0), f"{what}: an empty set must give a zero row"
        return 0.0, 0.0
    ref = O.attend(O.bf16_to_f64(x.q[b, h]), O.bf16_to_f64(x.k[b, h // G, :n_ctx]),
                   O.bf16_to_f64(x.v[b, h // G, :n_ctx]), sel, 1 / math.sqrt(D))
    return check_outputs(g_row[None], ref[None], what + " (over the GPU's set)")
