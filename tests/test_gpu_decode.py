"""GPU parity of the decode path against the fp64 oracle, through the C ABI.

Each call is checked on its own with oracle-made inputs (so a mismatch names the
call), then the whole decode step is checked end to end on every decode
configuration.  Sizes span several tiles and ragged tails; edge cases cover ties,
p = 1, p -> 0, tiny and capacity-padded contexts, empty and full sets.
"""
import math

import numpy as np
import pytest

from head_wise_sparse_amd import rtp
from head_wise_sparse_amd import workloads as W
from oracle import rtp_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu

_CACHE = {}


def _inputs(name, **over):
    key = (name, tuple(sorted(over.items())))
    if key not in _CACHE:
        cfg = W.CONFIGS[name]
        if over:
            cfg = W.scaled_decode(cfg, **over)
        _CACHE.clear()
        x = W.make_decode_inputs(cfg)
        _CACHE[key] = (x, P.DeviceDecode(x))
    return _CACHE[key]


def _torch():
    import torch
    return torch


# ----------------------------------------------------------------------------- indexer scores
@pytest.mark.parametrize("name,over", [("decode_tiny_2k", {}), ("decode_b8_32k", {}),
                                       ("decode_b8_32k", dict(n_ctx=3001, batch=2)),
                                       ("decode_b4_128k", {}),
                                       ("decode_b8_32k", dict(n_ctx=5000, batch=2, idx_dim=4)),
                                       ("decode_b8_32k", dict(n_ctx=5000, batch=2, idx_dim=8)),
                                       ("decode_b8_32k", dict(n_ctx=5000, batch=2, idx_dim=32)),
                                       ("decode_tiny_2k", dict(idx_dim=4))])
def test_indexer_scores(name, over):
    P.require_gpu()
    torch = _torch()
    x, d = _inputs(name, **over)
    cfg = x.cfg
    L = P.layer_for(cfg)
    B, R, N = cfg.batch, cfg.n_kv_r * cfg.group, cfg.n_ctx
    scores = torch.full((B * R * N,), float("nan"), dtype=torch.float32, device="cuda")
    rmax = torch.empty(B * R, dtype=torch.float32, device="cuda")
    rsum = torch.empty(B * R, dtype=torch.float32, device="cuda")
    ws = rtp.workspace(L, N, rtp.CALL_INDEXER_SCORE)
    rtp.rtp_indexer_score(L, N, d.q_pre, d.w_q_idx, cfg.head_dim * cfg.idx_dim, d.k_idx, 1.0, scores, rmax, rsum,
                          ws)
    torch.cuda.synchronize()
    sg = scores.view(B, R, N).cpu().numpy().astype(np.float64)
    mg, zg = rmax.view(B, R).cpu().numpy(), rsum.view(B, R).cpu().numpy()
    G = cfg.group
    for b in range(B):
        for ci in range(R):
            r = ci // G
            g = cfg.retrieval_kv[r]
            qi = O.indexer_query(O.bf16_to_f64(x.q_pre[b, g * G + ci % G]), O.bf16_to_f64(x.w_q_idx[ci]))
            so = O.indexer_scores(qi, O.bf16_to_f64(x.k_idx[b, r, :N]))
            scale = P.score_scale(x, b, ci, r, N)
            err = np.abs(sg[b, ci] - so)
            assert np.all(err <= P.SCORE_RTOL * scale), f"row ({b},{ci}): worst {np.max(err / scale):.2e}"
            assert abs(mg[b, ci] - so.max()) <= P.SCORE_RTOL * scale.max()
            z = np.exp(so - so.max()).sum()
            assert abs(zg[b, ci] - z) <= 1e-4 * z


def test_indexer_scores_exact_on_integer_inputs():
    """Small-integer bf16 inputs make every product and sum exact in fp32: bitwise equality."""
    P.require_gpu()
    torch = _torch()
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, N = 2, 8, 2, 64, 5000
    L = rtp.Layer(B, Hq, Hkv, D, N + 100, [1, 1], 0, 1)
    f = lambda a: W.f32_to_bf16_bits(a.astype(np.float32))
    q_pre = f(rng.integers(-2, 3, (B, Hq, D)))
    w = np.zeros((Hq, D, 16), np.float32)
    for c in range(Hq):
        w[c, rng.choice(D, 16, replace=False), np.arange(16)] = rng.integers(-2, 3, 16)
    w = f(w)
    k_idx = f(rng.integers(-3, 4, (B, 2, N + 100, 16)))
    scores = torch.zeros(B * Hq * (N + 100), dtype=torch.float32, device="cuda")
    rm = torch.empty(B * Hq, dtype=torch.float32, device="cuda")
    rs = torch.empty_like(rm)
    rtp.rtp_indexer_score(L, N, P.dev(q_pre), P.dev(w), D * 16, P.dev(k_idx), 1.0, scores, rm, rs,
                          rtp.workspace(L, N, rtp.CALL_INDEXER_SCORE))
    torch.cuda.synchronize()
    sg = scores.view(B, Hq, N + 100).cpu().numpy()
    for b in range(B):
        for c in range(Hq):
            qi = O.bf16_to_f64(q_pre[b, c]) @ O.bf16_to_f64(w[c])
            so = O.bf16_to_f64(k_idx[b, c // 4, :N]) @ qi
            assert np.array_equal(sg[b, c, :N].astype(np.float64), so)
            assert np.all(sg[b, c, N:] == 0)                  # rows past n_ctx untouched


# ----------------------------------------------------------------------------- top-p selection
def _run_select(L, n_ctx, scores32: np.ndarray, p: float, n_cap=None):
    """scores32: [rows][n_ctx] float32 -> list of selected index arrays."""
    torch = _torch()
    rows = scores32.shape[0]
    cap = L.n_cap
    s = np.zeros((rows, cap), np.float32)
    s[:, :n_ctx] = scores32
    st = torch.from_numpy(s).cuda()
    m = torch.from_numpy(scores32.max(axis=1).astype(np.float32)).cuda()
    z = torch.from_numpy(np.exp(scores32.astype(np.float64) - scores32.max(axis=1, keepdims=True))
                         .sum(axis=1).astype(np.float32)).cuda()
    sel = torch.full((rows * cap,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    nsplit = (n_ctx + rtp.SEL_RANGE - 1) // rtp.SEL_RANGE
    starts = torch.full((rows * (nsplit + 1),), -3, dtype=torch.int32, device="cuda")
    ws = rtp.workspace(L, n_ctx, rtp.CALL_TOPP_SELECT)
    rtp.rtp_topp_select(L, n_ctx, st, m, z, p, sel, cnt, starts, ws)
    torch.cuda.synchronize()
    assert not ws[:P.sel_zero_bytes(L, n_ctx)].any().item(), "the selection workspace must be left zero-filled"
    seln, cntn = sel.view(rows, cap).cpu().numpy(), cnt.cpu().numpy()
    stn = starts.view(rows, nsplit + 1).cpu().numpy()
    out = []
    for r in range(rows):
        c = int(cntn[r])
        assert 1 <= c <= n_ctx
        assert np.all(seln[r, c:] == -7), "entries past sel_count must be untouched"
        out.append(seln[r, :c])
        # range index: entry q counts the selected tokens below q * SEL_RANGE
        want = np.searchsorted(seln[r, :c], np.arange(nsplit + 1) * rtp.SEL_RANGE)
        want[nsplit] = c
        assert np.array_equal(stn[r], want), f"row {r}: range index differs"
    return out


def _check_rows(scores32, sets, p):
    ident = 0
    for r in range(scores32.shape[0]):
        s64 = scores32[r].astype(np.float64)
        _, info = O.topp_select(s64, p)
        same, _ = P.check_set(sets[r], info, p)
        P.check_prefix(sets[r], scores32[r], f"row {r}")
        ident += same
    return ident


@pytest.mark.parametrize("name,p", [("decode_tiny_2k", 0.9), ("decode_b8_32k", 0.95), ("decode_b4_128k", 0.9),
                                    ("decode_b4_128k", 0.95), ("decode_b4_128k", 0.99)])
def test_topp_select_on_oracle_scores(name, p):
    """Selection alone: the oracle's scores rounded to fp32 feed both sides, so both take
    the ranking decision in the kernel's precision."""
    P.require_gpu()
    x, _ = _inputs(name)
    cfg = x.cfg
    G = cfg.group
    rows = []
    for b in range(cfg.batch):
        for ci in range(cfg.n_kv_r * G):
            r = ci // G
            g = cfg.retrieval_kv[r]
            qi = O.indexer_query(O.bf16_to_f64(x.q_pre[b, g * G + ci % G]), O.bf16_to_f64(x.w_q_idx[ci]))
            rows.append(O.indexer_scores(qi, O.bf16_to_f64(x.k_idx[b, r, :cfg.n_ctx])).astype(np.float32))
    s32 = np.stack(rows)
    L = rtp.Layer(s32.shape[0], 1, 1, 128, cfg.n_ctx, [1], 0, 1)          # one score row per batch entry
    sets = _run_select(L, cfg.n_ctx, s32, p)
    ident = _check_rows(s32, sets, p)
    assert ident >= 0.9 * len(sets)


def _edge_rows():
    rng = np.random.default_rng(11)
    yield "all_tied", np.zeros((2, 5000), np.float32), 0.5
    two = np.zeros((1, 4097), np.float32)
    two[0, rng.choice(4097, 300, replace=False)] = 1.0
    yield "two_levels_tied", two, 0.37
    yield "p_one", rng.standard_normal((3, 2049)).astype(np.float32), 1.0
    yield "p_tiny", np.round(rng.standard_normal((3, 3000)), 1).astype(np.float32), 1e-7
    yield "single_token", np.float32([[3.5], [-2.0]]), 0.9
    z = rng.standard_normal((2, 6000)).astype(np.float32)
    z[:, ::7] = 0.0
    z[:, 3::7] = -0.0
    yield "signed_zeros", z, 0.8
    # rows of at most 8192 tokens take the single-block path: its boundaries (4096 and 8192
    # tokens: 16 or 32 scores per thread), a narrow spread that leaves the cut to the last
    # digit, a wide one, and near-equal clusters
    rs = np.random.default_rng(12)
    yield "short_narrow", (5 + rs.standard_normal((3, 8192)) * 1e-3).astype(np.float32), 0.9
    yield "short_wide", (rs.standard_normal((2, 8191)) * 300).astype(np.float32), 0.95
    yield "short_at_4096", (rs.standard_normal((2, 4096)) * 3).astype(np.float32), 0.9
    yield "short_at_4097", np.round(rs.standard_normal((2, 4097)) * 3, 1).astype(np.float32), 0.7
    c = np.full((2, 7000), -12.0, np.float32)
    pos = rs.choice(7000, 600, replace=False)
    c[:, pos] = (np.float32(1.0).view(np.uint32) + rs.integers(0, 40, 600).astype(np.uint32)).view(np.float32)
    yield "short_clustered", c, 0.5
    yield "short_many_rows", rs.standard_normal((300, 1500)).astype(np.float32) * 2, 0.9
    yield "wide_spread", (rng.standard_normal((2, 9000)) * 300).astype(np.float32), 0.95
    yield "narrow_spread", (5 + rng.standard_normal((2, 20000)) * 1e-3).astype(np.float32), 0.9
    yield "ragged_many_tiles", rng.standard_normal((4, 2048 * 5 + 3)).astype(np.float32) * 3, 0.99
    # near-equal clusters in every 4096-token tile: scores 1 + k ulp share the top 22 key
    # bits, so the cut falls among tokens the radix passes cannot tell apart until the
    # last 10 bits; 8 per tile stay within a tile record's digits, 12 per tile overflow it
    for name, per in (("clustered_light", 8), ("clustered_heavy", 12)):
        n = 4096 * 5 + 700
        c = np.full((2, n), -12.0, np.float32)
        for tile in range((n + 4095) // 4096):
            lo, hi = tile * 4096, min(n, tile * 4096 + 4096)
            pos = rng.choice(np.arange(lo, hi), per, replace=False)
            ulps = rng.integers(0, 4, per)
            c[:, pos] = (np.float32(1.0).view(np.uint32) + ulps.astype(np.uint32)).view(np.float32)
        yield name, c, 0.5
    # a narrow spread over more than 256 tiles: every range holds many distinct candidates
    # (a heavy record, counted from its table), and the last compaction block clears the
    # records in several rounds of 256
    yield "narrow_many_heavy_tiles", (5 + rng.standard_normal((1, 4096 * 268 + 100)) * 1e-3).astype(np.float32), 0.9
    # enough rows x tiles that the passes use 8192-token tiles: plain, tied and narrow rows,
    # ragged tail
    n = 8192 * 15 + 123
    z = (rng.standard_normal((36, n)) * 3).astype(np.float32)
    z[12:24] = np.round(z[12:24], 2)
    z[24:] = (5 + rng.standard_normal((12, n)) * 1e-3).astype(np.float32)
    yield "long_tiles", z, 0.9


@pytest.mark.parametrize("case", list(_edge_rows()), ids=lambda c: c[0])
def test_topp_select_edge_cases(case):
    P.require_gpu()
    _, s32, p = case
    n = s32.shape[1]
    L = rtp.Layer(s32.shape[0], 1, 1, 64, n + 37, [1], 0, 1)      # capacity larger than the context
    sets = _run_select(L, n, s32, p)
    _check_rows(s32, sets, p)
    if case[0] == "all_tied":
        assert all(np.array_equal(s, np.arange(2500)) for s in sets)   # lowest indices first
    if case[0] == "p_tiny":
        for r, s in enumerate(sets):
            assert s.tolist() == [int(np.flatnonzero(s32[r] == s32[r].max())[0])]


def test_topp_select_flat_row_at_largest_context():
    """A flat row (every score equal) at 2^24 tokens, the longest context top-p accepts: all
    weights equal the row max's, so the row total is n_ctx times the largest weight -- the
    case where a fixed-point total with too many fraction bits would wrap -- and the set is
    exactly the first ceil(p * n_ctx) tokens (ties are taken lowest index first)."""
    P.require_gpu()
    n = 1 << 24
    L = rtp.Layer(2, 1, 1, 64, n, [1], 0, 1)
    s32 = np.zeros((2, n), np.float32)
    s32[1] = 3.25
    for p in (0.5, 0.999):
        sets = _run_select(L, n, s32, p)
        k = math.ceil(p * n)
        for s in sets:
            assert s.size == k and s[0] == 0 and s[-1] == k - 1 and np.all(np.diff(s) == 1)


# ----------------------------------------------------------------------------- sparse decode
def _sel_tensors(sets, B, R, cap):
    torch = _torch()
    sel = np.zeros((B, R, cap), np.int32)
    cnt = np.zeros((B, R), np.int32)
    for (b, ci), s in sets.items():
        sel[b, ci, :len(s)] = s
        cnt[b, ci] = len(s)
    return torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda()


@pytest.mark.parametrize("name,over", [("decode_tiny_2k", {}), ("decode_b8_32k", {}),
                                       ("decode_b8_32k", dict(batch=2, n_ctx=5000)),
                                       ("decode_b1_1m", dict(n_ctx=200000))])     # > 128 splits: two-level merge
def test_sparse_decode_on_oracle_sets(name, over):
    P.require_gpu()
    torch = _torch()
    x, d = _inputs(name, **over)
    cfg = x.cfg
    N, B, G = cfg.n_ctx, cfg.batch, cfg.group
    R = cfg.n_kv_r * G
    ora = O.decode_step(x.q_pre, x.q, x.k, x.v, x.k_idx, x.w_q_idx, x.kv_role, N, cfg.top_p, cfg.n_sinks,
                        cfg.window)
    L = P.layer_for(cfg)
    sel, cnt = _sel_tensors(ora["sel"], B, R, N)
    out = torch.zeros(B * cfg.n_q_heads * cfg.head_dim, dtype=torch.bfloat16, device="cuda")
    rtp.rtp_sparse_decode_attn(L, N, d.q, d.k, d.v, sel, cnt, None, 1 / math.sqrt(cfg.head_dim), out,
                               rtp.workspace(L, N, rtp.CALL_SPARSE_DECODE))
    torch.cuda.synchronize()
    g = rtp.from_device_bf16(out).reshape(B, cfg.n_q_heads, cfg.head_dim)
    heads = [gg * G + t for gg in cfg.retrieval_kv for t in range(G)]
    P.check_outputs(g[:, heads], ora["out"][:, heads], "sparse decode")
    loc = [h for h in range(cfg.n_q_heads) if h not in heads]
    assert np.all(g[:, loc] == 0), "local-head rows must not be written"


def test_sparse_decode_ignores_indices_past_the_context():
    """Lists holding entries at or past n_ctx (a malformed caller list) make the call read no
    cache row there: the result is bit-identical to that of the clean lists.  The cache holds
    exactly n_ctx rows and the last index range runs past them."""
    P.require_gpu()
    torch = _torch()
    x, d = _inputs("decode_b8_32k", batch=2, n_ctx=5000)
    cfg = x.cfg
    N, B, G = cfg.n_ctx, cfg.batch, cfg.group
    R = cfg.n_kv_r * G
    L = P.layer_for(cfg)
    rng = np.random.default_rng(3)
    clean, bogus = {}, {}
    for b in range(B):
        for ci in range(R):
            s_ = np.unique(np.concatenate([rng.choice(N, 300, replace=False), [N - 1]]))
            clean[(b, ci)] = s_
            bogus[(b, ci)] = np.concatenate([s_, [N, N + 50, 5119]]) if (b + ci) % 2 == 0 else s_
    outs = []
    for sets in (clean, bogus):
        sel, cnt = _sel_tensors(sets, B, R, N)
        out = torch.zeros(B * cfg.n_q_heads * cfg.head_dim, dtype=torch.bfloat16, device="cuda")
        rtp.rtp_sparse_decode_attn(L, N, d.q, d.k, d.v, sel, cnt, None, 1 / math.sqrt(cfg.head_dim), out,
                                   rtp.workspace(L, N, rtp.CALL_SPARSE_DECODE))
        torch.cuda.synchronize()
        outs.append(rtp.from_device_bf16(out))
    assert np.array_equal(outs[0], outs[1])


def test_sparse_decode_special_sets():
    """Empty set -> zeros; one token -> that V row; every token -> dense attention;
    overlapping random sets inside a GQA group."""
    P.require_gpu()
    torch = _torch()
    x, d = _inputs("decode_b8_32k", batch=1, n_ctx=7000)
    cfg = x.cfg
    N, G = cfg.n_ctx, cfg.group
    rng = np.random.default_rng(3)
    sets = {(0, 0): np.zeros(0, np.int64), (0, 1): np.array([4321]), (0, 2): np.arange(N),
            (0, 3): np.sort(rng.choice(N, 3000, replace=False)),
            (0, 4): np.sort(rng.choice(N, 50, replace=False)), (0, 5): np.arange(0, N, 3),
            (0, 6): np.arange(2040, 2060), (0, 7): np.array([0, N - 1])}
    L = P.layer_for(cfg)
    sel, cnt = _sel_tensors(sets, 1, 8, N)
    out = torch.zeros(cfg.n_q_heads * cfg.head_dim, dtype=torch.bfloat16, device="cuda")
    rtp.rtp_sparse_decode_attn(L, N, d.q, d.k, d.v, sel, cnt, None, 1 / math.sqrt(128), out,
                               rtp.workspace(L, N, rtp.CALL_SPARSE_DECODE))
    # the same sets with a caller-built range index give the same bits
    nsplit = (N + rtp.SEL_RANGE - 1) // rtp.SEL_RANGE
    st = np.zeros((8, nsplit + 1), np.int32)
    for (b, ci), s_ in sets.items():
        st[ci] = np.searchsorted(s_, np.arange(nsplit + 1) * rtp.SEL_RANGE)
        st[ci, nsplit] = len(s_)
    out2 = torch.zeros_like(out)
    rtp.rtp_sparse_decode_attn(L, N, d.q, d.k, d.v, sel, cnt, torch.from_numpy(st).cuda(), 1 / math.sqrt(128), out2,
                               rtp.workspace(L, N, rtp.CALL_SPARSE_DECODE))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    g = rtp.from_device_bf16(out).reshape(cfg.n_q_heads, 128)
    for (b, ci), s in sets.items():
        h = cfg.retrieval_kv[ci // G] * G + ci % G
        kv = cfg.retrieval_kv[ci // G]
        if len(s) == 0:
            assert np.all(g[h] == 0)
            continue
        ref = O.attend(O.bf16_to_f64(x.q[0, h]), O.bf16_to_f64(x.k[0, kv, :N]), O.bf16_to_f64(x.v[0, kv, :N]), s,
                       1 / math.sqrt(128))
        P.check_outputs(g[h][None], ref[None], f"set {ci}")
    assert np.array_equal(g[cfg.retrieval_kv[0] * G + 1], x.v[0, cfg.retrieval_kv[0], 4321])


# ----------------------------------------------------------------------------- window + sinks
@pytest.mark.parametrize("name,over", [("decode_tiny_2k", {}), ("decode_b8_32k", {}),
                                       ("decode_b8_32k", dict(batch=1, n_ctx=3)),
                                       ("decode_b8_32k", dict(batch=1, n_ctx=700, window=5000)),
                                       ("decode_b8_32k", dict(batch=1, n_ctx=999, window=1, n_sinks=0)),
                                       ("decode_b8_32k", dict(batch=2, n_ctx=4000, window=3, n_sinks=7)),
                                       ("decode_tiny_2k", dict(n_sinks=300, window=1800))])
def test_window_sink_decode(name, over):
    P.require_gpu()
    torch = _torch()
    x, d = _inputs(name, **over)
    cfg = x.cfg
    N, B, G = cfg.n_ctx, cfg.batch, cfg.group
    L = P.layer_for(cfg)
    out = torch.zeros(B * cfg.n_q_heads * cfg.head_dim, dtype=torch.bfloat16, device="cuda")
    rtp.rtp_window_sink_attn(L, N, d.q, d.k, d.v, 1 / math.sqrt(cfg.head_dim), out,
                             rtp.workspace(L, N, rtp.CALL_WINDOW_SINK))
    torch.cuda.synchronize()
    g = rtp.from_device_bf16(out).reshape(B, cfg.n_q_heads, cfg.head_dim)
    lset = O.local_set(N, cfg.n_sinks, cfg.window)
    ref = np.zeros((B, cfg.n_q_heads, cfg.head_dim))
    loc = [gg * G + t for gg in range(cfg.n_kv_heads) if not x.kv_role[gg] for t in range(G)]
    for b in range(B):
        for h in loc:
            kv = h // G
            ref[b, h] = O.attend(O.bf16_to_f64(x.q[b, h]), O.bf16_to_f64(x.k[b, kv, :N]),
                                 O.bf16_to_f64(x.v[b, kv, :N]), lset, 1 / math.sqrt(cfg.head_dim))
    P.check_outputs(g[:, loc], ref[:, loc], "window decode")
    ret = [h for h in range(cfg.n_q_heads) if h not in loc]
    assert np.all(g[:, ret] == 0), "retrieval-head rows must not be written"


# ----------------------------------------------------------------------------- whole decode step
def _decode_step(name, p, **over):
    torch = _torch()
    x, d = _inputs(name, **over)
    cfg = x.cfg
    L = P.layer_for(cfg)
    step = rtp.DecodeStep(L, cfg.n_ctx, p)
    out = step.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)
    torch.cuda.synchronize()
    return x, d, step, out


@pytest.mark.parametrize("name,p", [("decode_tiny_2k", 0.9), ("decode_b8_32k", 0.95), ("decode_b4_128k", 0.9),
                                    ("decode_b4_128k", 0.95), ("decode_b4_128k", 0.99), ("decode_b1_1m", 0.95)])
def test_decode_step_end_to_end(name, p):
    P.require_gpu()
    x, d, step, out = _decode_step(name, p)
    cfg = x.cfg
    N, B, G = cfg.n_ctx, cfg.batch, cfg.group
    R = cfg.n_kv_r * G
    ora = O.decode_step(x.q_pre, x.q, x.k, x.v, x.k_idx, x.w_q_idx, x.kv_role, N, p, cfg.n_sinks, cfg.window)
    g = rtp.from_device_bf16(out).reshape(B, cfg.n_q_heads, cfg.head_dim)
    cnt = step.sel_count.view(B, R).cpu().numpy()
    sel = step.sel_idx.view(B, R, N).cpu().numpy()
    gsc = step.scores.view(B, R, -1)[:, :, :N].cpu().numpy()
    identical, sizes = [], []
    for b in range(B):
        for ci in range(R):
            r = ci // G
            P.check_prefix(sel[b, ci, :cnt[b, ci]], gsc[b, ci], f"row ({b},{ci})")   # on the kernel's own scores
            scale = P.score_scale(x, b, ci, r, N)
            same, _ = P.check_set(sel[b, ci, :cnt[b, ci]], ora["info"][(b, ci)], p, ora["scores"][(b, ci)],
                                  P.FP32_SCORE_SLACK * scale)
            h = cfg.retrieval_kv[r] * G + ci % G
            P.check_retrieval_row(g[b, h], x, b, h, sel[b, ci, :cnt[b, ci]], N, same, ora["out"][b, h],
                                  f"retrieval row ({b},{h})")
            identical.append(same)
            sizes.append(int(cnt[b, ci]))
    loc = [gg * G + t for gg in range(cfg.n_kv_heads) if not x.kv_role[gg] for t in range(G)]
    P.check_outputs(g[:, loc], ora["out"][:, loc], "local rows")
    print(f"\n{name} p={p}: |S| min {min(sizes)} median {int(np.median(sizes))} mean {np.mean(sizes):.0f} "
          f"max {max(sizes)}; sets identical {sum(identical)}/{len(identical)}")
    assert sum(identical) >= 0.9 * len(identical)


@pytest.mark.parametrize("fused", [True, False])
def test_decode_step_ignores_rows_past_the_context(fused):
    """Cache rows at or past n_ctx (K, V and indexer keys) hold NaN: the step reads none of
    them, so every output is bit-identical to the run on zero-filled rows."""
    P.require_gpu()
    torch = _torch()
    cfg = W.scaled_decode(W.CONFIGS["decode_b8_32k"], batch=2, n_ctx=5000)
    cap = 5000 + 700
    x = W.make_decode_inputs(cfg, n_cap=cap)
    L = P.layer_for(cfg, n_cap=cap)
    B, R = cfg.batch, cfg.n_kv_r * cfg.group
    res = []
    for poison in (False, True):
        if poison:
            nan = np.uint16(0x7FC0)
            x.k[:, :, cfg.n_ctx:] = nan
            x.v[:, :, cfg.n_ctx:] = nan
            x.k_idx[:, :, cfg.n_ctx:] = nan
        d = P.DeviceDecode(x)
        step = rtp.DecodeStep(L, cfg.n_ctx, cfg.top_p, fused=fused)
        step.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)
        torch.cuda.synchronize()
        res.append(_step_outputs(step, B, R, cfg.n_ctx))
    _assert_same(res[0], res[1], "NaN past n_ctx")


@pytest.mark.parametrize("head_dim,group", [(64, 1), (64, 2), (64, 4), (64, 8), (128, 1), (128, 2), (128, 8)])
def test_decode_step_shapes(head_dim, group):
    """Every (head_dim, group size) the decode kernels are built for: the fused step against
    the oracle, and bit-identical to the separate calls."""
    _fused_and_separate_against_oracle(dict(head_dim=head_dim, batch=2, n_ctx=6000, n_q_heads=8 * group),
                                       f"head_dim {head_dim}, G {group}")


@pytest.mark.parametrize("n_ctx", [1, 2, 17, 1025, 8192, 8193])
def test_decode_step_degenerate_contexts(n_ctx):
    """A context of one token (every set, sink and window is that token), two tokens, a range
    boundary crossed by one token (1025), and both sides of the single-block selection's
    limit (8192: one launch selects; 8193: the radix passes): the fused step against the
    oracle, and bit-identical to the separate calls."""
    _fused_and_separate_against_oracle(dict(batch=2, n_ctx=n_ctx), f"n_ctx {n_ctx}", min_same=1.0 if n_ctx <= 2 else 0.9)


def _fused_and_separate_against_oracle(over, what, min_same=0.9):
    P.require_gpu()
    torch = _torch()
    x, d = _inputs("decode_b8_32k", **over)
    cfg = x.cfg
    N, B, G = cfg.n_ctx, cfg.batch, cfg.group
    R = cfg.n_kv_r * G
    L = P.layer_for(cfg)
    res = []
    for fused in (False, True):
        step = rtp.DecodeStep(L, N, cfg.top_p, fused=fused)
        step.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)
        torch.cuda.synchronize()
        res.append(_step_outputs(step, B, R, N))
    _assert_same(res[0], res[1], what)
    ora = O.decode_step(x.q_pre, x.q, x.k, x.v, x.k_idx, x.w_q_idx, x.kv_role, N, cfg.top_p, cfg.n_sinks, cfg.window)
    g = res[1]["out"].reshape(B, cfg.n_q_heads, cfg.head_dim)
    same = 0
    for b in range(B):
        for ci in range(R):
            r = ci // G
            ok, _ = P.check_set(res[1]["sets"][b * R + ci], ora["info"][(b, ci)], cfg.top_p, ora["scores"][(b, ci)],
                                P.FP32_SCORE_SLACK * P.score_scale(x, b, ci, r, N))
            h = cfg.retrieval_kv[r] * G + ci % G
            P.check_retrieval_row(g[b, h], x, b, h, res[1]["sets"][b * R + ci], N, ok, ora["out"][b, h],
                                  f"retrieval row ({b},{h})")
            same += ok
    loc = [gg * G + t for gg in range(cfg.n_kv_heads) if not x.kv_role[gg] for t in range(G)]
    P.check_outputs(g[:, loc], ora["out"][:, loc], "local rows")
    assert same >= min_same * B * R


def test_decode_step_is_deterministic():
    P.require_gpu()
    torch = _torch()
    x, d, step, out = _decode_step("decode_b8_32k", 0.95)
    a = [t.clone() for t in (step.scores, step.row_max, step.sel_count, step.sel_idx, step.sel_starts, out)]
    out2 = step.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)
    torch.cuda.synchronize()
    b = [step.scores, step.row_max, step.sel_count, step.sel_idx, step.sel_starts, out2]
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))


def test_decode_step_graph_replay_matches_eager():
    """The decode step captured in a HIP graph (through torch) reproduces the eager result on
    every replay, with eager work and synchronisations between replays."""
    P.require_gpu()
    torch = _torch()
    x, d, step, out = _decode_step("decode_b8_32k", 0.95, batch=2, n_ctx=9000)
    step.sel_idx.fill_(-1)
    step.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (step.sel_count, step.sel_idx, out)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)
    for rep in range(4):
        step.sel_idx.fill_(-1)
        step.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for u, v in zip(ref, (step.sel_count, step.sel_idx, step.out)):
            assert torch.equal(u.view(torch.uint8), v.view(torch.uint8)), f"replay {rep}"
        step.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)      # eager work between replays
        torch.cuda.synchronize()


# ----------------------------------------------------------------------------- fused step
def _step_outputs(step, B, R, n):
    nsplit = (n + rtp.SEL_RANGE - 1) // rtp.SEL_RANGE
    cnt = step.sel_count.view(B, R).cpu().numpy()
    sel = step.sel_idx.view(B, R, -1).cpu().numpy()
    cap = sel.shape[2]
    sc = step.scores.view(B, R, cap)[:, :, :n].cpu().numpy()
    st = step.sel_starts[:B * R * (nsplit + 1)].view(B, R, nsplit + 1).cpu().numpy()
    sets = [sel[b, c, :cnt[b, c]].copy() for b in range(B) for c in range(R)]
    return dict(out=rtp.from_device_bf16(step.out), scores=sc, row_max=step.row_max.cpu().numpy(),
                row_sum=step.row_sum.cpu().numpy(), cnt=cnt, sets=sets, starts=st)


def _assert_same(a, b, what):
    for k in ("out", "scores", "row_max", "row_sum", "cnt", "starts"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), f"{what}: {k} differs"
    assert all(np.array_equal(x, y) for x, y in zip(a["sets"], b["sets"])), f"{what}: sets differ"


@pytest.mark.parametrize("name,p,over", [("decode_tiny_2k", 0.9, {}), ("decode_b8_32k", 0.95, dict(batch=2, n_ctx=9000)),
                                         ("decode_b8_32k", 1.0, dict(batch=1, n_ctx=5000)),
                                         ("decode_b4_128k", 0.99, dict(batch=1)),
                                         ("decode_b4_128k", 0.95, {}),
                                         ("decode_b1_1m", 0.95, dict(n_ctx=200000))])
def test_fused_step_matches_separate_calls(name, p, over):
    """rtp_decode_step gives the same bits as the four calls one after the other (at 128K,
    batch 4 the gather runs one block per 1024-token range, with up to 1014 union rows in
    a range)."""
    P.require_gpu()
    torch = _torch()
    x, d = _inputs(name, **over)
    cfg = x.cfg
    L = P.layer_for(cfg)
    B, R = cfg.batch, cfg.n_kv_r * cfg.group
    res = []
    for fused in (False, True):
        step = rtp.DecodeStep(L, cfg.n_ctx, p, fused=fused)
        step.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)
        torch.cuda.synchronize()
        res.append(_step_outputs(step, B, R, cfg.n_ctx))
        if fused:
            assert not step.ws[rtp.CALL_DECODE_STEP][:P.sel_zero_bytes(L, cfg.n_ctx)] \
                .any().item(), "the selection region must be left zero-filled"
    _assert_same(res[0], res[1], name)


@pytest.mark.parametrize("p", [0.5, 0.97])
def test_fused_step_tie_groups_across_ranges(p):
    """Exact ties at the threshold that span several index ranges (one indexer key repeated):
    the fused step, which takes each range's members from its scores and the range index,
    writes the lists and outputs the separate calls write, whose compaction takes tied
    tokens lowest index first."""
    P.require_gpu()
    torch = _torch()
    x, d = _inputs("decode_b8_32k", batch=1, n_ctx=9000)
    cfg = x.cfg
    L = P.layer_for(cfg)
    B, R, G = cfg.batch, cfg.n_kv_r * cfg.group, cfg.group
    kidx = x.k_idx.copy()
    for r in range(cfg.n_kv_r):
        g = cfg.retrieval_kv[r]
        for h, (lo, hi) in enumerate(((900, 3100), (5000, 6200))):
            # the key of head h's largest |score|, sign-flipped if needed and doubled (both exact
            # in bf16): its copies outscore every other token of that head
            qi = O.indexer_query(O.bf16_to_f64(x.q_pre[0, g * G + h]), O.bf16_to_f64(x.w_q_idx[r * G + h]))
            sc = O.indexer_scores(qi, O.bf16_to_f64(x.k_idx[0, r, :cfg.n_ctx]))
            j = int(np.argmax(np.abs(sc)))
            key = O.bf16_to_f64(x.k_idx[0, r, j]) * (2.0 if sc[j] > 0 else -2.0)
            kidx[0, r, lo:hi] = O.f64_to_bf16(key)
    k_dev = P.dev(kidx)
    res = []
    for fused in (False, True):
        step = rtp.DecodeStep(L, cfg.n_ctx, p, fused=fused)
        step.run(d.q_pre, d.q, d.k, d.v, k_dev, d.w_q_idx)
        torch.cuda.synchronize()
        res.append(_step_outputs(step, B, R, cfg.n_ctx))
    _assert_same(res[0], res[1], f"p={p}")
    if p == 0.5:         # some row takes only part of a tie group that crosses ranges
        part = [s for s in res[0]["sets"] if 0 < np.isin(np.arange(900, 3100), s).sum() < 2200 or
                0 < np.isin(np.arange(5000, 6200), s).sum() < 1200]
        assert part, "no tie group is cut"


def test_fused_step_near_flat_scores():
    """Near-flat scores: the query indexer vector is (1, 2^-14 (h+1), 0, ...) and every key
    (5, r_j, 0, ...) with r_j spread over [-1, 1], so the scores are 5 + r_j 2^-14 (h+1) (up
    to the indexer scale): all within a few 22-bit key prefixes, with many distinct low digits
    in every range.  The resolve then reads the heavy ranges' tables.  Fused step against the
    separate calls, bit for bit, twice on one workspace (the tables are scratch that the
    second call overwrites)."""
    P.require_gpu()
    torch = _torch()
    n, G, D = 40000, 4, 128
    L = rtp.Layer(2, G, 1, D, n, [1], 4, 64)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    bf = lambda *shape, s=1.0: (torch.randn(*shape, generator=gen, device="cuda") * s).to(torch.bfloat16)
    q = bf(2, G, D)
    q_pre = torch.zeros(2, G, D, device="cuda")
    q_pre[:, :, 0] = 1.0
    w_q_idx = torch.zeros(G, D, 16, device="cuda")
    w_q_idx[:, 0, 0] = 1.0
    w_q_idx[:, 0, 1] = torch.tensor([2.0 ** -14 * (h + 1) for h in range(G)], device="cuda")
    k_idx = torch.zeros(2, 1, n, 16, device="cuda")
    k_idx[..., 0] = 5.0
    k_idx[..., 1] = torch.rand(2, 1, n, generator=gen, device="cuda") * 2 - 1
    q_pre, w_q_idx, k_idx = q_pre.to(torch.bfloat16), w_q_idx.to(torch.bfloat16), k_idx.to(torch.bfloat16)
    k, v = bf(2, 1, n, D), bf(2, 1, n, D)
    ref = rtp.DecodeStep(L, n, 0.9, fused=False)
    ref.run(q_pre, q, k, v, k_idx, w_q_idx)
    fused = rtp.DecodeStep(L, n, 0.9, fused=True)
    for rep in range(2):
        fused.run(q_pre, q, k, v, k_idx, w_q_idx)
        torch.cuda.synchronize()
        _assert_same(_step_outputs(ref, 2, G, n), _step_outputs(fused, 2, G, n), f"near-flat, call {rep}")
        assert not fused.ws[rtp.CALL_DECODE_STEP][:P.sel_zero_bytes(L, n)].any().item()
    # the rows are near-flat indeed: a large share of the context is selected, and a range
    # holds many distinct candidate scores
    cnt = ref.sel_count.cpu().numpy()
    assert cnt.min() > n // 4, cnt
    sc = ref.scores.view(2, G, -1)[0, 0, :1024].cpu().numpy()
    assert np.unique(sc).size > 100


def test_fused_step_beyond_1m_tokens():
    """More than 1024 ranges per row (2^21 + 1234 tokens): the resolve block scans the row's
    records in more than one round, and the radix passes use 8192-token tiles of eight
    records.  Fused step against the separate calls, bit for bit, on a layer of one KV head
    (two query heads, head_dim 64) with inputs drawn on the device."""
    P.require_gpu()
    torch = _torch()
    n, G, D = (1 << 21) + 1234, 2, 64
    L = rtp.Layer(1, G, 1, D, n, [1], 4, 64)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    bf = lambda *shape, s=1.0: (torch.randn(*shape, generator=gen, device="cuda") * s).to(torch.bfloat16)
    q_pre, q = bf(1, G, D), bf(1, G, D)
    w_q_idx = bf(G, D, 16, s=0.125)
    k_idx = bf(1, 1, n, 16)
    k, v = bf(1, 1, n, D), bf(1, 1, n, D)
    res = []
    for fused in (False, True):
        step = rtp.DecodeStep(L, n, 0.9, fused=fused)
        step.run(q_pre, q, k, v, k_idx, w_q_idx)
        torch.cuda.synchronize()
        res.append(_step_outputs(step, 1, G, n))
        if fused:
            assert not step.ws[rtp.CALL_DECODE_STEP][:P.sel_zero_bytes(L, n)].any().item()
        del step
    assert all(1 < c.size < n for c in res[0]["sets"])
    _assert_same(res[0], res[1], "2M tokens")


def test_fused_step_growing_context_one_workspace():
    """One fused step object (one workspace) over a growing context: every step equals a
    fresh run of the separate calls at that length."""
    P.require_gpu()
    torch = _torch()
    x, d = _inputs("decode_b8_32k", batch=2, n_ctx=12000)
    cfg = x.cfg
    L = P.layer_for(cfg)
    B, R = cfg.batch, cfg.n_kv_r * cfg.group
    fused = rtp.DecodeStep(L, cfg.n_ctx, 0.95, fused=True)
    for n in (4095, 4096, 4097, 8192 + 5, 12000, 3000):
        fused.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx, n_ctx=n)
        torch.cuda.synchronize()
        a = _step_outputs(fused, B, R, n)
        ref = rtp.DecodeStep(L, n, 0.95, fused=False)
        ref.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx, n_ctx=n)
        torch.cuda.synchronize()
        _assert_same(_step_outputs(ref, B, R, n), a, f"n_ctx={n}")


@pytest.mark.parametrize("roles", ["all_local", "all_retrieval"])
def test_fused_step_single_head_kind(roles):
    P.require_gpu()
    torch = _torch()
    x, d = _inputs("decode_b8_32k", batch=1, n_ctx=6000)
    cfg = x.cfg
    role = [0] * cfg.n_kv_heads if roles == "all_local" else [1] * cfg.n_kv_heads
    L = rtp.Layer(1, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx, role, cfg.n_sinks, cfg.window)
    kidx = d.k_idx if roles == "all_local" else torch.zeros(cfg.n_kv_heads * cfg.n_ctx * 16, dtype=torch.bfloat16,
                                                             device="cuda")
    wq = d.w_q_idx                    # all retrieval: stride 0, every head reads the first matrix
    outs = []
    for fused in (False, True):
        step = rtp.DecodeStep(L, cfg.n_ctx, 0.9, fused=fused)
        step.run(d.q_pre, d.q, d.k, d.v, kidx, wq, w_head_stride=0 if roles == "all_retrieval" else None)
        torch.cuda.synchronize()
        outs.append(rtp.from_device_bf16(step.out))
    assert np.array_equal(outs[0], outs[1])
    if roles == "all_local":
        lset = O.local_set(cfg.n_ctx, cfg.n_sinks, cfg.window)
        g = outs[1].reshape(cfg.n_q_heads, cfg.head_dim)
        ref = np.stack([O.attend(O.bf16_to_f64(x.q[0, h]), O.bf16_to_f64(x.k[0, h // cfg.group, :cfg.n_ctx]),
                                 O.bf16_to_f64(x.v[0, h // cfg.group, :cfg.n_ctx]), lset, 1 / math.sqrt(128))
                        for h in range(cfg.n_q_heads)])
        P.check_outputs(g, ref, "all-local fused step")


# ----------------------------------------------------------------------------- static top-k
def _run_topk(L, n_ctx, scores32, k):
    torch = _torch()
    rows, cap = scores32.shape[0], L.n_cap
    s = np.zeros((rows, cap), np.float32)
    s[:, :n_ctx] = scores32
    sel = torch.full((rows * cap,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    nsplit = (n_ctx + rtp.SEL_RANGE - 1) // rtp.SEL_RANGE
    starts = torch.full((rows * (nsplit + 1),), -3, dtype=torch.int32, device="cuda")
    ws = rtp.workspace(L, n_ctx, rtp.CALL_TOPP_SELECT)
    rtp.rtp_topk_select(L, n_ctx, torch.from_numpy(s).cuda(), k, sel, cnt, starts, ws)
    torch.cuda.synchronize()
    assert not ws[:P.sel_zero_bytes(L, n_ctx)].any().item(), "the selection workspace must be left zero-filled"
    seln, cntn = sel.view(rows, cap).cpu().numpy(), cnt.cpu().numpy()
    stn = starts.view(rows, nsplit + 1).cpu().numpy()
    for r in range(rows):
        c = int(cntn[r])
        want = O.topk_select(scores32[r].astype(np.float64), k)
        assert c == want.size and np.array_equal(seln[r, :c], want), f"row {r}, k={k}"
        assert np.all(seln[r, c:] == -7)
        st = np.searchsorted(want, np.arange(nsplit + 1) * rtp.SEL_RANGE)
        st[nsplit] = c
        assert np.array_equal(stn[r], st)


@pytest.mark.parametrize("k", [1, 2, 255, 1000, 4096, 20000, 33000, 40000])
def test_topk_select_exact(k):
    """Static top-k on oracle-style scores with many exact ties: bit-exact sets."""
    P.require_gpu()
    rng = np.random.default_rng(k)
    n = 33000
    s32 = np.round(rng.standard_normal((5, n)) * 3, 2).astype(np.float32)
    s32[1, ::5] = 7.0                                     # a large tie group at the top
    s32[2] = 0.0                                          # everything tied
    s32[3, 1000:1300] = -0.0
    L = rtp.Layer(s32.shape[0], 1, 1, 64, n + 100, [1], 0, 1)
    _run_topk(L, n, s32, k)


@pytest.mark.parametrize("n,k", [(8192, 1), (8192, 7), (8192, 3000), (8191, 8190), (4096, 1000), (1000, 999)])
def test_topk_select_exact_short_rows(n, k):
    """Static top-k on rows short enough for the single-block path, with exact ties."""
    P.require_gpu()
    rng = np.random.default_rng(n + k)
    s32 = np.round(rng.standard_normal((4, n)) * 3, 1).astype(np.float32)
    s32[1, ::3] = 9.0                                     # a tie group at the top
    s32[2] = -1.5                                         # everything tied
    L = rtp.Layer(s32.shape[0], 1, 1, 64, n + 64, [1], 0, 1)
    _run_topk(L, n, s32, k)


def test_topk_select_real_scores():
    """Top-k over the indexer scores of the 32K decode workload, k = a typical top-p budget."""
    P.require_gpu()
    x, _ = _inputs("decode_b8_32k", batch=2)
    cfg = x.cfg
    G = cfg.group
    rows = []
    for b in range(cfg.batch):
        for ci in range(cfg.n_kv_r * G):
            r = ci // G
            g = cfg.retrieval_kv[r]
            qi = O.indexer_query(O.bf16_to_f64(x.q_pre[b, g * G + ci % G]), O.bf16_to_f64(x.w_q_idx[ci]))
            rows.append(O.indexer_scores(qi, O.bf16_to_f64(x.k_idx[b, r, :cfg.n_ctx])).astype(np.float32))
    s32 = np.stack(rows)
    L = rtp.Layer(s32.shape[0], 1, 1, 128, cfg.n_ctx, [1], 0, 1)
    for k in (64, 2048):
        _run_topk(L, cfg.n_ctx, s32, k)


# ----------------------------------------------------------------------------- compact layout + append
def _ring_slot(j, S, Wn):
    return j if j < S else S + (j - S) % Wn


def _compact_caches(x, n_ctx):
    """Host-built compact caches holding the same tokens as the full cache: retrieval heads'
    whole history, local heads' sinks and last `window` tokens at their ring rows."""
    torch = _torch()
    cfg = x.cfg
    S, Wn = cfg.n_sinks, cfg.window
    ret = [g for g in range(cfg.n_kv_heads) if x.kv_role[g]]
    loc = [g for g in range(cfg.n_kv_heads) if not x.kv_role[g]]
    kr, vr = x.k[:, ret], x.v[:, ret]
    rows = S + Wn
    kl = np.zeros((cfg.batch, len(loc), rows, cfg.head_dim), np.uint16)
    vl = np.zeros_like(kl)
    toks = list(range(min(S, n_ctx))) + list(range(max(n_ctx - Wn, min(S, n_ctx)), n_ctx))
    for j in toks:
        kl[:, :, _ring_slot(j, S, Wn)] = x.k[:, loc, j]
        vl[:, :, _ring_slot(j, S, Wn)] = x.v[:, loc, j]
    dev = lambda a: rtp.to_device_bf16(np.ascontiguousarray(a))
    return dev(kr), dev(vr), dev(kl), dev(vl)


def _layer_kind(cfg, layout, n_cap=None):
    return rtp.Layer(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx if n_cap is None else n_cap,
                     cfg.kv_role.tolist(), cfg.n_sinks, cfg.window, kv_layout=layout)


@pytest.mark.parametrize("over", [dict(batch=2, n_ctx=9000), dict(batch=1, n_ctx=1500),
                                  dict(batch=1, n_ctx=7777, window=1000, n_sinks=3)])
@pytest.mark.parametrize("fused", [True, False])
def test_compact_layout_matches_full(over, fused):
    """Retrieval-only full cache + local ring give the same bits as the full layout
    (ring partly filled, and wrapped several times)."""
    P.require_gpu()
    torch = _torch()
    x, d = _inputs("decode_b8_32k", **over)
    cfg = x.cfg
    B, R = cfg.batch, cfg.n_kv_r * cfg.group
    kr, vr, kl, vl = _compact_caches(x, cfg.n_ctx)
    res = []
    for layout in (rtp.KV_FULL, rtp.KV_COMPACT):
        L = _layer_kind(cfg, layout)
        step = rtp.DecodeStep(L, cfg.n_ctx, 0.95, fused=fused)
        if layout == rtp.KV_FULL:
            step.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)
        else:
            step.run(d.q_pre, d.q, kr, vr, d.k_idx, d.w_q_idx, k_loc=kl, v_loc=vl)
        torch.cuda.synchronize()
        res.append(_step_outputs(step, B, R, cfg.n_ctx))
    _assert_same(res[0], res[1], f"compact vs full {over}")


def test_append_then_decode_both_layouts():
    """Generate steps: append the next token into a full and a compact cache, then run the
    fused step on each.  Rows are copied exactly, the indexer keys are the bf16 of the
    projection within one bf16 ulp plus the fp32 bound, and both layouts give the same
    bits at every step; the first step is checked against the oracle."""
    P.require_gpu()
    torch = _torch()
    x, d = _inputs("decode_b8_32k", batch=2, n_ctx=6000, window=512)
    cfg = x.cfg
    B, R, D, Hkv = cfg.batch, cfg.n_kv_r * cfg.group, cfg.head_dim, cfg.n_kv_heads
    n0, T = cfg.n_ctx - 6, 6
    rng = np.random.default_rng(5)
    k_pre_new = W.f32_to_bf16_bits(rng.standard_normal((T, B, Hkv, D)).astype(np.float32))
    w_k = x.w_k_idx
    # full layout: the generator's caches with the last T rows cleared; compact: built at n0
    k_full, v_full = x.k.copy(), x.v.copy()
    k_full[:, :, n0:] = 0
    v_full[:, :, n0:] = 0
    kidx = x.k_idx.copy()
    kidx[:, :, n0:] = 0
    dev = lambda a: rtp.to_device_bf16(np.ascontiguousarray(a))
    kf, vf, kidx_f, kidx_c = dev(k_full), dev(v_full), dev(kidx), dev(kidx)
    xc = type("X", (), {})()
    xc.cfg, xc.k, xc.v, xc.kv_role = cfg, k_full, v_full, x.kv_role
    kr, vr, kl, vl = _compact_caches(xc, n0)
    Lf, Lc = _layer_kind(cfg, rtp.KV_FULL), _layer_kind(cfg, rtp.KV_COMPACT)
    sf, sc = rtp.DecodeStep(Lf, cfg.n_ctx, 0.95), rtp.DecodeStep(Lc, cfg.n_ctx, 0.95)
    ret = [g for g in range(Hkv) if x.kv_role[g]]
    for t in range(T):
        pos = n0 + t
        k_new, v_new = dev(x.k[:, :, pos]), dev(x.v[:, :, pos])
        kp = dev(k_pre_new[t])
        rtp.rtp_append_token(Lf, pos, k_new, v_new, kp, dev(w_k), D * 16, kf, vf, kidx_f)
        rtp.rtp_append_token(Lc, pos, k_new, v_new, kp, dev(w_k), D * 16, kr, vr, kidx_c, kl, vl)
        sf.run(d.q_pre, d.q, kf, vf, kidx_f, d.w_q_idx, n_ctx=pos + 1)
        sc.run(d.q_pre, d.q, kr, vr, kidx_c, d.w_q_idx, n_ctx=pos + 1, k_loc=kl, v_loc=vl)
        torch.cuda.synchronize()
        _assert_same(_step_outputs(sf, B, R, pos + 1), _step_outputs(sc, B, R, pos + 1), f"step {t}")
        got_k = rtp.from_device_bf16(kf).reshape(B, Hkv, -1, D)[:, :, pos]
        assert np.array_equal(got_k, x.k[:, :, pos])
        gi = rtp.from_device_bf16(kidx_f).reshape(B, cfg.n_kv_r, -1, 16)[:, :, pos]
        for b in range(B):
            for r, g in enumerate(ret):
                a = O.bf16_to_f64(k_pre_new[t, b, g])
                wr = O.bf16_to_f64(w_k[r])
                exact = a @ wr
                allow = P.bf16_ulp(exact) + 1e-6 * (np.abs(a) @ np.abs(wr))
                assert np.all(np.abs(O.bf16_to_f64(gi[b, r]) - exact) <= allow)
        assert np.array_equal(gi, rtp.from_device_bf16(kidx_c).reshape(B, cfg.n_kv_r, -1, 16)[:, :, pos])
        if t == 0:                                         # the first step against the oracle (local rows)
            kk = k_full.copy()
            kk[:, :, pos] = x.k[:, :, pos]
            vv = v_full.copy()
            vv[:, :, pos] = x.v[:, :, pos]
            g_out = rtp.from_device_bf16(sf.out).reshape(B, cfg.n_q_heads, D)
            lset = O.local_set(pos + 1, cfg.n_sinks, cfg.window)
            for b in range(B):
                for h in range(cfg.n_q_heads):
                    if x.kv_role[h // cfg.group]:
                        continue
                    ref = O.attend(O.bf16_to_f64(x.q[b, h]), O.bf16_to_f64(kk[b, h // cfg.group, :pos + 1]),
                                   O.bf16_to_f64(vv[b, h // cfg.group, :pos + 1]), lset, 1 / math.sqrt(D))
                    P.check_outputs(g_out[b, h][None], ref[None], f"local row ({b},{h}) after append")


# ----------------------------------------------------------------------------- indexer dimensions
@pytest.mark.parametrize("idx_dim", [4, 8, 32])
def test_decode_step_other_indexer_dims(idx_dim):
    """The separate calls with indexer dimensions 4 / 8 / 32 against the oracle (the fused
    call takes 16 only and says so)."""
    P.require_gpu()
    x, d = _inputs("decode_b8_32k", batch=2, n_ctx=9000, idx_dim=idx_dim)
    cfg = x.cfg
    L = P.layer_for(cfg)
    with pytest.raises(rtp.RtpError, match="idx_dim"):
        rtp.DecodeStep(L, cfg.n_ctx, cfg.top_p, fused=True).run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)
    step = rtp.DecodeStep(L, cfg.n_ctx, cfg.top_p, fused=False)
    out = step.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)
    _torch().cuda.synchronize()
    N, B, G = cfg.n_ctx, cfg.batch, cfg.group
    R = cfg.n_kv_r * G
    ora = O.decode_step(x.q_pre, x.q, x.k, x.v, x.k_idx, x.w_q_idx, x.kv_role, N, cfg.top_p, cfg.n_sinks, cfg.window)
    g = rtp.from_device_bf16(out).reshape(B, cfg.n_q_heads, cfg.head_dim)
    cnt = step.sel_count.view(B, R).cpu().numpy()
    sel = step.sel_idx.view(B, R, N).cpu().numpy()
    same_all = 0
    for b in range(B):
        for ci in range(R):
            r = ci // G
            same, _ = P.check_set(sel[b, ci, :cnt[b, ci]], ora["info"][(b, ci)], cfg.top_p, ora["scores"][(b, ci)],
                                  P.FP32_SCORE_SLACK * P.score_scale(x, b, ci, r, N))
            h = cfg.retrieval_kv[r] * G + ci % G
            P.check_retrieval_row(g[b, h], x, b, h, sel[b, ci, :cnt[b, ci]], N, same, ora["out"][b, h],
                                  f"row ({b},{h})")
            same_all += same
    assert same_all >= 0.9 * B * R
    loc = [gg * G + t for gg in range(cfg.n_kv_heads) if not x.kv_role[gg] for t in range(G)]
    P.check_outputs(g[:, loc], ora["out"][:, loc], "local rows")


# ----------------------------------------------------------------------------- long generation (device length)
def _check_step_against_oracle(x, cfg, n, k_full, v_full, kidx, out_bits, sel, cnt, gsc, p, what):
    """Every row of a decode step at context n against the oracle on the given caches."""
    B, G = cfg.batch, cfg.group
    R = cfg.n_kv_r * G
    ora = O.decode_step(x.q_pre, x.q, k_full, v_full, kidx, x.w_q_idx, x.kv_role, n, p, cfg.n_sinks, cfg.window)
    ob = np.asarray(out_bits).reshape(B, cfg.n_q_heads, cfg.head_dim)
    xs = type("X", (), {})()
    xs.cfg, xs.q, xs.k, xs.v = cfg, x.q, k_full, v_full
    same_all = 0
    for b in range(B):
        for ci in range(R):
            r = ci // G
            s_g = sel[b, ci, :cnt[b, ci]]
            P.check_prefix(s_g, gsc[b, ci, :n], f"{what} row ({b},{ci})")
            qi = O.indexer_query(O.bf16_to_f64(x.q_pre[b, cfg.retrieval_kv[r] * G + ci % G]),
                                 O.bf16_to_f64(x.w_q_idx[ci]))
            scale = np.abs(O.bf16_to_f64(kidx[b, r, :n])) @ np.abs(qi)
            same, _ = P.check_set(s_g, ora["info"][(b, ci)], p, ora["scores"][(b, ci)], P.FP32_SCORE_SLACK * scale)
            h = cfg.retrieval_kv[r] * G + ci % G
            P.check_retrieval_row(ob[b, h], xs, b, h, s_g, n, same, ora["out"][b, h], f"{what} retrieval row ({b},{h})")
            same_all += same
    loc = [gg * G + t for gg in range(cfg.n_kv_heads) if not x.kv_role[gg] for t in range(G)]
    P.check_outputs(ob[:, loc], ora["out"][:, loc], f"{what} local rows")
    return same_all


@pytest.mark.parametrize("layout", [rtp.KV_COMPACT, rtp.KV_FULL])
def test_generation_graph_with_device_length(layout):
    """Long generation (NEXT-3): [rtp_append_token_dev, rtp_decode_step_dev] captured once in a
    HIP graph and replayed for 10 tokens.  The context length lives in the device state
    {pos, n_ctx}, which every replay advances; after every replay, every retrieval and local
    row is checked against the oracle on the grown caches, and the appended indexer key
    against the exact projection."""
    P.require_gpu()
    torch = _torch()
    x, d = _inputs("decode_b8_32k", batch=2, n_ctx=6000, window=512)
    cfg = x.cfg
    B, R, D, Hkv, G = cfg.batch, cfg.n_kv_r * cfg.group, cfg.head_dim, cfg.n_kv_heads, cfg.group
    T = 10
    n0 = cfg.n_ctx - T
    p = 0.95
    rng = np.random.default_rng(21)
    k_pre_new = W.f32_to_bf16_bits(rng.standard_normal((T, B, Hkv, D)).astype(np.float32))
    k_full, v_full = x.k.copy(), x.v.copy()
    k_full[:, :, n0:] = 0
    v_full[:, :, n0:] = 0
    kidx = x.k_idx.copy()
    kidx[:, :, n0:] = 0
    dev = lambda a: rtp.to_device_bf16(np.ascontiguousarray(a))
    L = _layer_kind(cfg, layout)
    if layout == rtp.KV_COMPACT:
        xc = type("X", (), {})()
        xc.cfg, xc.k, xc.v, xc.kv_role = cfg, k_full, v_full, x.kv_role
        kc, vc, kl, vl = _compact_caches(xc, n0)
    else:
        kc, vc, kl, vl = dev(k_full), dev(v_full), None, None
    kidx_d = dev(kidx)
    w_k = dev(x.w_k_idx)
    step = rtp.DecodeStep(L, cfg.n_ctx, p)                      # grids and strides for the bound n0 + T
    gen = torch.tensor([n0, n0], dtype=torch.int64, device="cuda")
    knew = torch.empty(B * Hkv * D, dtype=torch.bfloat16, device="cuda")
    vnew, kpre = torch.empty_like(knew), torch.empty_like(knew)

    def fill(t):
        knew.copy_(dev(x.k[:, :, n0 + t]).view(-1))
        vnew.copy_(dev(x.v[:, :, n0 + t]).view(-1))
        kpre.copy_(dev(k_pre_new[t]).view(-1))

    def pair():
        rtp.rtp_append_token_dev(L, gen, knew, vnew, kpre, w_k, D * 16, kc, vc, kidx_d, kl, vl)
        step.run_dev(gen, d.q_pre, d.q, kc, vc, kidx_d, d.w_q_idx, k_loc=kl, v_loc=vl)

    fill(0)
    pair()                                                      # eager run of token 0 (re-appended below)
    torch.cuda.synchronize()
    gen.copy_(torch.tensor([n0, n0], dtype=torch.int64))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pair()
    torch.cuda.synchronize()
    ret = [gg for gg in range(Hkv) if x.kv_role[gg]]
    identical = 0
    for t in range(T):
        fill(t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        n = n0 + t + 1
        assert gen.cpu().tolist() == [n, n], f"state after token {t}: {gen.cpu().tolist()}"
        k_full[:, :, n - 1] = x.k[:, :, n - 1]
        v_full[:, :, n - 1] = x.v[:, :, n - 1]
        gi = rtp.from_device_bf16(kidx_d).reshape(B, cfg.n_kv_r, -1, 16)[:, :, n - 1]
        for b in range(B):
            for r, gg in enumerate(ret):
                a = O.bf16_to_f64(k_pre_new[t, b, gg])
                wr = O.bf16_to_f64(x.w_k_idx[r])
                exact = a @ wr
                allow = P.bf16_ulp(exact) + 1e-6 * (np.abs(a) @ np.abs(wr))
                assert np.all(np.abs(O.bf16_to_f64(gi[b, r]) - exact) <= allow)
        kidx[:, :, n - 1] = gi
        cnt = step.sel_count.view(B, R).cpu().numpy()
        sel = step.sel_idx.view(B, R, -1).cpu().numpy()
        gsc = step.scores.view(B, R, -1).cpu().numpy()
        assert np.all((cnt >= 1) & (cnt <= n)), f"token {t}: counts {cnt}"
        identical += _check_step_against_oracle(x, cfg, n, k_full, v_full, kidx, rtp.from_device_bf16(step.out), sel,
                                                cnt, gsc, p, f"token {t}")
    assert identical >= 0.9 * T * B * R
