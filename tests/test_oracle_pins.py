"""Pins for the fp64 oracle: what the pages and the mathematics fix, checked on the CPU.

Each test checks the oracle against something other than itself: brute-force
enumeration, hand-worked closed forms (tests/golden/), library routines
(torch float64 scaled_dot_product_attention, torch's bf16 cast) or exact
special cases (p = 1, window >= N, q = 0).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import rtp_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- bf16 rounding
def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_f64_to_bf16_matches_torch_rne_on_float32_values():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-5, 6, 200000)
    # exact halfway cases between neighbouring bf16 values, both parities
    base = rng.standard_normal(5000).astype(np.float32)
    hb = (base.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, hb.view(np.float32), np.float32([0.0, -0.0, 1.0, -2.5])])
    assert np.array_equal(O.f64_to_bf16(x.astype(np.float64)), _torch_bf16_bits(x))


def test_bf16_upcast_exact():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]       # finite only
    f = O.bf16_to_f64(bits)
    back = torch.from_numpy(f.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(back, bits)


# ----------------------------------------------------------------------------- indexer scores
def test_scores_closed_form_and_bilinear():
    rng = np.random.default_rng(2)
    q_pre = rng.integers(-3, 4, 64).astype(np.float64)
    w = np.zeros((64, 16))
    w[np.arange(16), np.arange(16)] = 1.0              # W picks the first 16 coordinates
    qi = O.indexer_query(q_pre, w)
    assert np.array_equal(qi, q_pre[:16])
    # k_idx rows that are multiples of q_idx: s_j = c_j * |q_idx|^2 exactly
    c = np.array([0.0, 1.0, -2.0, 4.0, 0.5])
    k = c[:, None] * qi[None, :]
    s = O.indexer_scores(qi, k)
    assert np.array_equal(s, c * float(qi @ qi))
    # idx_scale multiplies, and scores are linear in k
    k2 = rng.integers(-4, 5, (7, 16)).astype(np.float64)
    assert np.allclose(O.indexer_scores(qi, k2, 0.25), 0.25 * O.indexer_scores(qi, k2))
    assert np.allclose(O.indexer_scores(qi, k2 + k2), 2 * O.indexer_scores(qi, k2))


def test_scores_ignore_token_position():
    """Pre-RoPE indexer: moving a key to another slot moves its score with it."""
    rng = np.random.default_rng(3)
    qi = rng.standard_normal(16)
    k = rng.standard_normal((50, 16))
    perm = rng.permutation(50)
    assert np.array_equal(O.indexer_scores(qi, k[perm]), O.indexer_scores(qi, k)[perm])


# ----------------------------------------------------------------------------- top-p rule
def test_topp_golden_closed_form():
    with open(os.path.join(GOLDEN, "topp_closed_form.json")) as f:
        rows = json.load(f)["rows"]
    e = math.e
    for r in rows:
        sel, info = O.topp_select(np.array(r["scores"], np.float64), r["p"])
        assert sel.tolist() == r["expect"], r
        cum = eval(r["cum"], {"e": e})                       # closed form, math only
        assert abs(info["cum"][len(sel) - 1] - cum) < 1e-12, r
        if len(sel) < len(r["scores"]):
            assert cum >= r["p"]


def _brute_force_min_card(pi: np.ndarray, p: float):
    n = pi.size
    for k in range(1, n + 1):
        best = max(math.fsum(pi[list(c)]) for c in itertools.combinations(range(n), k))
        if best >= p:
            return k
    return n


@pytest.mark.parametrize("seed", range(40))
def test_topp_brute_force_minimal_set(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 11))
    # integer scores make ties common; a few rows use continuous scores
    s = rng.integers(-3, 4, n).astype(np.float64) if seed % 3 else rng.standard_normal(n) * 2
    ex = np.exp(s)
    pi = ex / math.fsum(ex.tolist())                         # independent softmax, no max shift
    p = float(rng.uniform(0.05, 0.999))
    masses = [math.fsum(pi[list(c)]) for k in range(1, n + 1) for c in itertools.combinations(range(n), k)]
    if min(abs(m - p) for m in masses) < 1e-9:
        pytest.skip("p too close to a subset mass")
    sel, info = O.topp_select(s, p)
    k = _brute_force_min_card(pi, p)
    assert len(sel) == k
    assert math.fsum(pi[sel].tolist()) >= p
    # the kept tokens outrank every dropped token: higher score, or equal score and lower index
    dropped = np.setdiff1d(np.arange(n), sel)
    for j in sel:
        for d in dropped:
            assert s[j] > s[d] or (s[j] == s[d] and j < d)


def test_topp_invariants():
    rng = np.random.default_rng(4)
    for trial in range(30):
        n = int(rng.integers(1, 3000))
        s = rng.standard_normal(n) * rng.uniform(0.1, 8)
        if trial % 4 == 0:
            s = np.round(s)                                  # many exact ties
        ps = np.sort(rng.uniform(0.01, 0.999, 5))
        sets = [set(O.topp_select(s, p)[0].tolist()) for p in ps]
        for a, b in zip(sets, sets[1:]):
            assert a <= b                                    # monotone in p
        p = float(ps[2])
        sel, info = O.topp_select(s, p)
        k = len(sel)
        assert info["cum"][k - 1] >= p and (k == 1 or info["cum"][k - 2] < p)   # minimal prefix
        # shift invariance (a constant added to every score changes no softmax mass)
        assert np.array_equal(O.topp_select(s + 3.0, p)[0], sel)
        assert np.array_equal(O.topp_select(s, 1.0)[0], np.arange(n))            # p = 1 keeps all
        am = int(np.flatnonzero(s == s.max())[0])
        assert O.topp_select(s, 1e-12)[0].tolist() == [am]                     # p -> 0: argmax, lowest index


def test_topp_rejects_nonpositive_p():
    with pytest.raises(ValueError):
        O.topp_select(np.zeros(3), 0.0)


def test_exempt_rule_and_set_mass():
    s = np.array([2.0, 1.0, 0.0, 0.0])
    sel, info = O.topp_select(s, 0.7)
    assert abs(O.set_mass(info, sel) - info["cum"][1]) < 1e-15
    ex = O.exempt_ranks(info, info["cum"][1], 1e-4)          # p exactly on a prefix mass
    assert set(ex.tolist()) == {1, 2}                        # rank ending at p, and rank starting at p


# ----------------------------------------------------------------------------- local set
def test_local_set_special_cases():
    assert O.local_set(10, 0, 1).tolist() == [9]                    # window 1: the query token only
    assert O.local_set(10, 3, 1).tolist() == [0, 1, 2, 9]
    assert O.local_set(10, 4, 100).tolist() == list(range(10))      # window >= N: dense
    assert O.local_set(5, 8, 2).tolist() == list(range(5))          # sinks beyond N are truncated
    assert O.local_set(10, 4, 7).tolist() == list(range(10))        # overlap counted once
    assert len(O.local_set(1000, 4, 256)) == 4 + 256


# ----------------------------------------------------------------------------- attention
def _sdpa64(q, k, v, mask=None, is_causal=False, scale=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q)[None, None], t(k)[None, None], t(v)[None, None],
        attn_mask=None if mask is None else torch.from_numpy(mask)[None, None],
        is_causal=is_causal, scale=scale)
    return out[0, 0].numpy()


def _bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return _torch_bf16_bits(x)


def _decode_inputs(rng, B=2, Hq=4, Hkv=2, D=32, N=300, qscale=1.0):
    q_pre = _bits(rng, (B, Hq, D), qscale)
    q = _bits(rng, (B, Hq, D), qscale)
    k = _bits(rng, (B, Hkv, N, D))
    v = _bits(rng, (B, Hkv, N, D))
    k_idx = _bits(rng, (B, 1, N, 16))
    w = _bits(rng, (Hq // Hkv, D, 16), 1 / math.sqrt(D))
    return q_pre, q, k, v, k_idx, w, np.array([1, 0], np.uint8)


def test_decode_p1_and_wide_window_equal_dense_sdpa():
    rng = np.random.default_rng(5)
    q_pre, q, k, v, k_idx, w, role = _decode_inputs(rng)
    N = k.shape[2]
    res = O.decode_step(q_pre, q, k, v, k_idx, w, role, N, 1.0, 4, N + 5)
    D = q.shape[-1]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            g = h // 2
            ref = _sdpa64(O.bf16_to_f64(q[b, h])[None], O.bf16_to_f64(k[b, g]), O.bf16_to_f64(v[b, g]),
                          scale=1 / math.sqrt(D))[0]
            assert np.allclose(res["out"][b, h], ref, rtol=1e-12, atol=1e-12)


def test_decode_zero_query_gives_mean_of_attended_values():
    rng = np.random.default_rng(6)
    q_pre, q, k, v, k_idx, w, role = _decode_inputs(rng, N=500)
    q[:] = 0                                                   # post-RoPE q = 0: uniform attention
    N, S, W = 500, 4, 37
    res = O.decode_step(q_pre, q, k, v, k_idx, w, role, N, 0.8, S, W)
    for b in range(2):
        for h in range(4):
            g = h // 2
            vv = O.bf16_to_f64(v[b, g])
            if role[g]:
                sel = res["sel"][(b, h % 2)]
                assert len(sel) < N
                exp = vv[sel].mean(axis=0)
            else:
                exp = np.concatenate([vv[:S], vv[N - W:]]).mean(axis=0)   # 4 sinks + last 37, disjoint
            assert np.allclose(res["out"][b, h], exp, rtol=1e-12, atol=1e-12)


def test_decode_dominant_logit_returns_that_value_row():
    rng = np.random.default_rng(7)
    D, N = 32, 64
    q = rng.standard_normal(D)
    k = rng.standard_normal((N, D)) * 0.01
    k[17] = 50 * q / np.linalg.norm(q)
    v = rng.standard_normal((N, D))
    o = O.attend(q, k, v, np.arange(N), 1.0)
    assert np.allclose(o, v[17], atol=1e-12)


def test_decode_retrieval_set_is_topp_of_indexer_scores():
    rng = np.random.default_rng(8)
    q_pre, q, k, v, k_idx, w, role = _decode_inputs(rng, N=256, qscale=3.0)
    res = O.decode_step(q_pre, q, k, v, k_idx, w, role, 256, 0.9, 4, 32)
    for (b, ci), sel in res["sel"].items():
        qi = O.bf16_to_f64(q_pre[b, ci]) @ O.bf16_to_f64(w[ci])      # head ci of KV head 0
        s = O.bf16_to_f64(k_idx[b, 0]) @ qi
        assert np.array_equal(O.topp_select(s, 0.9)[0], sel)
        assert res["info"][(b, ci)]["cum"][len(sel) - 1] >= 0.9


# ----------------------------------------------------------------------------- prefill
def test_prefill_retrieval_rows_equal_causal_sdpa():
    rng = np.random.default_rng(9)
    T, D = 200, 32
    q, k, v = _bits(rng, (T, D)), _bits(rng, (T, D)), _bits(rng, (T, D))
    rows = np.array([0, 1, 5, 63, 64, 199])
    got = O.prefill_rows(q[rows], rows, k, v, True, 4, 16)
    ref = _sdpa64(O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v), is_causal=True, scale=1 / math.sqrt(D))
    assert np.allclose(got, ref[rows], rtol=1e-12, atol=1e-12)
    # local heads with a window covering the sequence are the same causal attention
    got_l = O.prefill_rows(q[rows], rows, k, v, False, 4, T)
    assert np.allclose(got_l, ref[rows], rtol=1e-12, atol=1e-12)


def test_prefill_local_rows_equal_banded_sdpa():
    rng = np.random.default_rng(10)
    T, D, S, W = 180, 32, 3, 20
    q, k, v = _bits(rng, (T, D)), _bits(rng, (T, D)), _bits(rng, (T, D))
    ones = torch.ones(T, T, dtype=torch.bool)
    causal = torch.tril(ones)
    band = causal & ~torch.tril(ones, diagonal=-W)            # keys i-W+1 .. i
    sink_cols = torch.zeros(T, T, dtype=torch.bool)
    sink_cols[:, :S] = True
    mask = (band | (sink_cols & causal)).numpy()
    ref = _sdpa64(O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v), mask=mask, scale=1 / math.sqrt(D))
    rows = np.arange(T)
    got = O.prefill_rows(q, rows, k, v, False, S, W)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_prefill_local_row_matches_decode_local_head():
    """Prefill row i of a local head sees what a decode step with n_ctx = i+1 sees."""
    rng = np.random.default_rng(11)
    T, D, S, W = 90, 16, 2, 11
    q_pre = np.zeros((1, 2, D), np.uint16)
    k = _bits(rng, (1, 1, T, D))
    v = _bits(rng, (1, 1, T, D))
    qrow = _bits(rng, (1, 2, D))
    role = np.array([0], np.uint8)
    for i in [0, 1, 2, 5, 11, 12, 13, 40, 89]:
        dec = O.decode_step(q_pre, qrow, k[:, :, :i + 1], v[:, :, :i + 1], np.zeros((1, 0, i + 1, 16), np.uint16),
                            np.zeros((0, D, 16), np.uint16), role, i + 1, 0.9, S, W)
        pre = O.prefill_rows(qrow[0, :1], [i], k[0, 0], v[0, 0], False, S, W)
        assert np.allclose(dec["out"][0, 0], pre[0], rtol=1e-13, atol=1e-13)


def test_prefill_kidx_is_bf16_of_fp64_projection():
    rng = np.random.default_rng(12)
    C, Hkv, D = 257, 3, 64
    k_pre = _bits(rng, (C, Hkv, D))
    w = _bits(rng, (2, D, 16), 1 / 8)
    role = np.array([1, 0, 1], np.uint8)
    got = O.prefill_kidx(k_pre, w, role)
    assert got.shape == (2, C, 16)
    for r, g in enumerate([0, 2]):
        exact = torch.from_numpy(O.bf16_to_f64(k_pre[:, g])) @ torch.from_numpy(O.bf16_to_f64(w[r]))
        # torch rounds float64 -> float32 -> bf16; the oracle rounds float64 -> bf16 once.  They can
        # differ only where the float32 step lands exactly on a bf16 halfway point: at most 1 ulp.
        ref = exact.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        diff = np.abs(got[r].astype(np.int64) - ref.astype(np.int64))
        assert diff.max() <= 1 and (diff == 0).mean() > 0.999
        # and the oracle's bf16 value is the nearest bf16 to the exact projection
        e = exact.numpy()
        gv = O.bf16_to_f64(got[r])
        ulp = np.ldexp(1.0, np.frexp(np.abs(e))[1] - 8)
        assert np.all(np.abs(gv - e) <= 0.5 * ulp + 1e-300)


def test_recall_is_one_for_full_set():
    rng = np.random.default_rng(13)
    q = rng.standard_normal(16)
    k = rng.standard_normal((40, 16))
    assert abs(O.attention_recall(q, k, None, 40, np.arange(40), 0.25) - 1.0) < 1e-12
    r = O.attention_recall(q, k, None, 40, np.arange(10), 0.25)
    assert 0.0 < r < 1.0


def test_recall_hand_worked_three_keys():
    """Recall by hand: q = (2 ln 2, 0), keys (1,0), (0,1), (-1,0), sm_scale 1/2 give logits
    ln 2, 0, -ln 2, so softmax weights 2 : 1 : 1/2 of a total 7/2.  The first key holds 4/7 of
    the mass, the first and third 5/7.  With the scale left out (1 instead of 1/2) the weights
    would be 4 : 1 : 1/4 and the first key would hold 16/21, so the scale is pinned."""
    q = np.array([2.0 * math.log(2.0), 0.0])
    k = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0]])
    assert abs(O.attention_recall(q, k, None, 3, np.array([0]), 0.5) - 4.0 / 7.0) < 1e-12
    assert abs(O.attention_recall(q, k, None, 3, np.array([0, 2]), 0.5) - 5.0 / 7.0) < 1e-12
    assert abs(O.attention_recall(q, k, None, 3, np.array([1]), 0.5) - 2.0 / 7.0) < 1e-12
    # only the first n_ctx keys count: with n_ctx = 2 the third key is outside the context
    assert abs(O.attention_recall(q, k, None, 2, np.array([0]), 0.5) - 2.0 / 3.0) < 1e-12


# ----------------------------------------------------------------------------- static top-k
def _ranks_before(s, i, j):
    """Token i ranks before token j: higher score, or equal score and lower index."""
    return s[i] > s[j] or (s[i] == s[j] and i < j)


@pytest.mark.parametrize("seed", range(25))
def test_topk_brute_force(seed):
    """Among all k-subsets exactly one has every member ranked before every non-member;
    the oracle returns that one (ties are frequent: scores are drawn from 4 values)."""
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 10))
    s = rng.choice([-1.0, 0.0, 0.5, 2.0], size=n)
    for k in range(0, n + 2):
        got = O.topk_select(s, k)
        want = [c for c in itertools.combinations(range(n), min(k, n))
                if all(_ranks_before(s, i, j) for i in c for j in set(range(n)) - set(c))]
        assert len(want) == 1
        assert got.tolist() == list(want[0])


def test_topk_invariants_and_topp_prefix():
    rng = np.random.default_rng(7)
    s = np.round(rng.standard_normal(3000) * 2, 1)           # many exact ties
    for k in (1, 17, 500, 2999, 3000, 5000):
        sel = O.topk_select(s, k)
        assert sel.size == min(k, s.size)
        assert np.all(np.diff(sel) > 0)
        if 0 < sel.size < s.size:
            rest = np.setdiff1d(np.arange(s.size), sel)
            assert s[sel].min() >= s[rest].max()
            t = s[sel].min()                                 # boundary score: the lowest indices are kept
            tied_in, tied_out = sel[s[sel] == t], rest[s[rest] == t]
            assert tied_out.size == 0 or tied_in.max() < tied_out.min()
    # the top-p set is a prefix of the same ranking: it is the top-k set with k = |S_p|
    for p in (0.3, 0.9, 0.999):
        sp, _ = O.topp_select(s, p)
        assert np.array_equal(np.sort(sp), O.topk_select(s, sp.size))
