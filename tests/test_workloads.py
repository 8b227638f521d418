"""Checks of the seeded input generator (shapes, determinism, bf16 rounding, RoPE, needles)."""
import math

import numpy as np
import torch

from head_wise_sparse_amd import workloads as W
from oracle import rtp_oracle as O


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * 37
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(x), ref)
    assert np.array_equal(W.bf16_bits_to_f32(ref), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_rope_rotation_properties():
    rng = np.random.default_rng(1)
    x = W.f32_to_bf16_bits(rng.standard_normal((4, 64)).astype(np.float32))
    assert np.array_equal(W._rope_bf16(x, np.zeros(4, np.int64)), x)          # position 0: identity
    y = W.bf16_bits_to_f32(W._rope_bf16(x, np.array([5, 77, 1000, 123456])))
    n0 = np.linalg.norm(W.bf16_bits_to_f32(x), axis=1)
    assert np.allclose(np.linalg.norm(y, axis=1), n0, rtol=1e-2)            # a rotation (up to bf16)


def test_tiny_decode_inputs_shapes_and_determinism():
    cfg = W.CONFIGS["decode_tiny_2k"]
    a = W.make_decode_inputs(cfg)
    b = W.make_decode_inputs(cfg)
    assert a.q.shape == (1, 4, 64) and a.k.shape == (1, 2, 2048, 64) and a.k_idx.shape == (1, 1, 2048, 16)
    assert a.w_q_idx.shape == (2, 64, 16) and a.w_k_idx.shape == (1, 64, 16)
    for name in ["q_pre", "q", "k", "v", "k_idx", "w_q_idx", "needle_pos"]:
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    assert a.kv_role.tolist() == [1, 0]
    assert len(np.unique(a.needle_pos[0, 0])) == 8
    # the needle rule: the needle's indexer key is 4x the mean query indexer vector of the group
    qi = [W.bf16_bits_to_f32(a.q_pre[0, t]).astype(np.float64) @ W.bf16_bits_to_f32(a.w_q_idx[t]).astype(np.float64)
          for t in range(2)]
    needle = W.bf16_bits_to_f32(a.k_idx[0, 0, a.needle_pos[0, 0, 0]])
    assert np.allclose(needle, 4 * np.mean(qi, axis=0), rtol=1e-2, atol=1e-2)


def test_tiny_config_is_peaked_on_needles():
    """The planted needles carry most of the indexer mass (what makes retrieval heads sparse)."""
    cfg = W.CONFIGS["decode_tiny_2k"]
    x = W.make_decode_inputs(cfg)
    res = O.decode_step(x.q_pre, x.q, x.k, x.v, x.k_idx, x.w_q_idx, x.kv_role, cfg.n_ctx, cfg.top_p,
                        cfg.n_sinks, cfg.window)
    for (b, ci), sel in res["sel"].items():
        assert len(sel) < cfg.n_ctx // 4
        assert set(x.needle_pos[0, 0].tolist()) & set(sel.tolist())


def test_prefill_chunks_regenerate_identically():
    cfg = W.scaled_prefill(W.CONFIGS["prefill_32k"], seq_len=600, chunk=256, rows_per_head=8)
    p = W.PrefillInputs(cfg)
    k, v, kp = p.full_kv()
    assert k.shape == (8, 600, 128) and kp.shape == (600, 8, 128)
    assert np.array_equal(p.k_chunk(2), k[:, 512:600])
    assert np.array_equal(p.q_chunk(1)[:, 3], p.q_chunk(1, heads=[3])[:, 3])
    assert np.array_equal(p.q_chunk(1)[:, 3], p.q_head(1, 3))
    rows = p.sample_rows(0)
    assert len(rows) == 8 and rows.min() >= 0 and rows.max() < 600
