"""The allocation-free decode step (rtp_decode_step_noalloc) against rtp_decode_step.

Both run the same launches; the allocation-free one keeps its scratch in the library's
own device array, which holds whatever the previous call on the GPU left there.  Two
calls in a row, the second on a smaller layer and context, then the first again: every
output must equal the workspace call's bit for bit.
"""
import math

import numpy as np
import pytest

from head_wise_sparse_amd import rtp
from head_wise_sparse_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def _outputs(B, R, n, cap, scores, row_max, row_sum, sel_idx, sel_count, sel_starts, out):
    nsplit = (n + rtp.SEL_RANGE - 1) // rtp.SEL_RANGE
    cnt = sel_count.cpu().numpy()
    sel = sel_idx.view(B * R, cap).cpu().numpy()
    return dict(scores=scores.view(B * R, cap)[:, :n].cpu().numpy(), row_max=row_max.cpu().numpy(),
                row_sum=row_sum.cpu().numpy(), cnt=cnt, sets=[sel[i, :cnt[i]].copy() for i in range(B * R)],
                starts=sel_starts[:B * R * (nsplit + 1)].cpu().numpy(), out=rtp.from_device_bf16(out))


def _case(over, p):
    import torch
    cfg = W.scaled_decode(W.CONFIGS["decode_b8_32k"], **over)
    x = W.make_decode_inputs(cfg)
    d = P.DeviceDecode(x)
    L = P.layer_for(cfg)
    n, B, R, cap = cfg.n_ctx, cfg.batch, cfg.n_kv_r * cfg.group, cfg.n_ctx
    step = rtp.DecodeStep(L, n, p)                       # the workspace entry point
    step.run(d.q_pre, d.q, d.k, d.v, d.k_idx, d.w_q_idx)
    torch.cuda.synchronize()
    ref = _outputs(B, R, n, cap, step.scores, step.row_max, step.row_sum, step.sel_idx, step.sel_count,
                   step.sel_starts, step.out)
    nsplit = (cap + rtp.SEL_RANGE - 1) // rtp.SEL_RANGE
    f32 = lambda k: torch.full((k,), float("nan"), dtype=torch.float32, device="cuda")
    i32 = lambda k: torch.full((k,), -5, dtype=torch.int32, device="cuda")
    scores, row_max, row_sum = f32(B * R * cap), f32(B * R), f32(B * R)
    sel_idx, sel_count, sel_starts = i32(B * R * cap), i32(B * R), i32(B * R * (nsplit + 1))
    out = torch.zeros(B * cfg.n_q_heads * cfg.head_dim, dtype=torch.bfloat16, device="cuda")
    print(f"\nno-alloc step: batch {B}, n_ctx {n}, p {p}", flush=True)
    rtp.rtp_decode_step_noalloc(L, n, d.q_pre, d.w_q_idx, cfg.head_dim * 16, d.k_idx, 1.0, d.q, d.k, d.v, None, None,
                                p, 1 / math.sqrt(cfg.head_dim), scores, row_max, row_sum, sel_idx, sel_count,
                                sel_starts, out)
    torch.cuda.synchronize()
    got = _outputs(B, R, n, cap, scores, row_max, row_sum, sel_idx, sel_count, sel_starts, out)
    for k in ("scores", "row_max", "row_sum", "cnt", "starts", "out"):
        assert np.array_equal(got[k].view(np.uint8), ref[k].view(np.uint8)), f"{k} differs (batch {B}, n_ctx {n})"
    for a, b in zip(got["sets"], ref["sets"]):
        assert np.array_equal(a, b)


def test_noalloc_matches_workspace_call():
    P.require_gpu()
    _case(dict(batch=2, n_ctx=9000), 0.95)
    _case(dict(batch=1, n_ctx=3000, n_sinks=7, window=700), 0.9)      # smaller layer and context
    _case(dict(batch=2, n_ctx=9000), 0.95)                              # and the first one again


def test_noalloc_rejects_layers_beyond_its_scratch():
    P.require_gpu()
    L = rtp.Layer(8, 32, 8, 128, 1 << 20, [1, 0, 0, 1, 0, 0, 0, 0], 4, 8192)
    need = rtp.rtp_workspace_bytes(L, 1 << 20, rtp.CALL_DECODE_STEP)
    assert need > rtp.rtp_decode_step_noalloc_max_bytes()
    lib = rtp.load()
    fake = 0x10000000
    st = lib.rtp_decode_step_noalloc(L.desc, 1 << 20, fake, fake, 0, fake, 1.0, fake, fake, fake, None, None, 0.9,
                                     0.1, fake, fake, fake, fake, fake, None, fake, None)
    assert st == rtp.RTP_EUNSUPPORTED
    assert "scratch" in lib.rtp_last_error().decode()
