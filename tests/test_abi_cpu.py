"""The C-ABI library on the CPU: it loads, exports every symbol rtp.h declares, sizes
workspaces, and rejects bad arguments on the host before anything is enqueued.

No call here reaches a kernel launch (there is no GPU in this tier): every call
fails host validation, and the fake device pointers are never dereferenced.
"""
import ctypes as C
import math
import os
import re

import pytest

from head_wise_sparse_amd import rtp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000000            # 256-byte aligned stand-in address, never dereferenced


def _lib():
    if not os.path.exists(rtp.LIB_PATH):
        pytest.fail("librtp.so is not built (run python -m head_wise_sparse_amd.build)")
    return rtp.load()


def _declared():
    with open(os.path.join(ROOT, "include", "rtp.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(rtp_\w+)\s*\(", text, re.M)))


def test_header_declarations_are_exported():
    lib = _lib()
    names = _declared()
    assert {"rtp_indexer_score", "rtp_topp_select", "rtp_sparse_decode_attn", "rtp_window_sink_attn",
            "rtp_prefill_attn", "rtp_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(rtp.EXPORTED)


def test_status_strings_and_version():
    lib = _lib()
    assert [lib.rtp_status_string(i).decode() for i in range(5)] == [
        "RTP_OK", "RTP_EINVAL", "RTP_EUNSUPPORTED", "RTP_EWORKSPACE", "RTP_EDEVICE"]
    assert "gfx950" in rtp.rtp_version()


def _layer(**kw):
    d = dict(batch=4, n_q_heads=32, n_kv_heads=8, head_dim=128, n_cap=131072,
             kv_role=[1, 0, 0, 1, 0, 0, 0, 0], n_sinks=4, window=4096)
    d.update(kw)
    return rtp.Layer(**d)


def test_workspace_sizes():
    L = _layer()
    for w in range(6):
        assert rtp.rtp_workspace_bytes(L, 131072 if w != 4 else 4096, w) > 0
    # the selection region does not depend on n_ctx; the fused step holds it first
    assert rtp.rtp_workspace_bytes(L, 1000, rtp.CALL_TOPP_SELECT) == \
        rtp.rtp_workspace_bytes(L, 131072, rtp.CALL_TOPP_SELECT)
    assert rtp.rtp_workspace_bytes(L, 131072, rtp.CALL_DECODE_STEP) >= \
        rtp.rtp_workspace_bytes(L, 131072, rtp.CALL_TOPP_SELECT) + rtp.rtp_workspace_bytes(L, 131072, 0)
    # selection workspace: 3 histogram levels of 2048 (u64 mass + u32 count) per row
    assert rtp.rtp_workspace_bytes(L, 131072, rtp.CALL_TOPP_SELECT) >= 32 * 3 * 2048 * 12
    assert rtp.rtp_workspace_bytes(_layer(head_dim=96), 1000, 0) == 0          # invalid descriptor
    assert rtp.rtp_workspace_bytes(L, 0, 0) == 0
    assert rtp.rtp_workspace_bytes(L, 10, 9) == 0


def _call_step(L, n_ctx=1000, ws_bytes=1 << 30, top_p=0.9, sm=0.1, ptr=FAKE, ws=FAKE):
    lib = _lib()
    return lib.rtp_decode_step(L.desc, n_ctx, ptr, ptr, 0, ptr, 1.0, ptr, ptr, ptr, None, None, top_p, sm, ptr, ptr,
                               ptr, ptr, ptr, None, ptr, ws, ws_bytes, None)


def test_decode_step_validation():
    L = _layer()
    assert _call_step(L, n_ctx=0) == rtp.RTP_EINVAL
    assert _call_step(L, n_ctx=L.n_cap + 1) == rtp.RTP_EINVAL
    for p in (0.0, -1.0, math.nan):
        assert _call_step(L, top_p=p) == rtp.RTP_EINVAL
    assert _call_step(L, sm=math.inf) == rtp.RTP_EINVAL
    assert _call_step(L, ptr=None) == rtp.RTP_EINVAL
    assert _call_step(L, ptr=FAKE + 4) == rtp.RTP_EINVAL
    assert _call_step(L, ws_bytes=1024) == rtp.RTP_EWORKSPACE
    assert _call_step(L, ws=FAKE + 16) == rtp.RTP_EWORKSPACE
    assert "workspace" in _lib().rtp_last_error().decode()
    # the compact layout needs the local ring; prefill needs the full layout
    Lc = _layer(kv_layout=rtp.KV_COMPACT)
    assert _call_step(Lc) == rtp.RTP_EINVAL
    assert lib_prefill_compact() == rtp.RTP_EUNSUPPORTED


def lib_prefill_compact():
    L = _layer(batch=1, n_cap=32768, kv_layout=rtp.KV_COMPACT)
    return _lib().rtp_prefill_attn(L.desc, 0, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0.1, FAKE, FAKE, 1 << 30,
                                   None)


def test_append_validation():
    lib = _lib()
    L = _layer()
    call = lambda L, pos=5, ptr=FAKE, kl=None: lib.rtp_append_token(L.desc, pos, ptr, ptr, ptr, ptr, 0, ptr, ptr, ptr,
                                                                    kl, kl, None)
    assert call(L, pos=-1) == rtp.RTP_EINVAL
    assert call(L, pos=L.n_cap) == rtp.RTP_EINVAL
    assert call(L, ptr=None) == rtp.RTP_EINVAL
    assert call(L, ptr=FAKE + 8) == rtp.RTP_EINVAL
    assert call(_layer(kv_layout=rtp.KV_COMPACT)) == rtp.RTP_EINVAL           # ring missing
    assert call(_layer(kv_layout=2)) == rtp.RTP_EINVAL                        # unknown layout


def _call_score(L, n_ctx=1000, ws_bytes=1 << 20, scale=1.0, ptr=FAKE):
    lib = _lib()
    return lib.rtp_indexer_score(L.desc if L else None, n_ctx, ptr, ptr, 0, ptr, scale, ptr, ptr, ptr,
                                 FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(head_dim=96), rtp.RTP_EUNSUPPORTED, "head_dim"),
    (dict(n_q_heads=30), rtp.RTP_EINVAL, "multiple"),
    (dict(n_q_heads=24, n_kv_heads=2, kv_role=[1, 0]), rtp.RTP_EUNSUPPORTED, "group"),
    (dict(idx_dim=12), rtp.RTP_EUNSUPPORTED, "idx_dim"),
    (dict(idx_dim=32, n_q_heads=64), rtp.RTP_EUNSUPPORTED, "idx_dim 32"),
    (dict(window=0), rtp.RTP_EINVAL, "window"),
    (dict(n_sinks=-1), rtp.RTP_EINVAL, "n_sinks"),
    (dict(batch=0), rtp.RTP_EINVAL, "batch"),
    (dict(n_cap=1 << 30), rtp.RTP_EINVAL, "n_cap"),
    (dict(kv_role=[2, 0, 0, 0, 0, 0, 0, 0]), rtp.RTP_EINVAL, "kv_role"),
])
def test_descriptor_validation(kw, status, msg):
    st = _call_score(_layer(**kw))
    assert st == status
    assert msg in _lib().rtp_last_error().decode()


def test_call_validation():
    lib = _lib()
    L = _layer()
    assert _call_score(None) == rtp.RTP_EINVAL
    assert _call_score(L, n_ctx=0) == rtp.RTP_EINVAL
    assert _call_score(L, n_ctx=L.n_cap + 1) == rtp.RTP_EINVAL
    assert _call_score(L, ws_bytes=16) == rtp.RTP_EWORKSPACE
    assert _call_score(L, scale=math.nan) == rtp.RTP_EINVAL
    assert _call_score(L, ptr=FAKE + 2) == rtp.RTP_EINVAL                      # misaligned
    assert _call_score(L, ptr=None) == rtp.RTP_EINVAL                          # NULL tensors
    for p in (0.0, -0.5, math.nan):
        assert lib.rtp_topp_select(L.desc, 1000, FAKE, FAKE, FAKE, p, FAKE, FAKE, None, FAKE, 1 << 30, None) \
            == rtp.RTP_EINVAL
    assert lib.rtp_topp_select(L.desc, 1000, FAKE, FAKE, FAKE, 0.9, FAKE, FAKE, None, FAKE, 64, None) \
        == rtp.RTP_EWORKSPACE
    # top-p mass is fixed point sized from the context: refused above 2^24 tokens (p < 1 only)
    Lbig = _layer(batch=1, n_cap=(1 << 24) + 1)
    assert lib.rtp_topp_select(Lbig.desc, (1 << 24) + 1, FAKE, FAKE, FAKE, 0.9, FAKE, FAKE, None, FAKE, 1 << 40,
                               None) == rtp.RTP_EUNSUPPORTED
    assert "2^24" in lib.rtp_last_error().decode()
    assert _call_step(Lbig, n_ctx=(1 << 24) + 1, ws_bytes=1 << 40) == rtp.RTP_EUNSUPPORTED
    assert lib.rtp_sparse_decode_attn(L.desc, 1000, FAKE, FAKE, FAKE, None, FAKE, None, 0.1, FAKE, FAKE, 1 << 30,
                                      None) == rtp.RTP_EINVAL
    assert lib.rtp_sparse_decode_attn(L.desc, 1000, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, math.inf, FAKE, FAKE,
                                      1 << 30, None) == rtp.RTP_EINVAL
    assert lib.rtp_window_sink_attn(L.desc, 1000, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, 8, None) \
        == rtp.RTP_EWORKSPACE
    L1 = _layer(batch=1, n_cap=32768)
    assert lib.rtp_prefill_attn(_layer().desc, 0, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0.1, FAKE, FAKE,
                                1 << 30, None) == rtp.RTP_EINVAL                # batch must be 1
    assert lib.rtp_prefill_attn(L1.desc, 32700, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0.1, FAKE, FAKE,
                                1 << 30, None) == rtp.RTP_EINVAL                # c0 + C > n_cap
    assert lib.rtp_prefill_attn(L1.desc, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0.1, FAKE, FAKE,
                                1 << 30, None) == rtp.RTP_EINVAL                # C >= 1


def test_probe_validation():
    lib = rtp.load()
    fl = C.c_double(0.0)
    assert lib.rtp_mfma_probe(10, None, C.byref(fl), None) == rtp.RTP_EINVAL
    assert lib.rtp_mfma_probe(0, C.c_void_p(16), C.byref(fl), None) == rtp.RTP_EINVAL
    assert lib.rtp_mfma_probe((1 << 24) + 1, C.c_void_p(16), C.byref(fl), None) == rtp.RTP_EINVAL
    assert lib.rtp_hbm_read_probe(None, 64, C.c_void_p(16), None) == rtp.RTP_EINVAL


def test_binding_raises_with_message():
    L = _layer(head_dim=96)
    with pytest.raises(rtp.RtpError, match="RTP_EUNSUPPORTED: head_dim"):
        rtp._check(_call_score(L))


def test_injected_device_failure(monkeypatch):
    """With RTP_FAULT_INJECT set, every entry point whose host checks pass returns
    RTP_EDEVICE where it would first touch the device (nothing is launched, so this runs
    without a GPU), and the binding turns that status into RtpError.  Host checks still
    come first: a bad argument keeps its own status."""
    lib = _lib()
    monkeypatch.setenv("RTP_FAULT_INJECT", "1")
    L = _layer()
    L1 = _layer(batch=1, n_cap=32768)
    Ls = _layer(batch=1, n_cap=8192)                 # fits the allocation-free step's scratch
    big = 1 << 30
    fl = C.c_double(0.0)
    gen = C.c_void_p(FAKE)
    calls = {
        "rtp_indexer_score": lambda: _call_score(L),
        "rtp_topp_select": lambda: lib.rtp_topp_select(L.desc, 1000, FAKE, FAKE, FAKE, 0.9, FAKE, FAKE, None, FAKE,
                                                       big, None),
        "rtp_topk_select": lambda: lib.rtp_topk_select(L.desc, 1000, FAKE, 10, FAKE, FAKE, None, FAKE, big, None),
        "rtp_sparse_decode_attn": lambda: lib.rtp_sparse_decode_attn(L.desc, 1000, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                                                     0.1, FAKE, FAKE, big, None),
        "rtp_window_sink_attn": lambda: lib.rtp_window_sink_attn(L.desc, 1000, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, big,
                                                                 None),
        "rtp_prefill_attn": lambda: lib.rtp_prefill_attn(L1.desc, 0, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 128 * 16,
                                                         FAKE, 0.1, FAKE, FAKE, big, None),
        "rtp_decode_step": lambda: _call_step(L),
        "rtp_decode_step_dev": lambda: lib.rtp_decode_step_dev(L.desc, 1000, gen, FAKE, FAKE, 0, FAKE, 1.0, FAKE,
                                                               FAKE, FAKE, None, None, 0.9, 0.1, FAKE, FAKE, FAKE,
                                                               FAKE, FAKE, None, FAKE, FAKE, big, None),
        "rtp_decode_step_noalloc": lambda: lib.rtp_decode_step_noalloc(Ls.desc, 1000, FAKE, FAKE, 0, FAKE, 1.0, FAKE,
                                                                       FAKE, FAKE, None, None, 0.9, 0.1, FAKE, FAKE,
                                                                       FAKE, FAKE, FAKE, None, FAKE, None),
        "rtp_append_token": lambda: lib.rtp_append_token(L.desc, 100, FAKE, FAKE, FAKE, FAKE, 128 * 16, FAKE, FAKE,
                                                         FAKE, None, None, None),
        "rtp_append_token_dev": lambda: lib.rtp_append_token_dev(L.desc, gen, FAKE, FAKE, FAKE, FAKE, 128 * 16, FAKE,
                                                                 FAKE, FAKE, None, None, None),
        "rtp_mfma_probe": lambda: lib.rtp_mfma_probe(10, C.c_void_p(FAKE), C.byref(fl), None),
        "rtp_hbm_read_probe": lambda: lib.rtp_hbm_read_probe(FAKE, 1 << 20, C.c_void_p(FAKE), None),
    }
    for name, call in calls.items():
        st = call()
        msg = lib.rtp_last_error().decode()
        assert st == rtp.RTP_EDEVICE, f"{name}: status {st} ({msg})"
        assert "injected" in msg, f"{name}: {msg}"
        with pytest.raises(rtp.RtpError, match="RTP_EDEVICE: .*injected") as ei:
            rtp._check(st)
        assert ei.value.status == rtp.RTP_EDEVICE
    # host checks come before the gate
    assert _call_score(L, n_ctx=0) == rtp.RTP_EINVAL
    assert _call_step(L, top_p=math.nan) == rtp.RTP_EINVAL
    assert lib.rtp_mfma_probe(0, C.c_void_p(FAKE), C.byref(fl), None) == rtp.RTP_EINVAL
    # every exported entry point that enqueues work is covered
    enqueue = {n for n in rtp.EXPORTED if n not in ("rtp_workspace_bytes", "rtp_status_string", "rtp_last_error",
                                                    "rtp_version", "rtp_decode_step_noalloc_max_bytes")}
    assert enqueue == set(calls)


def test_roctx_ranges_behind_env_flag():
    """RTP_ROCTX=1 makes the library open the roctx library at its first call and wrap
    every call in a range (here a call that fails its host checks); without the flag the
    roctx library is never loaded."""
    import subprocess
    import sys
    code = ("import ctypes as C\n"
            "from head_wise_sparse_amd import rtp\n"
            "lib = rtp.load()\n"
            "L = rtp.Layer(1, 8, 2, 128, 4096, [1, 0], 4, 64)\n"
            "assert lib.rtp_window_sink_attn(L.desc, 0, 16, 16, 16, 0.1, 16, 16, 1 << 20, None) == rtp.RTP_EINVAL\n"
            "print('roctx' in open('/proc/self/maps').read())\n")
    seen = {}
    for flag in ("1", ""):
        env = dict(os.environ, RTP_ROCTX=flag)
        r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=120)
        assert r.returncode == 0, r.stderr[-2000:]
        seen[flag] = r.stdout.strip().splitlines()[-1]
    assert seen[""] == "False"
    roctx_present = any(os.path.exists(os.path.join(d, n)) for d in ("/opt/rocm/lib",)
                        for n in ("librocprofiler-sdk-roctx.so.1", "libroctx64.so.4"))
    assert seen["1"] == str(roctx_present)
