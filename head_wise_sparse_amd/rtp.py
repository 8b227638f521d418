"""ctypes binding of librtp (the C ABI declared in include/rtp.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch is used for device memory and streams.  The functions keep the C
names; tensors are torch CUDA (ROCm) tensors in the layouts rtp.h documents, and
``stream`` defaults to torch's current stream.  A non-OK status raises RtpError.
If the shared library has not been built, every call raises: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

# RTP_LIB_PATH names another build of the same library (the host-sanitized one of the CPU tests)
LIB_PATH = os.environ.get("RTP_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib",
                                                          "librtp.so")

RTP_OK, RTP_EINVAL, RTP_EUNSUPPORTED, RTP_EWORKSPACE, RTP_EDEVICE = range(5)
CALL_INDEXER_SCORE, CALL_TOPP_SELECT, CALL_SPARSE_DECODE, CALL_WINDOW_SINK, CALL_PREFILL, CALL_DECODE_STEP = range(6)
SEL_RANGE = 1024          # RTP_SEL_RANGE: token range of one entry of a selected-set range index
KV_FULL, KV_COMPACT = 0, 1

EXPORTED = ["rtp_workspace_bytes", "rtp_indexer_score", "rtp_topp_select", "rtp_sparse_decode_attn",
            "rtp_window_sink_attn", "rtp_prefill_attn", "rtp_decode_step", "rtp_topk_select", "rtp_append_token",
            "rtp_hbm_read_probe", "rtp_mfma_probe", "rtp_status_string", "rtp_last_error", "rtp_version",
            "rtp_decode_step_noalloc", "rtp_decode_step_noalloc_max_bytes", "rtp_append_token_dev",
            "rtp_decode_step_dev"]


class RtpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


class _Desc(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("idx_dim", C.c_int32), ("n_cap", C.c_int64),
                ("kv_role", C.POINTER(C.c_uint8)), ("n_sinks", C.c_int32), ("window", C.c_int32),
                ("kv_layout", C.c_int32)]


_lib = None
_P = C.c_void_p


def load() -> C.CDLL:
    """Load librtp.so (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m head_wise_sparse_amd.build` "
                           "(the HIP library is required, there is no fallback)")
    lib = C.CDLL(LIB_PATH)
    D = C.POINTER(_Desc)
    sig = {
        "rtp_workspace_bytes": (C.c_size_t, [D, C.c_int64, C.c_int]),
        "rtp_indexer_score": (C.c_int, [D, C.c_int64, _P, _P, C.c_int64, _P, C.c_float, _P, _P, _P, _P,
                                        C.c_size_t, _P]),
        "rtp_topp_select": (C.c_int, [D, C.c_int64, _P, _P, _P, C.c_float, _P, _P, _P, _P, C.c_size_t, _P]),
        "rtp_sparse_decode_attn": (C.c_int, [D, C.c_int64, _P, _P, _P, _P, _P, _P, C.c_float, _P, _P,
                                             C.c_size_t, _P]),
        "rtp_window_sink_attn": (C.c_int, [D, C.c_int64, _P, _P, _P, C.c_float, _P, _P, C.c_size_t, _P]),
        "rtp_prefill_attn": (C.c_int, [D, C.c_int64, C.c_int32, _P, _P, _P, _P, _P, C.c_int64, _P, C.c_float,
                                       _P, _P, C.c_size_t, _P]),
        "rtp_decode_step": (C.c_int, [D, C.c_int64, _P, _P, C.c_int64, _P, C.c_float, _P, _P, _P, _P, _P,
                                      C.c_float, C.c_float, _P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
        "rtp_decode_step_noalloc": (C.c_int, [D, C.c_int64, _P, _P, C.c_int64, _P, C.c_float, _P, _P, _P, _P, _P,
                                              C.c_float, C.c_float, _P, _P, _P, _P, _P, _P, _P, _P]),
        "rtp_decode_step_noalloc_max_bytes": (C.c_size_t, []),
        "rtp_decode_step_dev": (C.c_int, [D, C.c_int64, _P, _P, _P, C.c_int64, _P, C.c_float, _P, _P, _P, _P, _P,
                                          C.c_float, C.c_float, _P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
        "rtp_append_token_dev": (C.c_int, [D, _P, _P, _P, _P, _P, C.c_int64, _P, _P, _P, _P, _P, _P]),
        "rtp_append_token": (C.c_int, [D, C.c_int64, _P, _P, _P, _P, C.c_int64, _P, _P, _P, _P, _P, _P]),
        "rtp_topk_select": (C.c_int, [D, C.c_int64, _P, C.c_int64, _P, _P, _P, _P, C.c_size_t, _P]),
        "rtp_hbm_read_probe": (C.c_int, [_P, C.c_size_t, _P, _P]),
        "rtp_mfma_probe": (C.c_int, [C.c_uint32, _P, C.POINTER(C.c_double), _P]),
        "rtp_status_string": (C.c_char_p, [C.c_int]),
        "rtp_last_error": (C.c_char_p, []),
        "rtp_version": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _status_name(s: int) -> str:
    try:
        return load().rtp_status_string(s).decode()
    except Exception:  # pragma: no cover - only when the library itself is missing
        return f"status {s}"


def _check(status: int):
    if status != RTP_OK:
        raise RtpError(status, load().rtp_last_error().decode())


@dataclass
class Layer:
    """Host-side description of one attention layer (mirrors rtp_layer_desc)."""
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_cap: int
    kv_role: Sequence[int]
    n_sinks: int
    window: int
    idx_dim: int = 16
    kv_layout: int = KV_FULL

    def __post_init__(self):
        self._role = (C.c_uint8 * len(self.kv_role))(*[int(r) for r in self.kv_role])
        self._desc = _Desc(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.idx_dim,
                           self.n_cap, C.cast(self._role, C.POINTER(C.c_uint8)), self.n_sinks, self.window,
                           self.kv_layout)

    @property
    def desc(self):
        return C.byref(self._desc)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_kv_r(self) -> int:
        return int(sum(1 for r in self.kv_role if r))

    @property
    def n_q_r(self) -> int:
        return self.n_kv_r * self.group


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("rtp: tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("rtp: tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ws(ws):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def rtp_workspace_bytes(layer: Layer, n_ctx: int, which: int) -> int:
    return int(load().rtp_workspace_bytes(layer.desc, int(n_ctx), int(which)))


def workspace(layer: Layer, n_ctx: int, which: int, device="cuda"):
    """A workspace tensor of the size the call needs (256-byte aligned by torch's allocator)."""
    import torch
    n = max(256, rtp_workspace_bytes(layer, n_ctx, which))
    return torch.zeros(n, dtype=torch.uint8, device=device)      # workspaces start zero-filled


def rtp_indexer_score(layer: Layer, n_ctx: int, q_pre, w_q_idx, w_head_stride: int, k_idx, idx_scale: float,
                      scores, row_max, row_sum, ws, stream=None):
    p, n = _ws(ws)
    _check(load().rtp_indexer_score(layer.desc, int(n_ctx), _ptr(q_pre), _ptr(w_q_idx), int(w_head_stride),
                                    _ptr(k_idx), float(idx_scale), _ptr(scores), _ptr(row_max), _ptr(row_sum),
                                    p, n, _stream(stream)))


def rtp_topp_select(layer: Layer, n_ctx: int, scores, row_max, row_sum, top_p: float, sel_idx, sel_count,
                    sel_starts, ws, stream=None):
    p, n = _ws(ws)
    _check(load().rtp_topp_select(layer.desc, int(n_ctx), _ptr(scores), _ptr(row_max), _ptr(row_sum),
                                  float(top_p), _ptr(sel_idx), _ptr(sel_count), _ptr(sel_starts), p, n,
                                  _stream(stream)))


def rtp_topk_select(layer: Layer, n_ctx: int, scores, k: int, sel_idx, sel_count, sel_starts, ws, stream=None):
    p, n = _ws(ws)
    _check(load().rtp_topk_select(layer.desc, int(n_ctx), _ptr(scores), int(k), _ptr(sel_idx), _ptr(sel_count),
                                  _ptr(sel_starts), p, n, _stream(stream)))


def rtp_sparse_decode_attn(layer: Layer, n_ctx: int, q, k_cache, v_cache, sel_idx, sel_count, sel_starts,
                           sm_scale: float, out, ws, stream=None):
    p, n = _ws(ws)
    _check(load().rtp_sparse_decode_attn(layer.desc, int(n_ctx), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(sel_idx), _ptr(sel_count), _ptr(sel_starts), float(sm_scale),
                                         _ptr(out), p, n, _stream(stream)))


def rtp_window_sink_attn(layer: Layer, n_ctx: int, q, k_cache, v_cache, sm_scale: float, out, ws, stream=None):
    p, n = _ws(ws)
    _check(load().rtp_window_sink_attn(layer.desc, int(n_ctx), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       float(sm_scale), _ptr(out), p, n, _stream(stream)))


def rtp_prefill_attn(layer: Layer, c0: int, C_rows: int, q, k_cache, v_cache, k_pre, w_k_idx, w_head_stride: int,
                     k_idx_cache, sm_scale: float, out, ws, stream=None):
    p, n = _ws(ws)
    _check(load().rtp_prefill_attn(layer.desc, int(c0), int(C_rows), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(k_pre), _ptr(w_k_idx), int(w_head_stride), _ptr(k_idx_cache),
                                   float(sm_scale), _ptr(out), p, n, _stream(stream)))


def rtp_decode_step(layer: Layer, n_ctx: int, q_pre, w_q_idx, w_head_stride: int, k_idx, idx_scale: float, q,
                    k_cache, v_cache, k_loc, v_loc, top_p: float, sm_scale: float, scores, row_max, row_sum, sel_idx,
                    sel_count, sel_starts, out, ws, stream=None):
    p, n = _ws(ws)
    _check(load().rtp_decode_step(layer.desc, int(n_ctx), _ptr(q_pre), _ptr(w_q_idx), int(w_head_stride),
                                  _ptr(k_idx), float(idx_scale), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_loc),
                                  _ptr(v_loc), float(top_p), float(sm_scale), _ptr(scores), _ptr(row_max),
                                  _ptr(row_sum), _ptr(sel_idx), _ptr(sel_count), _ptr(sel_starts), _ptr(out), p, n,
                                  _stream(stream)))


def rtp_decode_step_noalloc(layer: Layer, n_ctx: int, q_pre, w_q_idx, w_head_stride: int, k_idx, idx_scale: float,
                            q, k_cache, v_cache, k_loc, v_loc, top_p: float, sm_scale: float, scores, row_max,
                            row_sum, sel_idx, sel_count, sel_starts, out, stream=None):
    _check(load().rtp_decode_step_noalloc(layer.desc, int(n_ctx), _ptr(q_pre), _ptr(w_q_idx), int(w_head_stride),
                                          _ptr(k_idx), float(idx_scale), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(k_loc), _ptr(v_loc), float(top_p), float(sm_scale), _ptr(scores),
                                          _ptr(row_max), _ptr(row_sum), _ptr(sel_idx), _ptr(sel_count),
                                          _ptr(sel_starts), _ptr(out), _stream(stream)))


def rtp_decode_step_dev(layer: Layer, n_max: int, gen, q_pre, w_q_idx, w_head_stride: int, k_idx, idx_scale: float,
                        q, k_cache, v_cache, k_loc, v_loc, top_p: float, sm_scale: float, scores, row_max, row_sum,
                        sel_idx, sel_count, sel_starts, out, ws, stream=None):
    p, n = _ws(ws)
    _check(load().rtp_decode_step_dev(layer.desc, int(n_max), _ptr(gen), _ptr(q_pre), _ptr(w_q_idx),
                                      int(w_head_stride), _ptr(k_idx), float(idx_scale), _ptr(q), _ptr(k_cache),
                                      _ptr(v_cache), _ptr(k_loc), _ptr(v_loc), float(top_p), float(sm_scale),
                                      _ptr(scores), _ptr(row_max), _ptr(row_sum), _ptr(sel_idx), _ptr(sel_count),
                                      _ptr(sel_starts), _ptr(out), p, n, _stream(stream)))


def rtp_append_token_dev(layer: Layer, gen, k_new, v_new, k_pre, w_k_idx, w_head_stride: int, k_cache, v_cache,
                         k_idx_cache, k_loc=None, v_loc=None, stream=None):
    _check(load().rtp_append_token_dev(layer.desc, _ptr(gen), _ptr(k_new), _ptr(v_new), _ptr(k_pre), _ptr(w_k_idx),
                                       int(w_head_stride), _ptr(k_cache), _ptr(v_cache), _ptr(k_idx_cache),
                                       _ptr(k_loc), _ptr(v_loc), _stream(stream)))


def rtp_decode_step_noalloc_max_bytes() -> int:
    return int(load().rtp_decode_step_noalloc_max_bytes())


def rtp_append_token(layer: Layer, pos: int, k_new, v_new, k_pre, w_k_idx, w_head_stride: int, k_cache, v_cache,
                     k_idx_cache, k_loc=None, v_loc=None, stream=None):
    _check(load().rtp_append_token(layer.desc, int(pos), _ptr(k_new), _ptr(v_new), _ptr(k_pre), _ptr(w_k_idx),
                                   int(w_head_stride), _ptr(k_cache), _ptr(v_cache), _ptr(k_idx_cache), _ptr(k_loc),
                                   _ptr(v_loc), _stream(stream)))


def rtp_hbm_read_probe(buf, sink, stream=None):
    _check(load().rtp_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def rtp_mfma_probe(iters: int, sink, stream=None) -> float:
    """Enqueue the MFMA throughput probe; returns the launch's flop count."""
    fl = C.c_double(0.0)
    _check(load().rtp_mfma_probe(int(iters), _ptr(sink), C.byref(fl), _stream(stream)))
    return fl.value


def rtp_version() -> str:
    return load().rtp_version().decode()


# ----------------------------------------------------------------------------- conveniences
def to_device_bf16(bits: np.ndarray, device="cuda"):
    """uint16 bf16 bits (numpy) -> torch.bfloat16 tensor on the device."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def from_device_bf16(t) -> np.ndarray:
    """torch.bfloat16 tensor -> uint16 bf16 bits (numpy)."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DecodeStep:
    """One decode step of one layer, with every output and workspace allocated once.
    ``run`` enqueues, on one stream, either the fused call (``rtp_decode_step``, the
    default) or the four separate calls: indexer scores -> top-p sets (with their range
    index) -> sparse attention of the retrieval heads, and sink+window attention of the
    local heads.  Both give the same bits."""

    def __init__(self, layer: Layer, n_ctx: int, top_p: float, sm_scale: Optional[float] = None,
                 idx_scale: float = 1.0, device="cuda", fused: bool = True):
        import torch
        self.layer, self.n_ctx, self.top_p, self.fused = layer, int(n_ctx), float(top_p), bool(fused)
        self.sm_scale = (1.0 / layer.head_dim ** 0.5) if sm_scale is None else float(sm_scale)
        self.idx_scale = float(idx_scale)
        B, R, cap = layer.batch, layer.n_q_r, layer.n_cap
        nsplit = (cap + SEL_RANGE - 1) // SEL_RANGE
        self.scores = torch.empty(B * R * cap, dtype=torch.float32, device=device)
        self.row_max = torch.empty(B * R, dtype=torch.float32, device=device)
        self.row_sum = torch.empty(B * R, dtype=torch.float32, device=device)
        self.sel_idx = torch.empty(B * R * cap, dtype=torch.int32, device=device)
        self.sel_count = torch.empty(B * R, dtype=torch.int32, device=device)
        self.sel_starts = torch.empty(B * R * (nsplit + 1), dtype=torch.int32, device=device)
        self.out = torch.zeros(B * layer.n_q_heads * layer.head_dim, dtype=torch.bfloat16, device=device)
        which = (CALL_DECODE_STEP,) if self.fused else (CALL_INDEXER_SCORE, CALL_TOPP_SELECT, CALL_SPARSE_DECODE,
                                                         CALL_WINDOW_SINK)
        # sized for the full capacity, so one step object serves any n_ctx <= n_cap
        self.ws = {w: workspace(layer, cap, w, device) for w in which}

    def run(self, q_pre, q, k_cache, v_cache, k_idx, w_q_idx, w_head_stride: Optional[int] = None, stream=None,
            n_ctx: Optional[int] = None, k_loc=None, v_loc=None):
        """k_cache/v_cache: the full cache (KV_FULL) or the retrieval cache (KV_COMPACT,
        with the local ring in k_loc/v_loc)."""
        L = self.layer
        n = self.n_ctx if n_ctx is None else int(n_ctx)
        if w_head_stride is None:
            w_head_stride = L.head_dim * L.idx_dim
        if self.fused:
            rtp_decode_step(L, n, q_pre, w_q_idx, w_head_stride, k_idx, self.idx_scale, q, k_cache, v_cache, k_loc,
                            v_loc, self.top_p, self.sm_scale, self.scores, self.row_max, self.row_sum, self.sel_idx,
                            self.sel_count, self.sel_starts, self.out, self.ws[CALL_DECODE_STEP], stream)
            return self.out
        rtp_indexer_score(L, n, q_pre, w_q_idx, w_head_stride, k_idx, self.idx_scale, self.scores, self.row_max,
                          self.row_sum, self.ws[CALL_INDEXER_SCORE], stream)
        rtp_topp_select(L, n, self.scores, self.row_max, self.row_sum, self.top_p, self.sel_idx, self.sel_count,
                        self.sel_starts, self.ws[CALL_TOPP_SELECT], stream)
        rtp_sparse_decode_attn(L, n, q, k_cache, v_cache, self.sel_idx, self.sel_count, self.sel_starts,
                               self.sm_scale, self.out, self.ws[CALL_SPARSE_DECODE], stream)
        compact = L.kv_layout == KV_COMPACT
        rtp_window_sink_attn(L, n, q, k_loc if compact else k_cache, v_loc if compact else v_cache, self.sm_scale,
                             self.out, self.ws[CALL_WINDOW_SINK], stream)
        return self.out

    def run_dev(self, gen, q_pre, q, k_cache, v_cache, k_idx, w_q_idx, w_head_stride: Optional[int] = None,
                stream=None, k_loc=None, v_loc=None):
        """The fused step with the context length read from the device state `gen` (int64
        {pos, n_ctx}); grids and strides are sized for this object's n_ctx (the bound)."""
        L = self.layer
        if w_head_stride is None:
            w_head_stride = L.head_dim * L.idx_dim
        rtp_decode_step_dev(L, self.n_ctx, gen, q_pre, w_q_idx, w_head_stride, k_idx, self.idx_scale, q, k_cache,
                            v_cache, k_loc, v_loc, self.top_p, self.sm_scale, self.scores, self.row_max,
                            self.row_sum, self.sel_idx, self.sel_count, self.sel_starts, self.out,
                            self.ws[CALL_DECODE_STEP], stream)
        return self.out
