#!/usr/bin/env python3
"""Benchmark of the head-wise sparse attention hot path on one MI355X.

One step = one pass of the whole path over synthetic inputs:
  * a decode step of one layer at 128K context, batch 4, 32 q / 8 KV heads, d128:
    indexer scores -> top-p sets (p = 0.95) -> sparse attention of the 2 retrieval
    KV heads (+ their 8 q heads) and sink+window attention of the 6 local KV heads;
  * a causal 32K-token prefill of one sequence in 4K chunks (retrieval heads dense,
    local heads 4 sinks + 4096 window, indexer keys projected in the chunk).

Inputs are resident in HBM before the timed region.  Decode rotates over several
copies of the layer's caches so consecutive steps do not hit in the 256 MB
Infinity Cache.  Prints one JSON line (see the fields below).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

# HBM bytes per call from rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch, summed over the call's kernels), with the scale each counter showed for a
# plain 1 GiB device copy: FETCH_SIZE read half the bytes moved, WRITE_SIZE all of them.
# `src` is the sha256 prefix of the kernel source the counters were taken on; once it
# changes the figure no longer describes the kernel and `traffic` is reported as null.
COPY_SCALE = {"fetch": 1.9999, "write": 1.0000}
MEASURED_KIB = {
    "prefill_attn": {"src": ("rtp_prefill.hip", "9c8e4c2435f8d8e8"),
                     "fetch": 211933.4, "write": 41691.5},
    "sparse_decode": {"src": ("decode_dev.hpp", "e31967e96b51ec13"),
                      "fetch": 172546.0 + 1086.5, "write": 2176.3 + 8.0},
}


def measured_traffic(name):
    """HBM bytes per call of `name` as the counters measured it, or None if its source changed."""
    import hashlib
    m = MEASURED_KIB[name]
    path = os.path.join(ROOT, "head_wise_sparse_amd", "csrc", m["src"][0])
    with open(path, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest()[:16] != m["src"][1]:
            return None
    return int((m["fetch"] * COPY_SCALE["fetch"] + m["write"] * COPY_SCALE["write"]) * 1024)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--copies", type=int, default=3, help="decode cache copies rotated across steps")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the p = 0.9 / 0.99 decode timings")
    ap.add_argument("--gen-steps", type=int, default=128,
                    help="generated tokens of the growing-context workload (0: skip it)")
    ap.add_argument("--only", choices=["decode", "prefill", "prefill_1m"], default=None,
                    help="run only one part (for profiling); the JSON line is still printed "
                         "(prefill_1m: the 1M-token chunked prefill alone, as one timing report line)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the timings of the other decode and prefill workloads in the default run")
    ap.add_argument("--report-configs", action="store_true",
                    help="per-config timings of every decode and prefill workload (one JSON report line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device-to-device 3 times (scale reference for HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain device copy of known size: what FETCH_SIZE / WRITE_SIZE read for it is the
    scale that turns those counters into bytes for the kernels measured alongside."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- decode
class DecodeBench:
    def __init__(self, copies: int, name: str = "decode_b4_128k"):
        import torch
        from head_wise_sparse_amd import rtp
        from head_wise_sparse_amd import workloads as W
        self.torch, self.rtp = torch, rtp
        self.cfg = cfg = W.CONFIGS[name]
        t = time.time()
        self.x = x = W.make_decode_inputs(cfg)
        log(f"decode inputs drawn in {time.time() - t:.1f}s")
        self.L = rtp.Layer(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx,
                           cfg.kv_role.tolist(), cfg.n_sinks, cfg.window)
        dev = rtp.to_device_bf16
        base = dict(q_pre=dev(x.q_pre), q=dev(x.q), k=dev(x.k), v=dev(x.v), k_idx=dev(x.k_idx),
                    w_q_idx=dev(x.w_q_idx))
        self.sets = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(copies - 1)]
        self.steps = {}
        self.graphs = {}
        torch.cuda.synchronize()

    def _step_obj(self, p: float, fused: bool = True):
        if (p, fused) not in self.steps:
            self.steps[(p, fused)] = self.rtp.DecodeStep(self.L, self.cfg.n_ctx, p, fused=fused)
        return self.steps[(p, fused)]

    def _launch(self, p: float, i: int, which=None):
        """Enqueue the decode step (fused call; which="separate": the four calls), or one
        of the four calls, on the current stream."""
        rtp, L, n = self.rtp, self.L, self.cfg.n_ctx
        s = self.sets[i % len(self.sets)]
        if which is None:
            return self._step_obj(p).run(s["q_pre"], s["q"], s["k"], s["v"], s["k_idx"], s["w_q_idx"])
        st = self._step_obj(p, fused=False)
        if which == "separate":
            return st.run(s["q_pre"], s["q"], s["k"], s["v"], s["k_idx"], s["w_q_idx"])
        if which == "indexer_score":
            rtp.rtp_indexer_score(L, n, s["q_pre"], s["w_q_idx"], L.head_dim * 16, s["k_idx"], 1.0, st.scores,
                                  st.row_max, st.row_sum, st.ws[rtp.CALL_INDEXER_SCORE])
        elif which == "topp_select":
            rtp.rtp_topp_select(L, n, st.scores, st.row_max, st.row_sum, p, st.sel_idx, st.sel_count,
                                st.sel_starts, st.ws[rtp.CALL_TOPP_SELECT])
        elif which == "sparse_decode":
            rtp.rtp_sparse_decode_attn(L, n, s["q"], s["k"], s["v"], st.sel_idx, st.sel_count, st.sel_starts,
                                       st.sm_scale, st.out, st.ws[rtp.CALL_SPARSE_DECODE])
        elif which == "window_sink":
            rtp.rtp_window_sink_attn(L, n, s["q"], s["k"], s["v"], st.sm_scale, st.out,
                                     st.ws[rtp.CALL_WINDOW_SINK])

    def graph(self, p: float, i: int, which=None):
        """A HIP graph (captured through torch) of the step or of one call, on cache copy i."""
        key = (p, i % len(self.sets), which)
        if key not in self.graphs:
            torch = self.torch
            self._launch(p, i, which)                 # eager run first: allocations happen outside capture
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._launch(p, i, which)
            torch.cuda.synchronize()
            self.graphs[key] = g
        return self.graphs[key]

    def step(self, p: float, i: int):
        """One fused decode step on cache copy i, launched directly (seven kernel launches)."""
        self._launch(p, i)

    def step_graph(self, p: float, i: int):
        self.graph(p, i).replay()

    def call_times(self, p: float, reps: int = 20):
        """Average duration (ms) of each of the four calls: each call is captured in its own
        graph and replayed `reps` times between HIP events on the launch stream."""
        torch = self.torch
        names = ["indexer_score", "topp_select", "sparse_decode", "window_sink"]
        out = {}
        for k in names:
            gs = [self.graph(p, i, k) for i in range(len(self.sets))]
            for g in gs:
                g.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for i in range(reps):
                gs[i % len(gs)].replay()
            b.record()
            torch.cuda.synchronize()
            out[k] = a.elapsed_time(b) / reps
        return out

    def algorithmic_bytes(self, p: float):
        """Bytes the method must move for one decode step (not the dense work it avoids)."""
        cfg, st = self.cfg, self.steps[(p, True)]
        B, N, D, G = cfg.batch, cfg.n_ctx, cfg.head_dim, cfg.group
        R = cfg.n_kv_r * G
        cnt = st.sel_count.view(B, R).cpu().numpy()
        sel = st.sel_idx.view(B, R, -1).cpu().numpy()
        union = 0
        per_head = int(cnt.sum())
        for b in range(B):
            for r in range(cfg.n_kv_r):
                u = np.unique(np.concatenate([sel[b, r * G + t, :cnt[b, r * G + t]] for t in range(G)]))
                union += u.size
        s_end = min(cfg.n_sinks, N)
        w_start = max(N - cfg.window, s_end)
        n_local = s_end + (N - w_start)
        n_loc_kv = cfg.n_kv_heads - cfg.n_kv_r
        kidx = 32 * N * B * cfg.n_kv_r
        local = 4 * D * n_local * B * n_loc_kv
        gathered = 4 * D * union
        qo = 2 * 2 * D * B * cfg.n_q_heads
        groups = B * cfg.n_kv_r
        return {"kidx": kidx, "local_kv": local, "gathered_kv_union": gathered, "q_out": qo,
                "total": kidx + local + gathered + qo, "union_tokens": union, "per_head_tokens": per_head,
                "sel_min": int(cnt.min()), "sel_median": int(np.median(cnt)), "sel_mean": float(cnt.mean()),
                "sel_max": int(cnt.max()),
                # compute sparsity (summary, "Experimental setup", metrics): share of the context a
                # retrieval head does not attend to, per query head and per GQA group's union
                "compute_sparsity": {"per_head_mean": round(1.0 - float(cnt.mean()) / N, 4),
                                     "per_head_min": round(1.0 - float(cnt.max()) / N, 4),
                                     "gqa_union_mean": round(1.0 - union / (groups * N), 4)}}


# ----------------------------------------------------------------------------- long generation
class GenBench:
    """Generation over a growing context in the compact KV layout: every step appends the
    next token (its K/V rows and, for retrieval heads, its indexer key) and runs the fused
    decode step at the new length.  Launched eagerly: the context length changes every
    step.  The retrieval heads keep their whole history, the local heads a ring of
    sinks + window."""

    def __init__(self, dec: "DecodeBench", steps: int):
        torch, rtp = dec.torch, dec.rtp
        self.torch, self.rtp = torch, rtp
        cfg, x = dec.cfg, dec.x
        self.cfg, self.T = cfg, steps
        self.n0 = cfg.n_ctx - steps
        self.L = rtp.Layer(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx, cfg.kv_role.tolist(),
                           cfg.n_sinks, cfg.window, kv_layout=rtp.KV_COMPACT)
        ret = [g for g in range(cfg.n_kv_heads) if cfg.kv_role[g]]
        loc = [g for g in range(cfg.n_kv_heads) if not cfg.kv_role[g]]
        S, Wn, n0 = cfg.n_sinks, cfg.window, self.n0
        dev = lambda a: rtp.to_device_bf16(np.ascontiguousarray(a))
        self.kr, self.vr = dev(x.k[:, ret]), dev(x.v[:, ret])
        rows = S + Wn
        kl = np.zeros((cfg.batch, len(loc), rows, cfg.head_dim), np.uint16)
        vl = np.zeros_like(kl)
        for j in list(range(min(S, n0))) + list(range(max(n0 - Wn, S), n0)):
            slot = j if j < S else S + (j - S) % Wn
            kl[:, :, slot] = x.k[:, loc, j]
            vl[:, :, slot] = x.v[:, loc, j]
        self.kl, self.vl = dev(kl), dev(vl)
        self.kidx = dev(x.k_idx)
        self.k_new = dev(np.moveaxis(x.k[:, :, n0:n0 + steps], 2, 0))      # [T][B][Hkv][D]
        self.v_new = dev(np.moveaxis(x.v[:, :, n0:n0 + steps], 2, 0))
        rng = np.random.default_rng(0)
        from head_wise_sparse_amd.workloads import f32_to_bf16_bits
        self.k_pre = dev(f32_to_bf16_bits(rng.standard_normal((steps, cfg.batch, cfg.n_kv_heads, cfg.head_dim))
                                          .astype(np.float32)))
        self.w_k = dev(x.w_k_idx)
        self.q_pre, self.q, self.w_q = dev(x.q_pre), dev(x.q), dev(x.w_q_idx)
        self.step = rtp.DecodeStep(self.L, cfg.n_ctx, cfg.top_p)
        D = cfg.head_dim
        self.tok = cfg.batch * cfg.n_kv_heads * D
        self.full_bytes = cfg.batch * cfg.n_kv_heads * cfg.n_ctx * D * 4
        self.compact_bytes = cfg.batch * (len(ret) * cfg.n_ctx + len(loc) * rows) * D * 4
        torch.cuda.synchronize()

    def run(self):
        rtp, D = self.rtp, self.cfg.head_dim
        for t in range(self.T):
            pos = self.n0 + t
            rtp.rtp_append_token(self.L, pos, self.k_new[t], self.v_new[t], self.k_pre[t], self.w_k, D * 16, self.kr,
                                 self.vr, self.kidx, self.kl, self.vl)
            self.step.run(self.q_pre, self.q, self.kr, self.vr, self.kidx, self.w_q, n_ctx=pos + 1, k_loc=self.kl,
                          v_loc=self.vl)

    def capture(self):
        """One HIP graph of [rtp_append_token_dev, rtp_decode_step_dev]: the context length is
        the device state {pos, n_ctx} that every replay advances by one token.  The replays
        append the same new-token vectors at successive positions (the work per token does
        not depend on their values)."""
        torch, rtp, D = self.torch, self.rtp, self.cfg.head_dim
        self.gen = torch.tensor([self.n0, self.n0], dtype=torch.int64, device="cuda")
        self.knew, self.vnew, self.kpnew = self.k_new[0].clone(), self.v_new[0].clone(), self.k_pre[0].clone()

        def pair():
            rtp.rtp_append_token_dev(self.L, self.gen, self.knew, self.vnew, self.kpnew, self.w_k, D * 16, self.kr,
                                     self.vr, self.kidx, self.kl, self.vl)
            self.step.run_dev(self.gen, self.q_pre, self.q, self.kr, self.vr, self.kidx, self.w_q, k_loc=self.kl,
                              v_loc=self.vl)
        pair()
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            pair()
        torch.cuda.synchronize()

    def run_graph(self):
        self.gen.fill_(self.n0)
        for _ in range(self.T):
            self.graph.replay()

    def capture_layers(self, n_layers: int):
        """One HIP graph per token that holds n_layers layers' [append, step] pairs, as a
        model's per-token decode graph would: every layer has its own caches and device
        state {pos, n_ctx}; the layers share the new-token vectors, the weights and the step's
        workspace (each call leaves it zeroed).  The first layer is this workload's own."""
        torch, rtp, D = self.torch, self.rtp, self.cfg.head_dim
        own = (self.kr, self.vr, self.kidx, self.kl, self.vl)
        self.layers = [own] + [tuple(t.clone() for t in own) for _ in range(n_layers - 1)]
        self.gens = [torch.tensor([self.n0, self.n0], dtype=torch.int64, device="cuda") for _ in range(n_layers)]

        def token():
            for (kr, vr, kidx, kl, vl), gen in zip(self.layers, self.gens):
                rtp.rtp_append_token_dev(self.L, gen, self.knew, self.vnew, self.kpnew, self.w_k, D * 16, kr, vr,
                                         kidx, kl, vl)
                self.step.run_dev(gen, self.q_pre, self.q, kr, vr, kidx, self.w_q, k_loc=kl, v_loc=vl)
        token()
        torch.cuda.synchronize()
        self.graph_layers = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph_layers):
            token()
        torch.cuda.synchronize()

    def run_graph_layers(self):
        for g in self.gens:
            g.fill_(self.n0)
        for _ in range(self.T):
            self.graph_layers.replay()


# ----------------------------------------------------------------------------- prefill
class PrefillBench:
    def __init__(self, name: str = "prefill_32k", q_distinct: int = 0):
        """q_distinct > 0: draw only that many distinct query chunks and cycle them (the
        prefill's work does not depend on the values; drawing all 64 chunks of the 1M
        workload would take minutes of host time)."""
        import torch
        from head_wise_sparse_amd import rtp
        from head_wise_sparse_amd import workloads as W
        self.torch, self.rtp = torch, rtp
        self.cfg = cfg = W.CONFIGS[name]
        t = time.time()
        self.pi = W.PrefillInputs(cfg)
        k, v, kp = self.pi.full_kv()
        nq = cfg.n_chunks if q_distinct <= 0 else min(q_distinct, cfg.n_chunks)
        qs = [self.pi.q_chunk(c) for c in range(nq)]
        log(f"prefill inputs drawn in {time.time() - t:.1f}s")
        dev = rtp.to_device_bf16
        self.L = rtp.Layer(1, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len, cfg.kv_role.tolist(),
                           cfg.n_sinks, cfg.window)
        self.k, self.v = dev(k), dev(v)
        self.k_pre = [dev(kp[c * cfg.chunk:(c + 1) * cfg.chunk]) for c in range(cfg.n_chunks)]
        self.q = [dev(q) for q in qs]
        del k, v, kp, qs
        self.w = dev(self.pi.w_k_idx)
        self.k_idx = torch.zeros(cfg.n_kv_r * cfg.seq_len * 16, dtype=torch.bfloat16, device="cuda")
        self.out = [torch.empty(cfg.chunk * cfg.n_q_heads * cfg.head_dim, dtype=torch.bfloat16, device="cuda")
                    for _ in range(len(self.q))]
        self.ws = rtp.workspace(self.L, cfg.chunk, rtp.CALL_PREFILL)
        self.sm = 1.0 / math.sqrt(cfg.head_dim)
        torch.cuda.synchronize()

    def run(self):
        cfg, rtp = self.cfg, self.rtp
        for c in range(cfg.n_chunks):
            c0, c1 = self.pi.chunk_bounds(c)
            j = c % len(self.q)
            rtp.rtp_prefill_attn(self.L, c0, c1 - c0, self.q[j], self.k, self.v, self.k_pre[c], self.w,
                                 cfg.head_dim * 16, self.k_idx, self.sm, self.out[j], self.ws)

    def flops(self):
        """Algorithmic FLOPs: 4*D per attended (row, key) pair, exact mask pair counts, plus the projection."""
        cfg = self.cfg
        T, D, G = cfg.seq_len, cfg.head_dim, cfg.group
        n_ret_q = cfg.n_kv_r * G
        n_loc_q = (cfg.n_kv_heads - cfg.n_kv_r) * G
        dense_pairs = T * (T + 1) // 2
        i = np.arange(T, dtype=np.int64)
        s = np.minimum(cfg.n_sinks, i + 1)
        wlo = np.maximum(s, i - cfg.window + 1)           # window part not already counted as sinks
        band_pairs = int((s + (i + 1 - wlo)).sum())
        attn = 4 * D * (dense_pairs * n_ret_q + band_pairs * n_loc_q)
        proj = 2 * T * D * 16 * cfg.n_kv_r
        return {"dense_pairs_per_head": dense_pairs, "band_pairs_per_head": band_pairs, "attn": attn,
                "kidx_proj": proj, "total": attn + proj}


# ----------------------------------------------------------------------------- CPU baseline
def host_identity():
    """CPU model of this host and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def cpu_baseline(dec: DecodeBench, prefill: bool = True):
    """The fp64 oracle, single-threaded, on a bounded sample of each workload.

    Decode: each batch entry of the 128K step once (all 32 heads), the time per entry
    scaled by the batch size to a whole step.  Prefill (32K in 4K chunks): the indexer-key
    projection of the whole sequence plus the seeded sample rows of every head, measured;
    the time per sampled row times the 32768 x 32 rows of the pass is reported as an
    extrapolation."""
    from threadpoolctl import threadpool_limits
    from oracle import rtp_oracle as O
    x, cfg = dec.x, dec.cfg
    host = host_identity()
    with threadpool_limits(limits=1):
        t0 = time.time()
        for b in range(cfg.batch):
            O.decode_step(x.q_pre, x.q, x.k, x.v, x.k_idx, x.w_q_idx, x.kv_role, cfg.n_ctx, cfg.top_p, cfg.n_sinks,
                          cfg.window, batch_rows=[b])
        per_entry = (time.time() - t0) / cfg.batch
    res = {"value": round(per_entry * cfg.batch * 1e6, 1), "unit": "us/step/layer", "cores": 1, "kind": "oracle",
           "sample": f"each of the {cfg.batch} batch entries of the 128K decode step once (all 32 heads, p=0.95), "
                     f"fp64 numpy on 1 thread: the whole step, measured",
           **host}
    if prefill:
        res["prefill"] = cpu_baseline_prefill()
    return res


def cpu_baseline_prefill(max_rows_per_head: int = 64):
    """The oracle's prefill leg (see cpu_baseline)."""
    from threadpoolctl import threadpool_limits
    from head_wise_sparse_amd import workloads as W
    from oracle import rtp_oracle as O
    cfg = W.CONFIGS["prefill_32k"]
    pi = W.PrefillInputs(cfg)
    k, v, kp = pi.full_kv()
    G = cfg.group
    rows_of = {h: pi.sample_rows(h)[:max_rows_per_head] for h in range(cfg.n_q_heads)}
    qrows = {}
    for h, rows in rows_of.items():
        chunks = {}
        for r in rows:
            c = int(r) // cfg.chunk
            if c not in chunks:
                chunks[c] = pi.q_chunk(c, heads=[h])
        qrows[h] = np.stack([chunks[int(r) // cfg.chunk][int(r) % cfg.chunk, h] for r in rows])
    with threadpool_limits(limits=1):
        t0 = time.time()
        O.prefill_kidx(kp, pi.w_k_idx, cfg.kv_role)
        t_proj = time.time() - t0
        t1 = time.time()
        n_rows = 0
        for h, rows in rows_of.items():
            g = h // G
            O.prefill_rows(qrows[h], rows, k[g], v[g], bool(cfg.kv_role[g]), cfg.n_sinks, cfg.window)
            n_rows += len(rows)
        t_rows = time.time() - t1
    per_row = t_rows / n_rows
    total_rows = cfg.seq_len * cfg.n_q_heads
    return {"measured_s": round(t_proj + t_rows, 3), "projection_s": round(t_proj, 3),
            "sampled_rows": n_rows, "rows_s": round(t_rows, 3),
            "extrapolated_ms_per_pass": round((t_proj + per_row * total_rows) * 1e3, 1),
            "extrapolation": f"time per sampled row x {cfg.seq_len} rows x {cfg.n_q_heads} heads + the measured "
                             "projection (an estimate, not a measurement)",
            "sample": f"32K prefill (4K chunks): indexer-key projection of all {cfg.seq_len} tokens and "
                      f"{max_rows_per_head} seeded query rows of each of the {cfg.n_q_heads} heads, fp64 numpy on "
                      "1 thread", "cores": 1}


def selection_rows(args):
    """rtp_topp_select alone on two 1M-token score rows: a peaked row (scores N(0, 3^2)) and a
    near-flat one (5 + 1e-3 N(0,1)), where many tokens share the threshold's upper key bits and
    every selection tile holds more distinct candidates than its record keeps."""
    import torch
    from head_wise_sparse_amd import rtp
    ev = lambda: torch.cuda.Event(enable_timing=True)
    n = 1 << 20
    rng = np.random.default_rng(3)
    rows = {"peaked": (rng.standard_normal(n) * 3).astype(np.float32),
            "near_flat": (5 + rng.standard_normal(n) * 1e-3).astype(np.float32)}
    L = rtp.Layer(1, 1, 1, 128, n, [1], 0, 1)
    out = {}
    for name, r in rows.items():
        sc = torch.from_numpy(r).cuda()
        m = torch.tensor([float(r.max())], device="cuda")
        z = torch.tensor([float(np.exp(r.astype(np.float64) - r.max()).sum())], device="cuda")
        sel = torch.empty(n, dtype=torch.int32, device="cuda")
        cnt = torch.empty(1, dtype=torch.int32, device="cuda")
        ws = rtp.workspace(L, n, rtp.CALL_TOPP_SELECT)
        for _ in range(3):
            rtp.rtp_topp_select(L, n, sc, m, z, 0.95, sel, cnt, None, ws)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(args.steps):
            rtp.rtp_topp_select(L, n, sc, m, z, 0.95, sel, cnt, None, ws)
        b.record()
        torch.cuda.synchronize()
        out[name] = {"us_per_call": round(a.elapsed_time(b) / args.steps * 1e3, 2), "selected": int(cnt.item())}
        log(f"selection 1M {name}: {out[name]}")
    return out


HEADLINE_DECODE, HEADLINE_PREFILL = "decode_b4_128k", "prefill_32k"   # the workloads `value` and `prefill` time
DECODE_CONFIGS = (("decode_tiny_2k", 0.9, 3), ("decode_b8_32k", 0.95, 3), ("decode_b4_128k", 0.95, 3),
                  ("decode_b1_1m", 0.95, 2))        # (workload, p, cache copies rotated across steps)
PREFILL_CONFIGS = (("prefill_32k", 0, None), ("prefill_1m", 4, 2))  # (workload, distinct query chunks, passes)


def config_timings(args, names):
    """The fused decode step of each named decode workload at its p (args.steps steps after
    warm-up, rotating cache copies), and the chunked prefill of each named prefill workload."""
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)
    out = {}
    for name, p, copies in DECODE_CONFIGS:
        if name not in names:
            continue
        dec = DecodeBench(copies, name)
        for i in range(max(args.warmup, len(dec.sets))):
            dec.step(p, i)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for i in range(args.steps):
            dec.step(p, i)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / args.steps * 1e3
        ab = dec.algorithmic_bytes(p)
        gbs = ab["total"] / (us * 1e-6) / 1e9
        out[name] = {"p": p, "us_per_step": round(us, 2), "hbm_GBps": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": ab["total"],
                     "union_tokens": ab["union_tokens"], "sel_mean": ab["sel_mean"], "sel_median": ab["sel_median"],
                     "steps": args.steps}
        log(f"{name}: {us:.1f} us/step")
        del dec
        torch.cuda.empty_cache()
    for name, qd, passes in PREFILL_CONFIGS:
        if name not in names:
            continue
        passes = passes or args.steps
        pre = PrefillBench(name, qd)
        pre.run()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(passes):
            pre.run()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / passes
        fl = pre.flops()["total"]
        tf = fl / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 3), "tflops": round(tf, 1), "mfma_util": round(tf / BF16_PEAK_TFLOPS, 4),
                     "algorithmic_flops": fl, "chunks": pre.cfg.n_chunks, "distinct_q_chunks": len(pre.q),
                     "passes": passes}
        log(f"{name}: {ms:.2f} ms")
        del pre
        torch.cuda.empty_cache()
    return out


def report_configs(args):
    """Per-config timings of every workload (one JSON report line, not the headline line),
    plus top-p selection alone on two 1M-token rows."""
    import torch
    from head_wise_sparse_amd import rtp
    torch.cuda.set_device(0)
    names = [c[0] for c in DECODE_CONFIGS] + [c[0] for c in PREFILL_CONFIGS]
    out = {"report": "per-config timings", "device": torch.cuda.get_device_name(0), "rtp": rtp.rtp_version(),
           "data": "synthetic (seeded)", "configs": config_timings(args, names)}
    out["selection_rows"] = selection_rows(args)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.report_configs:
        report_configs(args)
        return
    if args.only == "prefill_1m":          # the 1M-token prefill alone (for profiling): one report line
        import torch
        torch.cuda.set_device(0)
        print(json.dumps({"report": "prefill_1m timing", "configs": config_timings(args, ["prefill_1m"])}), flush=True)
        return
    import torch
    from head_wise_sparse_amd import rtp
    torch.cuda.set_device(0)
    log(f"device {torch.cuda.get_device_name(0)}, {rtp.rtp_version()}")
    ev = lambda: torch.cuda.Event(enable_timing=True)

    do_dec = args.only in (None, "decode")
    do_pre = args.only in (None, "prefill") and not args.no_prefill
    dec = DecodeBench(args.copies) if do_dec else None
    pre = None
    if do_pre:
        pre = PrefillBench()
        try:
            pre.run()
            torch.cuda.synchronize()
        except rtp.RtpError as e:
            log(f"prefill unavailable: {e}")
            pre = None

    p0 = 0.95
    if dec:                                  # capture the graph of every cache copy before timing
        for i in range(len(dec.sets)):
            dec.graph(p0, i)
    for i in range(args.warmup):
        if dec:
            dec.step(p0, i)
        if pre:
            pre.run()
    torch.cuda.synchronize()

    # Decode: K fused steps enqueued back to back (direct launches, rotating cache copies),
    # HIP events on the launch stream around all of them; then the K prefill passes likewise.
    wall0 = time.time()
    e_all0, e_all1 = ev(), ev()
    e_all0.record()
    dec_ms = pre_ms = None
    if dec:
        a, b = ev(), ev()
        a.record()
        for i in range(args.steps):
            dec.step(p0, i)
        b.record()
    if pre:
        c, d = ev(), ev()
        c.record()
        for i in range(args.steps):
            pre.run()
        d.record()
    e_all1.record()
    torch.cuda.synchronize()
    wall = time.time() - wall0
    ms_step = e_all0.elapsed_time(e_all1) / args.steps
    if dec:
        dec_ms = a.elapsed_time(b) / args.steps
    if pre:
        pre_ms = c.elapsed_time(d) / args.steps

    res = {"metric": "sparse decode us/step/layer + HBM GB/s @128K; prefill attn ms + MFMA util",
           "value": round(dec_ms * 1e3, 3) if dec_ms is not None else None, "unit": "us/step/layer",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; needles planted in the indexer keys; no datasets or trained weights)",
           "config": {"workload": "decode 128K x batch 4, 32q/8kv heads d128, 2 retrieval KV heads p=0.95, "
                                  "6 local KV heads (4 sinks + 4096 window); + prefill 32K in 4K chunks",
                      "decode": "decode_b4_128k", "prefill": "prefill_32k"}}
    rooflines = {}
    if dec:
        ab = dec.algorithmic_bytes(p0)
        calls = dec.call_times(p0)
        gbs = ab["total"] / (dec_ms * 1e-3) / 1e9
        res["decode"] = {"us_per_step": round(dec_ms * 1e3, 2), "launch": "direct (rtp_decode_step per step)",
                         "hbm_GBps": round(gbs, 1),
                         "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bytes": ab,
                         "call_us": {k: round(v * 1e3, 2) for k, v in calls.items()}}
        sp_bytes = ab["gathered_kv_union"] + 2 * 2 * dec.cfg.head_dim * dec.cfg.batch * dec.cfg.n_kv_r * dec.cfg.group
        sp_gbs = sp_bytes / (calls["sparse_decode"] * 1e-3) / 1e9
        rooflines["sparse_decode"] = {"bound": "hbm", "achieved": round(sp_gbs, 1), "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": round(sp_gbs / HBM_PEAK_GBS, 4),
                                      "traffic": measured_traffic("sparse_decode"), "algorithmic_bytes": sp_bytes,
                                      "kernel": "rtp_sparse_decode_attn (k_decode_partial + k_decode_merge)", "us": round(calls["sparse_decode"] * 1e3, 2)}
        # for reference: the four separate calls in one graph, and the fused call replayed
        # from a HIP graph (consecutive replays leave the GPU idle between them on this stack)
        for i in range(len(dec.sets)):
            dec.graph(p0, i, "separate").replay()
            dec.step_graph(p0, i)
        torch.cuda.synchronize()
        a, b, c, d = ev(), ev(), ev(), ev()
        a.record()
        for i in range(10):
            dec.graph(p0, i, "separate").replay()
        b.record()
        for i in range(10):
            dec.step_graph(p0, i)
        c.record()
        torch.cuda.synchronize()
        res["decode"]["separate_calls_us_per_step"] = round(a.elapsed_time(b) / 10 * 1e3, 2)
        res["decode"]["graph_us_per_step"] = round(b.elapsed_time(c) / 10 * 1e3, 2)
        if not args.no_sweep:
            sweep = {}
            for p in (0.9, 0.99):
                for i in range(len(dec.sets)):
                    dec.step(p, i)
                torch.cuda.synchronize()
                a, b = ev(), ev()
                a.record()
                for i in range(10):
                    dec.step(p, i)
                b.record()
                torch.cuda.synchronize()
                us = a.elapsed_time(b) / 10 * 1e3
                abp = dec.algorithmic_bytes(p)
                sweep[str(p)] = {"us_per_step": round(us, 2),
                                 "hbm_GBps": round(abp["total"] / (us * 1e-6) / 1e9, 1),
                                 "sel_mean": round(abp["sel_mean"], 1), "union_tokens": abp["union_tokens"]}
            res["decode"]["p_sweep"] = sweep
    if dec:
        # the device's practical HBM read rate (plain streaming read of 4 GiB), the ceiling
        # the decode kernels' bandwidth is read against; the roofline peak stays 8 TB/s
        buf = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        for _ in range(2):
            rtp.rtp_hbm_read_probe(buf, sink)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(5):
            rtp.rtp_hbm_read_probe(buf, sink)
        b.record()
        torch.cuda.synchronize()
        read_tbs = 5 * buf.numel() * 4 / (a.elapsed_time(b) * 1e-3) / 1e12
        res["decode"]["hbm_read_probe_TBps"] = round(read_tbs, 2)
        res["decode"]["frac_of_read_probe"] = round(res["decode"]["hbm_GBps"] / 1e3 / read_tbs, 4)
        del buf
    if dec and args.gen_steps > 0:
        gen = GenBench(dec, args.gen_steps)
        gen.capture()
        gen.run_graph()                      # warm-up of the graph path
        gen.run()                            # warm-up (re-appending the same tokens is idempotent)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        gen.run()
        b.record()
        torch.cuda.synchronize()
        us_tok = a.elapsed_time(b) / gen.T * 1e3
        a, b = ev(), ev()
        a.record()
        gen.run_graph()
        b.record()
        torch.cuda.synchronize()
        us_tok_graph = a.elapsed_time(b) / gen.T * 1e3
        n_layers = 3
        gen.capture_layers(n_layers)
        gen.run_graph_layers()               # warm-up
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        gen.run_graph_layers()
        b.record()
        torch.cuda.synchronize()
        us_tok_layers = a.elapsed_time(b) / (gen.T * n_layers) * 1e3
        del gen.layers[1:], gen.graph_layers
        gen.run()                            # restore the generated tokens' cache rows
        torch.cuda.synchronize()
        res["generation"] = {
            "workload": f"{gen.T} tokens generated from {gen.n0} to {gen.n0 + gen.T}, batch {dec.cfg.batch}, "
                        "compact KV (retrieval heads: whole history; local heads: sinks + window ring), "
                        "append + fused decode step per token",
            "us_per_token_per_layer": round(us_tok, 2),
            "launch": "eager (host context length per token)",
            "graph_us_per_token_per_layer": round(us_tok_graph, 2),
            "graph": "one captured graph of rtp_append_token_dev + rtp_decode_step_dev replayed per token "
                     "(context length in device memory)",
            "graph_3_layers_us_per_token_per_layer": round(us_tok_layers, 2),
            "graph_3_layers": "one captured graph per token holding three layers' append + step pairs "
                              "(each layer its own caches and device length), replayed per token",
            "kv_bytes_full_layout": gen.full_bytes, "kv_bytes_compact_layout": gen.compact_bytes,
            "memory_sparsity": round(1 - gen.compact_bytes / gen.full_bytes, 4)}
        del gen
    if pre:
        fl = pre.flops()
        tflops = fl["total"] / (pre_ms * 1e-3) / 1e12
        res["prefill"] = {"ms": round(pre_ms, 3), "tflops": round(tflops, 1),
                          "mfma_util": round(tflops / BF16_PEAK_TFLOPS, 4), "flops": fl}
        # the dense bf16 MFMA rate this chip sustains (4 independent 32x32x16 chains per
        # wave, 2 waves per SIMD: its clock under an MFMA load), the ceiling the prefill's
        # rate is read against; the roofline peak stays 2.5 PFLOP/s
        sink = torch.zeros(1, dtype=torch.float32, device="cuda")
        for _ in range(2):
            rtp.rtp_mfma_probe(20000, sink)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        pfl = sum(rtp.rtp_mfma_probe(100000, sink) for _ in range(3))
        b.record()
        torch.cuda.synchronize()
        probe_tf = pfl / (a.elapsed_time(b) * 1e-3) / 1e12
        res["prefill"]["mfma_probe_TFLOPs"] = round(probe_tf, 1)
        res["prefill"]["frac_of_mfma_probe"] = round(tflops / probe_tf, 4)
        rooflines["prefill_attn"] = {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                                     "traffic": measured_traffic("prefill_attn"),
                                     "kernel": "rtp_prefill_attn (k_prefill_attn: attention blocks + indexer-key projection blocks)",
                                     "ms_per_chunk": round(pre_ms / pre.cfg.n_chunks, 4)}
    # the dominant kernel of the step is the one that takes the most time
    if rooflines:
        dom = "prefill_attn" if "prefill_attn" in rooflines else "sparse_decode"
        res["roofline"] = rooflines[dom]
        res["rooflines"] = rooflines
    if dec and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(dec, prefill=pre is not None)
    res["wall_s_timed"] = round(wall, 3)
    if dec and pre and not args.no_configs:
        # the other workloads, timed in this same run (not part of `value`)
        dec = pre = None
        torch.cuda.empty_cache()
        others = [c[0] for c in DECODE_CONFIGS if c[0] != HEADLINE_DECODE] + \
                 [c[0] for c in PREFILL_CONFIGS if c[0] != HEADLINE_PREFILL]
        res["other_configs"] = config_timings(args, others)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
