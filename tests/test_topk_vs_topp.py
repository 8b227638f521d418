"""Top-p against the static top-k rule at the same total budget (the comparison the
abstract's observation (3) rests on), on the oracle, for the 32K decode workload.

Measured on the indexer's own softmax: the mass each row's set captures.  Top-p gives
every row at least p by construction with a per-row budget; top-k with the same mean
budget spends it uniformly, so rows whose mass is spread get less than p and peaked
rows get more than they need.  (Attention-mass recall is not used: on synthetic inputs
the indexer and the attention logits are unrelated, so it would measure nothing.)
Run with -s to see the table.
"""
import numpy as np

from head_wise_sparse_amd import workloads as W
from oracle import rtp_oracle as O


def test_topk_vs_topp_equal_budget_report():
    cfg = W.scaled_decode(W.CONFIGS["decode_b8_32k"], batch=4)
    x = W.make_decode_inputs(cfg)
    G, p = cfg.group, cfg.top_p
    rows = []
    for b in range(cfg.batch):
        for ci in range(cfg.n_kv_r * G):
            r = ci // G
            g = cfg.retrieval_kv[r]
            qi = O.indexer_query(O.bf16_to_f64(x.q_pre[b, g * G + ci % G]), O.bf16_to_f64(x.w_q_idx[ci]))
            rows.append(O.indexer_scores(qi, O.bf16_to_f64(x.k_idx[b, r, :cfg.n_ctx])))
    sizes, mass_p = [], []
    for s in rows:
        sel, info = O.topp_select(s, p)
        sizes.append(sel.size)
        mass_p.append(O.softmax_mass(s)[sel].sum())
    k = int(round(np.mean(sizes)))
    mass_k = [O.softmax_mass(s)[O.topk_select(s, k)].sum() for s in rows]
    mass_p, mass_k = np.array(mass_p), np.array(mass_k)
    print(f"\n32K decode, {len(rows)} retrieval rows, p={p}: top-p budget min {min(sizes)} median "
          f"{int(np.median(sizes))} mean {np.mean(sizes):.0f} max {max(sizes)}")
    print(f"  top-p: indexer mass min {mass_p.min():.4f} mean {mass_p.mean():.4f}; "
          f"rows below p: {(mass_p < p - 1e-9).sum()}")
    print(f"  top-k (k={k}, same mean budget): mass min {mass_k.min():.4f} mean {mass_k.mean():.4f}; "
          f"rows below p: {(mass_k < p - 1e-9).sum()}")
    assert (mass_p >= p - 1e-9).all()                      # the rule itself
    assert np.isclose(np.mean(sizes), k, atol=0.5)
