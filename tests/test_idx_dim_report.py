"""Top-p budget against the indexer dimension (the ablation of the research-map summary,
"Surprising findings": a lower indexer dimension kept more tokens), on the oracle, for
the 32K decode workload with its own seeded weights at d = 4, 8, 16, 32.

On these synthetic inputs the score spread grows with d (q_idx is a d-dim projection),
so at fixed p a smaller d gives flatter rows and larger sets -- the direction the pages
report; the accuracy side of the ablation needs trained weights and stays out of scope.
Run with -s to see the table.
"""
import numpy as np

from head_wise_sparse_amd import workloads as W
from oracle import rtp_oracle as O


def _budgets(d):
    cfg = W.scaled_decode(W.CONFIGS["decode_b8_32k"], batch=2, idx_dim=d)
    x = W.make_decode_inputs(cfg)
    G = cfg.group
    sizes = []
    for b in range(cfg.batch):
        for ci in range(cfg.n_kv_r * G):
            r = ci // G
            g = cfg.retrieval_kv[r]
            qi = O.indexer_query(O.bf16_to_f64(x.q_pre[b, g * G + ci % G]), O.bf16_to_f64(x.w_q_idx[ci]))
            s = O.indexer_scores(qi, O.bf16_to_f64(x.k_idx[b, r, :cfg.n_ctx]))
            sel, _ = O.topp_select(s, cfg.top_p)
            sizes.append(sel.size)
    return np.array(sizes), cfg.n_ctx


def test_topp_budget_against_indexer_dim():
    rows = {}
    for d in (4, 8, 16, 32):
        sizes, n = _budgets(d)
        rows[d] = sizes
        print(f"\nd={d:2d}: |S| median {int(np.median(sizes))} mean {sizes.mean():.0f} "
              f"(compute sparsity {1 - sizes.mean() / n:.3f})", end="")
    print()
    assert all(len(v) == len(rows[16]) for v in rows.values())
    assert all((v >= 1).all() for v in rows.values())
