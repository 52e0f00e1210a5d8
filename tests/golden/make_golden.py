"""Write oracle regression fixtures (text JSON) for a small seeded workload.

The pages print no worked example with numbers, so nothing here is the
pages' own value.  This script calls only the oracle (and the seeded input
generator) and freezes its output, so that any later change to the oracle's
arithmetic shows up as a failing regression test and has to be justified.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from sparse_attention_long_amd import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")


def fixture_workload():
    return W.small("golden", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, ctx=None,
                   ctx_range=(150, 260), gamma=3, budget=40, n_sink=4, window=16, planted=4,
                   seed=424242)


def compute():
    w = fixture_workload()
    x = W.make_layer(w)
    o, lse = oracle.verify_attention(x.q, x.k, x.v, x.seq_lens)
    logits = oracle.collected_logits(x.q, x.k, x.seq_lens, w.collect_rows)
    scores = oracle.aggregate_scores(oracle.kvgroup_sum(logits, w.num_kv_heads))
    idx = oracle.select_topk_batch(scores, x.seq_lens, w.budget, w.n_sink, w.window)
    so, slse = oracle.sparse_attention(x.q, x.k, x.v, x.seq_lens, idx)
    probe_rows = [(0, 0, 0), (0, 5, 3), (1, 7, 2), (1, 2, 0)]
    probe_pos = [0, 17, 100, 140]
    return {
        "workload": {k: getattr(w, k) for k in ("batch", "num_q_heads", "num_kv_heads", "head_dim",
                                                "gamma", "budget", "n_sink", "window", "seed")},
        "ctx_range": list(w.ctx_range),
        "seq_lens": [int(L) for L in x.seq_lens],
        "planted": [p.tolist() for p in x.planted],
        "selected": [i.tolist() for i in idx],
        "verify_o_first4": {f"{b},{h},{t}": o[b, h, t, :4].tolist() for b, h, t in probe_rows},
        "verify_lse": {f"{b},{h},{t}": float(lse[b, h, t]) for b, h, t in probe_rows},
        "sparse_o_first4": {f"{b},{h},{t}": so[b, h, t, :4].tolist() for b, h, t in probe_rows},
        "sparse_lse": {f"{b},{h},{t}": float(slse[b, h, t]) for b, h, t in probe_rows},
        "scores": {f"{b},{j}": float(scores[b, j]) for b in range(2) for j in probe_pos},
    }


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", OUT)
