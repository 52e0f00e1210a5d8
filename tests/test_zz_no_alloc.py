"""The verify entry point that allocates nothing (its split partials live in
the library's static scratch) against the workspace entry point, through the
C ABI, on two calls in a row, the second with a smaller input: bit-identical
logits, out and lse equal to within fp32 accumulation order (the verify
kernel's wavefronts claim their tiles at run time), and against the oracle at
the parity bar."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_long_amd import binding as Bn
from sparse_attention_long_amd import workloads as W
from tests.gpu_helpers import assert_lse_close, assert_out_close, say, to_device

pytestmark = pytest.mark.gpu

CALLS = [
    # the headline shape: 42 MB of partials, 4 splits, balanced items
    ("ctx32k_b16_h64kv8_d128", W.WORKLOADS["ctx32k_b16_h64kv8_d128"], "kvgroup_sum", False),
    # then a smaller ragged paged input with per-head logits: the scratch
    # still holds the first call's partials, none of which may leak in
    ("paged_small", W.small("noalloc_pg", batch=3, num_q_heads=16, num_kv_heads=2, head_dim=64,
                            gamma=5, ctx=None, ctx_range=(300, 2600), paged=True, budget=48,
                            n_sink=4, window=12, seed=61), "per_head", True),
]


def _outputs(w, d, layout):
    B, Hq, T, dh = w.batch, w.num_q_heads, w.q_len, w.head_dim
    out = torch.empty((B, Hq, T, dh), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    R = len(w.collect_rows)
    shape = (B, R, Hq, d.max_ctx) if layout == "per_head" else (B, w.num_kv_heads, d.max_ctx)
    return out, lse, torch.empty(shape, dtype=torch.float32, device="cuda")


def test_noalloc_verify_matches_workspace_form_twice():
    for name, w, layout, check_oracle in CALLS:
        say(f"[noalloc verify] {name} {layout}")
        x = W.make_layer(w)
        d = to_device(x)
        out, lse, lg = _outputs(w, d, layout)
        Bn.verify_attention_noalloc(d.q, d.k, d.v, d.seq_lens, out, lse, lg,
                                    block_table=d.block_table, max_ctx=d.max_ctx,
                                    collect_rows=w.collect_rows, layout=layout)
        ref_out, ref_lse, ref_lg = Bn.verify_attention(d.q, d.k, d.v, d.seq_lens,
                                                       block_table=d.block_table,
                                                       max_ctx=d.max_ctx,
                                                       collect_rows=w.collect_rows, layout=layout)
        torch.cuda.synchronize()
        # the same kernels on the same plan: identical logits; out and lse up
        # to the order in which each wavefront accumulated its tiles
        np.testing.assert_allclose(out.float().cpu().numpy(), ref_out.float().cpu().numpy(),
                                   atol=8e-3, rtol=1e-2, err_msg=f"{name} out")
        np.testing.assert_allclose(lse.cpu().numpy(), ref_lse.cpu().numpy(), atol=1e-5, rtol=0,
                                   err_msg=f"{name} lse")
        for b, L in enumerate(x.seq_lens):
            assert torch.equal(lg[b, ..., :int(L)], ref_lg[b, ..., :int(L)]), f"{name} logits b={b}"
        if check_oracle:
            o_ref, lse_ref = oracle.verify_attention(x.q, x.k, x.v, x.seq_lens)
            assert_out_close(out, o_ref, f"{name} noalloc out")
            assert_lse_close(lse, lse_ref, f"{name} noalloc lse")
        del d
        torch.cuda.empty_cache()
