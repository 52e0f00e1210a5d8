"""GPU parity at the full workload sizes, on sampled outputs.

Every workload runs the whole per-layer iteration on the GPU in the launch
configuration the benchmark times (same descriptors, same split plans):
verify with the kv-group-summed logit epilogue, aggregate, select, then the
sparse pass (sparse verify over the T rows and/or single-query draft steps
whose lists carry the freshly drafted positions).  The oracle checks:
  * selection for every sequence, bit-exact on the GPU's own scores;
  * for rows of up to 65536 positions, the benchmark's form (verify partials,
    then combine + aggregate + select in one launch) gives the same scores and
    selection bit for bit, and outputs within the oracle bar;
  * outputs, lse, collected logits and scores of every sequence, element by
    element, on kv-head b mod Hkv of sequence b (plus the first and last
    kv-heads for the first and last sequences).  Every sequence matters: the
    ragged verify hands a long sequence's extra items to the workgroups of
    other sequences.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_long_amd import binding as Bn
from sparse_attention_long_amd import workloads as W
from tests.gpu_helpers import (assert_lse_close, assert_logits_close, assert_out_close, dev_bf16,
                               dev_i32, say, to_device)

pytestmark = pytest.mark.gpu

FULL = ["ctx32k_b1_h32kv8_d128_draft4", "ctx32k_b16_h64kv8_d128", "ctx128k_b8_h32kv8_d128_draft6",
        "ragged8k-64k_b4_h64kv8_d64_paged16_l24"]


def sub(x, b):
    return x[b:b + 1]


@pytest.mark.parametrize("name", FULL)
def test_fullsize_sampled(name):
    w = W.WORKLOADS[name]
    layers = [0] if w.layers == 1 else [0, w.layers - 1]
    for layer in layers:
        say(f"[fullsize] {name} layer {layer}: generating")
        x = W.make_layer(w, layer)
        d = to_device(x)
        say(f"[fullsize] {name} layer {layer}: gpu iteration")
        out, lse, lg = Bn.verify_attention(d.q, d.k, d.v, d.seq_lens, block_table=d.block_table,
                                           max_ctx=d.max_ctx, collect_rows=w.collect_rows,
                                           layout="kvgroup_sum")
        scores = Bn.aggregate_scores(lg, d.seq_lens, w.num_q_heads, w.num_kv_heads)
        stride = w.budget
        idx, n_idx = Bn.select_topk(scores, d.seq_lens, w.budget, w.n_sink, w.window,
                                    idx_stride=stride)
        torch.cuda.synchronize()
        sc = scores.cpu().numpy()
        lens = [int(L) for L in x.seq_lens]
        say(f"[fullsize] {name} layer {layer}: oracle selection")
        want = oracle.select_topk_batch(sc, lens, w.budget, w.n_sink, w.window)
        idx_h, n_h = idx.cpu().numpy(), n_idx.cpu().numpy()
        for b in range(w.batch):
            assert n_h[b] == len(want[b])
            assert np.array_equal(idx_h[b, :n_h[b]], want[b]), f"{name} idx b={b}"
            assert set(x.planted[b].tolist()) <= set(want[b].tolist()), f"planted key dropped b={b}"

        # the benchmark's form for rows of up to 65536 positions: verify partials,
        # then the split combine, the score aggregation and the selection in one
        # launch (vgsa_verify_finish_select)
        out_f = lse_f = None
        if d.max_ctx <= 65536:
            say(f"[fullsize] {name} layer {layer}: verify partials + finish-select")
            desc = Bn.make_desc(d.q, d.k, d.block_table, d.max_ctx)
            ws = torch.empty(Bn.verify_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
            lg_f = torch.empty_like(lg)
            Bn.verify_partials(desc, d.q, d.k, d.v, d.seq_lens, d.block_table, w.collect_rows,
                               Bn.LOGITS_KVGROUP_SUM, lg_f, ws)
            out_f, lse_f = torch.empty_like(out), torch.empty_like(lse)
            sc_f = torch.empty_like(scores)
            idx_f = torch.full_like(idx, -1)
            n_f = torch.empty_like(n_idx)
            sws = torch.zeros(Bn.finish_select_workspace_bytes(w.batch, d.max_ctx), dtype=torch.uint8,
                              device="cuda")
            Bn.verify_finish_select(desc, d.seq_lens, ws, out_f, lse_f, Bn.LOGITS_KVGROUP_SUM, lg_f,
                                    sc_f, w.budget, w.n_sink, w.window, idx_f, n_f, sws)
            torch.cuda.synchronize()
            for b in range(w.batch):
                L = lens[b]
                assert torch.equal(sc_f[b, :L], scores[b, :L]), f"{name} b={b} fused scores"
                assert int(n_f[b]) == n_h[b], f"{name} b={b} fused count"
                assert torch.equal(idx_f[b, :n_h[b]], idx[b, :n_h[b]]), f"{name} b={b} fused idx"

        G = w.group

        def heads_of(b):
            gs = {b % w.num_kv_heads}
            if b in (0, w.batch - 1):
                gs |= {0, w.num_kv_heads - 1}
            return sorted(gs), [h for g in sorted(gs) for h in range(g * G, (g + 1) * G)]

        lg_h = lg.cpu().numpy()
        for b in range(w.batch):
            say(f"[fullsize] {name} layer {layer}: oracle b={b}")
            gs, heads = heads_of(b)
            qb, kb, vb = sub(x.q, b), sub(x.k, b), sub(x.v, b)
            o_ref, lse_ref = oracle.verify_attention(qb, kb, vb, lens[b:b + 1], heads=heads)
            assert_out_close(out[b:b + 1, heads], o_ref[:, heads], f"{name} b={b} verify out")
            assert_lse_close(lse[b:b + 1, heads], lse_ref[:, heads], f"{name} b={b} verify lse")
            if out_f is not None:
                assert_out_close(out_f[b:b + 1, heads], o_ref[:, heads], f"{name} b={b} fused out")
                assert_lse_close(lse_f[b:b + 1, heads], lse_ref[:, heads], f"{name} b={b} fused lse")
            l_ref = oracle.collected_logits(qb, kb, lens[b:b + 1], w.collect_rows)
            absl = np.where(np.isneginf(l_ref), 0.0, np.abs(l_ref))
            grp = oracle.kvgroup_sum(l_ref, w.num_kv_heads)
            assert_logits_close(lg_h[b:b + 1, gs], grp[:, gs], f"{name} b={b} group logits",
                                floor=oracle.kvgroup_sum(absl, w.num_kv_heads)[:, gs])
            assert_logits_close(sc[b:b + 1], oracle.aggregate_scores(l_ref), f"{name} b={b} scores",
                                floor=oracle.aggregate_scores(absl))

        if w.sparse_verify:
            say(f"[fullsize] {name} layer {layer}: sparse verify")
            so, sl = Bn.sparse_attention(d.q, d.k, d.v, d.seq_lens, idx, n_idx,
                                         block_table=d.block_table, max_ctx=d.max_ctx)
            torch.cuda.synchronize()
            for b in range(w.batch):
                heads = heads_of(b)[1]
                o_ref, lse_ref = oracle.sparse_attention(sub(x.q, b), sub(x.k, b), sub(x.v, b),
                                                         lens[b:b + 1], [want[b]], heads=heads)
                assert_out_close(so[b:b + 1, heads], o_ref[:, heads], f"{name} b={b} sparse out")
                assert_lse_close(sl[b:b + 1, heads], lse_ref[:, heads], f"{name} b={b} sparse lse")

        for s in range(1, w.draft_steps + 1):
            say(f"[fullsize] {name} layer {layer}: draft step {s}")
            # step s: the kept list plus the s positions L..L+s-1 drafted since,
            # passed as the trailing positions of length L + s (as the benchmark does)
            lists = [np.concatenate([want[b], np.arange(lens[b], lens[b] + s)]) for b in range(w.batch)]
            lens_s = [L + s for L in lens]
            qd = dev_bf16(x.q_draft[s - 1])
            so, sl = Bn.sparse_attention(qd, d.k, d.v, dev_i32(lens_s), idx, n_idx, tail=s,
                                         block_table=d.block_table, max_ctx=d.max_ctx)
            torch.cuda.synchronize()
            for b in range(w.batch):
                heads = heads_of(b)[1]
                o_ref, lse_ref = oracle.sparse_attention(sub(x.q_draft[s - 1], b), sub(x.k, b),
                                                         sub(x.v, b), lens_s[b:b + 1], [lists[b]],
                                                         heads=heads)
                assert_out_close(so[b:b + 1, heads], o_ref[:, heads], f"{name} b={b} draft {s}")
                assert_lse_close(sl[b:b + 1, heads], lse_ref[:, heads], f"{name} b={b} draft {s} lse")
        del d
        torch.cuda.empty_cache()
