"""Block lists (structured block sparsity): vgsa_select_block_ids against the
position form of block selection and the oracle, and
vgsa_sparse_attention_blocks against the oracle on the positions the blocks
expand to (oracle.block_positions) and against vgsa_sparse_attention on that
expanded list (same entries in the same order and the same split plan, so
identical bytes)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_long_amd import binding as Bn
from sparse_attention_long_amd import workloads as W
from tests.gpu_helpers import assert_lse_close, assert_out_close, dev_i32, say, to_device

pytestmark = pytest.mark.gpu

CASES = {
    "g4t5_d64": W.small("bl_g4t5", batch=2, num_q_heads=16, num_kv_heads=4, head_dim=64, gamma=4,
                        lens=(33, 257), budget=24, n_sink=2, window=6, seed=11),
    "g8t5_d128": W.small("bl_g8t5", batch=2, num_q_heads=16, num_kv_heads=2, head_dim=128, gamma=4,
                         lens=(700, 129), budget=64, n_sink=4, window=16, seed=12),
    "paged_g8t6_d64": W.small("bl_pg", batch=3, num_q_heads=16, num_kv_heads=2, head_dim=64,
                              gamma=5, ctx=None, ctx_range=(40, 300), paged=True, budget=48,
                              n_sink=4, window=12, seed=15),
    # long lists: several splits per (sequence, kv-head), merged in the launch
    "long_paged_g4t3_d128": W.small("bl_long", batch=2, num_q_heads=8, num_kv_heads=2,
                                    head_dim=128, gamma=2, lens=(33000, 20001), paged=True,
                                    budget=4096, n_sink=4, window=64, seed=18),
}


def _random_ids(rng, lens_sel, block, count, stride):
    """Ascending distinct block ids below ceil(L / block) per sequence (the
    last block, often partial, included every other row), padded with -1."""
    ids = np.full((len(lens_sel), stride), -1, np.int32)
    n = np.zeros(len(lens_sel), np.int32)
    for b, L in enumerate(lens_sel):
        nb = -(-int(L) // block)
        m = min(count, nb)
        pick = np.sort(rng.choice(nb, size=m, replace=False)) if m else np.zeros(0, np.int64)
        if b % 2 == 0 and m and pick[-1] != nb - 1:
            pick[-1] = nb - 1
            pick = np.unique(pick)
        ids[b, :len(pick)] = pick
        n[b] = len(pick)
    return ids, n


def _expand(ids, n, block, lens_sel, stride_pos):
    idx = np.zeros((ids.shape[0], stride_pos), np.int32)
    cnt = np.zeros(ids.shape[0], np.int32)
    lists = []
    for b in range(ids.shape[0]):
        pos = oracle.block_positions(ids[b, :n[b]], block, int(lens_sel[b]))
        idx[b, :len(pos)] = pos
        cnt[b] = len(pos)
        lists.append(pos)
    return idx, cnt, lists


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("block", [16, 5, 64])
def test_sparse_blocks_equal_expanded_positions(name, block):
    w = CASES[name]
    x = W.make_layer(w)
    d = to_device(x)
    rng = np.random.default_rng(31 * block + list(CASES).index(name))
    count = max(2, w.budget // block + 1)
    for T, tail in ((w.q_len, 0), (1, 3)):
        say(f"[block lists] {name} block={block} T'={T} tail={tail}")
        q = d.q[:, :, :T].contiguous()
        lens_t = np.asarray(x.seq_lens, np.int32)
        lens_sel = np.maximum(lens_t - tail, 1)
        ids, n = _random_ids(rng, lens_sel, block, count, count + 2)
        if w.batch > 2:
            n[1] = 0  # an empty block list (the tail alone, or nothing)
        out, lse = Bn.sparse_attention_blocks(q, d.k, d.v, dev_i32(lens_t), dev_i32(ids), dev_i32(n),
                                              block, block_table=d.block_table, max_ctx=d.max_ctx,
                                              tail=tail)
        stride_pos = ids.shape[1] * block
        idx, cnt, lists = _expand(ids, n, block, lens_sel, stride_pos)
        out2, lse2 = Bn.sparse_attention(q, d.k, d.v, dev_i32(lens_t), dev_i32(idx), dev_i32(cnt),
                                         block_table=d.block_table, max_ctx=d.max_ctx, tail=tail)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), (name, block, tail)
        assert torch.equal(lse, lse2), (name, block, tail)
        ref_lists = [np.concatenate([lists[b], np.arange(lens_t[b] - tail, lens_t[b])])
                     for b in range(w.batch)]
        o_ref, lse_ref = oracle.sparse_attention(x.q[:, :, :T], x.k, x.v, lens_t, ref_lists)
        assert_out_close(out, o_ref, f"{name} block {block} tail {tail} out")
        assert_lse_close(lse, lse_ref, f"{name} block {block} tail {tail} lse")


@pytest.mark.parametrize("L", [1, 17, 1000, 4100, 32768, 40001])
def test_select_block_ids_match_block_positions(L):
    """The block ids are the blocks of the position form's selection (same
    scores, same sums), and the oracle's selection ranking the GPU's own
    block sums, expanded, gives the same positions."""
    rng = np.random.default_rng(900 + L)
    ctx = (L + 15) // 16 * 16
    lens = [L, max(1, L // 3), max(1, L - 5)]
    sc_h = (rng.standard_normal((3, ctx)) * 10).astype(np.float32)
    sc_h[2, ::9] = sc_h[2, 0]  # ties in block sums
    sc = torch.from_numpy(sc_h).cuda()
    for block, kb, ns, win in [(16, 32, 4, 64), (16, 8, 0, 0), (5, 20, 3, 7), (64, 3, 1, 1),
                               (16, 8192, 4, 256)]:
        if -(-ctx // block) > 8704:
            continue
        say(f"[select block ids] L={L} block={block} kb={kb}")
        nbs = -(-ctx // block)
        sums = torch.full((3, nbs), float("nan"), dtype=torch.float32, device="cuda")
        ids, n_ids = Bn.select_block_ids(sc, dev_i32(lens), kb, block, ns, win, ids_stride=kb + 1,
                                         block_sums=sums)
        pos, n_pos = Bn.select_blocks(sc, dev_i32(lens), kb, block, ns, win)
        torch.cuda.synchronize()
        ids_h, n_h, pos_h, np_h = ids.cpu().numpy(), n_ids.cpu().numpy(), pos.cpu().numpy(), n_pos.cpu().numpy()
        sums_h = sums.cpu().numpy()
        for b, Lb in enumerate(lens):
            got = ids_h[b, :n_h[b]]
            assert np.all(np.diff(got) > 0), (L, b, block)
            assert np.array_equal(oracle.block_positions(got, block, Lb), pos_h[b, :np_h[b]]), (L, b, block)
            nb = -(-Lb // block)
            want = oracle.select_blocks(sc_h[b], Lb, kb, block, ns, win,
                                        sums=sums_h[b, :nb].astype(np.float64))
            assert np.array_equal(oracle.block_positions(got, block, Lb), want), (L, b, block)


@pytest.mark.parametrize("name", ["paged_g8t6_d64", "g8t5_d128"])
def test_block_pipeline_on_verify_scores(name):
    """verify -> scores -> block ids -> gather over the blocks, against the
    oracle's attention over the positions of the kept blocks."""
    w = CASES[name]
    say(f"[block-id pipeline] {name}")
    x = W.make_layer(w)
    d = to_device(x)
    _, _, lg = Bn.verify_attention(d.q, d.k, d.v, d.seq_lens, block_table=d.block_table,
                                   max_ctx=d.max_ctx, collect_rows=w.collect_rows,
                                   layout="kvgroup_sum")
    sc = Bn.aggregate_scores(lg, d.seq_lens, w.num_q_heads, w.num_kv_heads)
    kb = max(3, w.budget // 16)
    ids, n_ids = Bn.select_block_ids(sc, d.seq_lens, kb, 16, w.n_sink, w.window)
    out, lse = Bn.sparse_attention_blocks(d.q, d.k, d.v, d.seq_lens, ids, n_ids, 16,
                                          block_table=d.block_table, max_ctx=d.max_ctx)
    torch.cuda.synchronize()
    ids_h, n_h = ids.cpu().numpy(), n_ids.cpu().numpy()
    lists = [oracle.block_positions(ids_h[b, :n_h[b]], 16, int(x.seq_lens[b])) for b in range(w.batch)]
    o_ref, lse_ref = oracle.sparse_attention(x.q, x.k, x.v, x.seq_lens, lists)
    assert_out_close(out, o_ref, f"{name} block-id pipeline out")
    assert_lse_close(lse, lse_ref, f"{name} block-id pipeline lse")
