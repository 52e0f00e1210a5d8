"""Seeded input generator: determinism, slice regeneration, recipe invariants."""
import numpy as np
import torch

from sparse_attention_long_amd import workloads as W


def test_bf16_rounding_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37.0
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]  # exact ties and a representable value
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_same_seed_same_bytes_and_slices_regenerate():
    w = W.small(batch=2, ctx=97, planted=3)
    a, b = W.make_layer(w), W.make_layer(w)
    for name in ("q", "k", "v"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    k1, v1 = W.kv_slice(w, 0, 1, 1, int(a.seq_lens[1]))
    assert np.array_equal(k1, a.k[1, 1]) and np.array_equal(v1, a.v[1, 1])
    assert np.array_equal(W.q_group(w, 0, 1, 1), a.q[1, w.group:2 * w.group])
    c = W.make_layer(W.small(batch=2, ctx=97, planted=3, seed=8))
    assert not np.array_equal(a.k, c.k)


def test_planted_keys_point_along_group_query():
    w = W.small(batch=1, ctx=200, planted=5, head_dim=64)
    x = W.make_layer(w)
    pos = x.planted[0]
    assert len(pos) == 5 and np.all(pos >= w.n_sink) and np.all(pos < 200 - w.window)
    for g in range(w.num_kv_heads):
        qg = W.bf16_bits_to_f32(x.q[0, g * w.group:(g + 1) * w.group]).astype(np.float64)
        u = qg.reshape(-1, w.head_dim).sum(0)
        u /= np.linalg.norm(u)
        kp = W.bf16_bits_to_f32(x.k[0, g, pos]).astype(np.float64)
        cos = (kp @ u) / np.linalg.norm(kp, axis=1)
        assert np.all(cos > 0.999)
        norm_ratio = np.linalg.norm(kp, axis=1).mean() / np.sqrt(w.head_dim)
        assert 3.0 < norm_ratio < 5.0


def test_workload_table_sizes():
    c = W.WORKLOADS
    w = c["ctx32k_b16_h64kv8_d128"]
    assert (w.batch, w.group, w.q_len, w.budget, w.collect_rows) == (16, 8, 5, 512, (0, 4))
    assert w.planted_count(32768) == 328
    w4 = c["ctx128k_b8_h32kv8_d128_draft6"]
    assert w4.planted_count(131072) == 655 and w4.max_ctx() == 131088 and w4.budget == 6554
    w5 = c["ragged8k-64k_b4_h64kv8_d64_paged16_l24"]
    lens = W.seq_lens(w5)
    assert np.all(lens >= 8192) and np.all(lens <= 65536) and w5.max_ctx() % 16 == 0


def test_paged_pool_holds_logical_rows():
    w = W.small(batch=3, ctx=None, ctx_range=(40, 90), paged=True, head_dim=64)
    x = W.make_layer(w)
    tab = x.block_table
    used = np.concatenate([tab[b, :-(-int(L) // 16)] for b, L in enumerate(x.seq_lens)])
    assert sorted(used.tolist()) == list(range(x.k_pool.shape[0]))  # a permutation
    for b, L in enumerate(x.seq_lens):
        for j in range(int(L)):
            blk, off = tab[b, j // 16], j % 16
            assert np.array_equal(x.k_pool[blk, :, off], x.k[b, :, j])
            assert np.array_equal(x.v_pool[blk, :, off], x.v[b, :, j])


def test_draft_scores_recipe():
    """Seeded N(0, 1) per position below the length, planted positions raised
    by 8, zero past the length; regenerates bit-identically."""
    w = W.small("ds", batch=3, lens=(300, 41, 1000), budget=64, n_sink=4, window=16,
                planted=5, seed=9)
    a, b = W.draft_scores(w), W.draft_scores(w)
    assert a.dtype == np.float32 and a.shape == (3, w.max_ctx())
    assert np.array_equal(a, b)
    for i, L in enumerate(W.seq_lens(w)):
        assert np.all(a[i, L:] == 0)
        pos = W.planted_positions(w, 0, i, int(L))
        others = np.setdiff1d(np.arange(L), pos)
        assert np.all(a[i, pos] > a[i, others].max() - 8 + 2) or pos.size == 0
        assert abs(a[i, others].mean()) < 0.3 and 0.7 < a[i, others].std() < 1.3
    assert w.draft_m == (64 - 4 - 16) // 2
