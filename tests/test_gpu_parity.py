"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Sizes here run the oracle in seconds but span several 32-position tiles,
several splits, ragged tails, every MFMA row-block count (1-4 blocks of 16
query rows), both head dims, contiguous and paged caches.  Full-size
workloads are in test_gpu_fullsize.py.
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


def _ragged_lens(n, seed):
    """n lengths: one in eight long (900-1299), the rest short (2-199).  With
    5 splits of 256 positions the balanced item length drops to 64, so each
    long sequence has about 20 items and its items past the 5th are handed to
    the short sequences' free workgroups."""
    rng = np.random.default_rng(seed)
    n_long = max(1, n // 8)
    lens = np.concatenate([rng.integers(900, 1300, size=n_long), rng.integers(2, 200, size=n - n_long)])
    rng.shuffle(lens)
    return tuple(int(x) for x in lens)


CASES = {
    # name: workload (G*T query rows -> MFMA row blocks)
    # capacities 301 and 257 (cap_align=1): logit and score rows not 16-byte aligned
    "g4t4_d128_ragged": W.small("g4t4", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                gamma=3, lens=(301, 4, 128), budget=40, n_sink=4, window=8,
                                cap_align=1),
    "g4t5_d64": W.small("g4t5", batch=2, num_q_heads=16, num_kv_heads=4, head_dim=64, gamma=4,
                        lens=(33, 257), budget=24, n_sink=2, window=6, seed=11, cap_align=1),
    "g8t5_d128": W.small("g8t5", batch=2, num_q_heads=16, num_kv_heads=2, head_dim=128, gamma=4,
                         lens=(700, 129), budget=64, n_sink=4, window=16, seed=12),
    "g8t8_d64": W.small("g8t8", batch=1, num_q_heads=32, num_kv_heads=4, head_dim=64, gamma=7,
                        lens=(513,), budget=100, n_sink=4, window=32, seed=13),
    # 21 rows: the one-split sparse pass shares them unevenly (11 + 10) between
    # two workgroups; 4 (sequence, kv-head) pairs leave padding workgroups
    "g3t7_d64": W.small("g3t7", batch=2, num_q_heads=6, num_kv_heads=2, head_dim=64, gamma=6,
                        lens=(520, 90), budget=44, n_sink=3, window=10, seed=18, cap_align=1),
    "g1t2_d128": W.small("g1t2", batch=2, num_q_heads=4, num_kv_heads=4, head_dim=128, gamma=1,
                         lens=(1000, 2), budget=50, n_sink=1, window=3, seed=14),
    "paged_g8t6_d64": W.small("pg", batch=3, num_q_heads=16, num_kv_heads=2, head_dim=64, gamma=5,
                              ctx=None, ctx_range=(40, 300), paged=True, budget=48, n_sink=4,
                              window=12, seed=15),
    "ctx2k_b1_h32kv8_d128": W.WORKLOADS["ctx2k_b1_h32kv8_d128"],
    # 8 x 8 workgroup rows -> 4224-position chunks: ragged last chunks and
    # chunks shorter than the LDS logit buffer (contiguous launches hold 8192
    # positions, so nothing flushes mid-chunk here; the paged twin does)
    "chunk4224_g1t3_d64": W.small("c4224", batch=8, num_q_heads=8, num_kv_heads=8, head_dim=64,
                                  gamma=2, lens=(33000, 20000, 4500, 8300, 12289, 30000, 4097, 16500),
                                  budget=300, n_sink=4, window=32, seed=16),
    # paged twin with equal lengths: 8 x 8 workgroup rows, items of 4224
    # positions, so the paged launch's 4096-position logit buffer fills
    # mid-chunk (contiguous launches hold 8192)
    "chunk4224_paged_g1t3_d64": W.small("c4224p", batch=8, num_q_heads=8, num_kv_heads=8,
                                        head_dim=64, gamma=2, ctx=33000, paged=True, budget=300,
                                        n_sink=4, window=32, seed=17),
    # balanced items over many sequences: 64 sequences (the lengths held one
    # per lane) and 72 (over 64: the lengths read in a loop), items of long
    # sequences handed to other sequences' workgroups
    "b64_balance_g2t2_d64": W.small("b64", batch=64, num_q_heads=4, num_kv_heads=2, head_dim=64,
                                    gamma=1, lens=_ragged_lens(64, 21), budget=40, n_sink=2,
                                    window=8, seed=21),
    "b72_balance_paged_g2t2_d128": W.small("b72", batch=72, num_q_heads=4, num_kv_heads=2,
                                           head_dim=128, gamma=1, lens=_ragged_lens(72, 22),
                                           paged=True, budget=40, n_sink=2, window=8, seed=22),
}


def run_verify(d, w, layout):
    return Bn.verify_attention(d.q, d.k, d.v, d.seq_lens, block_table=d.block_table,
                               max_ctx=d.max_ctx, collect_rows=w.collect_rows, layout=layout)


@pytest.mark.parametrize("name", list(CASES))
def test_verify_logits_scores_select_sparse(name):
    _check_pipeline(name, CASES[name])


def _random_workload(seed: int):
    """A seeded random small shape: batch 1-4, 1/2/4 kv-heads, 1-8 q-heads per
    kv-head, T = 2..8 rows (G*T <= 64), d = 64 or 128, contiguous or paged,
    ragged lengths 1..1600, budget, sinks and window drawn too."""
    rng = np.random.default_rng([2026, seed])
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 6, 8], p=[0.1, 0.1, 0.15, 0.2, 0.2, 0.25]))
    t = int(rng.integers(2, min(8, 64 // g) + 1))
    b = int(rng.integers(1, 5))
    lens = tuple(int(v) for v in rng.integers(1, 1601, size=b))
    k = int(rng.integers(8, 200))
    n_sink = int(rng.integers(0, 5))
    window = int(rng.integers(0, min(32, k - n_sink) + 1))  # the call needs n_sink + window <= k
    return W.small(f"rnd{seed}", batch=b, num_q_heads=g * hkv, num_kv_heads=hkv,
                   head_dim=int(rng.choice([64, 128])), gamma=t - 1, lens=lens,
                   budget=k, n_sink=n_sink, window=window, paged=bool(rng.integers(0, 2)),
                   cap_align=int(rng.choice([1, 16])), seed=1000 + seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(seed):
    """The whole path on seeded random small shapes (the same checks as the
    named cases)."""
    w = _random_workload(seed)
    say(f"[random shape] seed={seed} B={w.batch} Hq/Hkv={w.num_q_heads}/{w.num_kv_heads} "
        f"T={w.q_len} d={w.head_dim} paged={w.paged} lens={w.lens} k={w.budget}")
    # (planted keys are not checked: whether they win is a property of the
    # named workloads' data, not of the selection, which is compared exactly)
    _check_pipeline(f"rnd{seed}", w, planted=False)


@pytest.mark.parametrize("seed", range(12))
def test_random_long_lists(seed):
    """Seeded random long lists (1025-5000 entries: several splits merged in
    the launch), with T' = 1 or all T rows, a tail of 0-6 trailing positions
    after the list, contiguous or paged, d = 64 or 128."""
    rng = np.random.default_rng([2027, seed])
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8]))
    t = int(rng.integers(2, min(8, 64 // g) + 1))
    b = int(rng.integers(1, 4))
    lens = tuple(int(v) for v in rng.integers(1300, 6001, size=b))
    w = W.small(f"rl{seed}", batch=b, num_q_heads=g * hkv, num_kv_heads=hkv,
                head_dim=int(rng.choice([64, 128])), gamma=t - 1, lens=lens, budget=64, n_sink=4,
                window=16, paged=bool(rng.integers(0, 2)), seed=3000 + seed)
    tail = int(rng.integers(0, 7))
    one_row = bool(rng.integers(0, 2))
    count = int(rng.integers(1025, min(5000, min(lens) - tail) + 1))
    say(f"[random long lists] seed={seed} B={b} Hq/Hkv={w.num_q_heads}/{hkv} T={t} d={w.head_dim} "
        f"paged={w.paged} count={count} tail={tail} one_row={one_row}")
    x = W.make_layer(w)
    d = to_device(x)
    below = np.array([int(L) - tail for L in x.seq_lens], np.int32)  # listed positions stay below L - tail
    idx, n = W.index_lists(w.seed + 1, below, count=count, stride=count)
    qd = d.q[:, :, -1:].contiguous() if one_row else d.q
    qh = x.q[:, :, -1:] if one_row else x.q
    out, lse = Bn.sparse_attention(qd, d.k, d.v, d.seq_lens, dev_i32(idx), dev_i32(n),
                                   block_table=d.block_table, max_ctx=d.max_ctx, tail=tail)
    torch.cuda.synchronize()
    lists = [np.concatenate([idx[i, :n[i]], np.arange(int(x.seq_lens[i]) - tail, int(x.seq_lens[i]))])
             for i in range(b)]
    o_ref, lse_ref = oracle.sparse_attention(qh, x.k, x.v, x.seq_lens, lists)
    assert_out_close(out, o_ref, f"random long lists seed {seed} out")
    assert_lse_close(lse, lse_ref, f"random long lists seed {seed} lse")


def _check_pipeline(name, w, planted=True):
    say(f"[verify pipeline] {name}")
    x = W.make_layer(w)
    d = to_device(x)
    o_ref, lse_ref = oracle.verify_attention(x.q, x.k, x.v, x.seq_lens)
    l_ref = oracle.collected_logits(x.q, x.k, x.seq_lens, w.collect_rows)
    absl = np.where(np.isneginf(l_ref), 0.0, np.abs(l_ref))
    for layout in ("per_head", "kvgroup_sum"):
        out, lse, logits = run_verify(d, w, layout)
        torch.cuda.synchronize()
        assert_out_close(out, o_ref, f"{name}/{layout} out")
        assert_lse_close(lse, lse_ref, f"{name}/{layout} lse")
        lg = logits.cpu().numpy()
        if layout == "per_head":
            assert_logits_close(lg, l_ref, f"{name} per-head logits")
            s_floor = oracle.aggregate_scores(absl)
        else:
            assert_logits_close(lg, oracle.kvgroup_sum(l_ref, w.num_kv_heads), f"{name} group logits",
                                floor=oracle.kvgroup_sum(absl, w.num_kv_heads))
            s_floor = oracle.aggregate_scores(absl)
        scores = Bn.aggregate_scores(logits, d.seq_lens, w.num_q_heads, w.num_kv_heads, layout=layout)
        torch.cuda.synchronize()
        s_ref = oracle.aggregate_scores(l_ref)
        assert_logits_close(scores.cpu().numpy(), s_ref, f"{name}/{layout} scores", floor=s_floor)

        # selection: bit-exact against the oracle run on the GPU's own scores
        sc = scores.cpu().numpy()
        idx, n_idx = Bn.select_topk(scores, d.seq_lens, w.budget, w.n_sink, w.window,
                                    idx_stride=w.budget + 3)
        torch.cuda.synchronize()
        idx_h, n_h = idx.cpu().numpy(), n_idx.cpu().numpy()
        want = oracle.select_topk_batch(sc, x.seq_lens, w.budget, w.n_sink, w.window)
        for b in range(w.batch):
            assert n_h[b] == len(want[b])
            assert np.array_equal(idx_h[b, :n_h[b]], want[b]), f"{name}/{layout} idx b={b}"
        for b, pos in enumerate(x.planted if planted else []):
            if w.budget < int(x.seq_lens[b]):
                assert set(pos.tolist()) <= set(want[b].tolist()), f"planted key dropped b={b}"

    # sparse verify over the selected positions (same T rows)
    out_s, lse_s = Bn.sparse_attention(d.q, d.k, d.v, d.seq_lens, idx, n_idx,
                                       block_table=d.block_table, max_ctx=d.max_ctx)
    torch.cuda.synchronize()
    so_ref, slse_ref = oracle.sparse_attention(x.q, x.k, x.v, x.seq_lens, want)
    assert_out_close(out_s, so_ref, f"{name} sparse out")
    assert_lse_close(lse_s, slse_ref, f"{name} sparse lse")


@pytest.mark.parametrize("name", ["g4t5_d64", "ctx2k_b1_h32kv8_d128", "paged_g8t6_d64"])
def test_sparse_random_lists_and_draft_step(name):
    """Index lists from the seeded generator; T' = 1 draft query at the newest position."""
    w = CASES[name]
    say(f"[sparse lists] {name}")
    x = W.make_layer(w)
    d = to_device(x)
    lens = x.seq_lens
    idx, n = W.index_lists(w.seed, lens, count=max(1, w.budget // 2), stride=w.budget)
    out, lse = Bn.sparse_attention(d.q, d.k, d.v, d.seq_lens, dev_i32(idx), dev_i32(n),
                                   block_table=d.block_table, max_ctx=d.max_ctx)
    torch.cuda.synchronize()
    lists = [idx[b, :n[b]] for b in range(w.batch)]
    o_ref, lse_ref = oracle.sparse_attention(x.q, x.k, x.v, lens, lists)
    assert_out_close(out, o_ref, f"{name} sparse lists")
    assert_lse_close(lse, lse_ref, f"{name} sparse lists lse")
    # one query row (a draft step): q = last verify row
    q1 = d.q[:, :, -1:, :].contiguous()
    out1, lse1 = Bn.sparse_attention(q1, d.k, d.v, d.seq_lens, dev_i32(idx), dev_i32(n),
                                     block_table=d.block_table, max_ctx=d.max_ctx)
    torch.cuda.synchronize()
    o1_ref, l1_ref = oracle.sparse_attention(x.q[:, :, -1:, :], x.k, x.v, lens, lists)
    assert_out_close(out1, o1_ref, f"{name} sparse T'=1")
    assert_lse_close(lse1, l1_ref, f"{name} sparse T'=1 lse")


def test_sparse_degenerate_lists():
    """Empty list, one listed position, and rows that see no listed position."""
    w = CASES["g4t4_d128_ragged"]
    x = W.make_layer(w)
    d = to_device(x)
    lens = [int(L) for L in x.seq_lens]
    T = w.q_len
    lists = [np.zeros(0, np.int64), np.array([lens[1] - 1]), np.array([5, lens[2] - 1])]
    stride = 4
    idx = np.zeros((3, stride), np.int32)
    n = np.array([len(li) for li in lists], np.int32)
    for b, li in enumerate(lists):
        idx[b, :len(li)] = li
    out, lse = Bn.sparse_attention(d.q, d.k, d.v, d.seq_lens, dev_i32(idx), dev_i32(n))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_attention(x.q, x.k, x.v, lens, lists)
    assert_out_close(out, o_ref, "degenerate sparse")
    assert_lse_close(lse, lse_ref, "degenerate sparse lse")
    lh = lse.cpu().numpy()
    assert np.all(np.isneginf(lh[0])) and np.all(out[0].float().cpu().numpy() == 0)
    assert np.all(np.isneginf(lh[1, :, :T - 1]))  # rows before the last cannot see L-1


def test_verify_no_logits_and_explicit_scale():
    w = CASES["g8t5_d128"]
    x = W.make_layer(w)
    d = to_device(x)
    out, lse, logits = Bn.verify_attention(d.q, d.k, d.v, d.seq_lens, layout="none", scale=0.05)
    torch.cuda.synchronize()
    assert logits is None
    o_ref, lse_ref = oracle.verify_attention(x.q, x.k, x.v, x.seq_lens, scale=0.05)
    assert_out_close(out, o_ref, "scale=0.05")
    assert_lse_close(lse, lse_ref, "scale=0.05 lse")


# ------------------------------------------------------------------ selection stress
def _select_case(scores_h, lens, k, n_sink, window, stride=None):
    scores = torch.from_numpy(np.ascontiguousarray(scores_h, dtype=np.float32)).cuda()
    idx, n = Bn.select_topk(scores, dev_i32(lens), k, n_sink, window, idx_stride=stride or k)
    torch.cuda.synchronize()
    idx_h, n_h = idx.cpu().numpy(), n.cpu().numpy()
    for b, L in enumerate(lens):
        want = oracle.select_topk(scores_h[b], int(L), k, n_sink, window)
        assert n_h[b] == len(want), (b, L, k, n_h[b], len(want))
        assert np.array_equal(idx_h[b, :n_h[b]], want), (b, L, k, n_sink, window)


@pytest.mark.parametrize("L", [1, 2, 7, 64, 100, 1000, 4095, 4096, 4097, 32768, 40000, 131072])
def test_select_random_scores(L):
    rng = np.random.default_rng(L)
    lens = [L, max(1, L // 3), max(1, L - 1)]
    ctx = L + 5
    sc = rng.standard_normal((3, ctx)).astype(np.float32) * 10
    for k, ns, win in [(1, 0, 0), (16, 4, 8), (512, 4, 64), (6554, 4, 256), (L, 0, 0)]:
        if k < 1 or ns + win > k:
            continue
        _select_case(sc, lens, k, ns, win)


@pytest.mark.parametrize("L", [5, 64, 1000, 4096, 20001, 32768, 32769, 65536, 100001, 131072, 270000])
def test_select_random_scores_aligned_rows(L):
    """Rows whose length is a multiple of 4 (16-byte aligned): one round of
    32768 positions with keys in registers, up to 8 reloaded rounds, and the
    general kernel beyond 262144 positions.  (Rows in
    test_select_random_scores are not a multiple of 4: 4-byte loads.)"""
    rng = np.random.default_rng(100 + L)
    ctx = (L + 3) // 4 * 4
    lens = [L, max(1, L // 3), max(1, L - 1), max(1, L // 2 + 1)]
    sc = rng.standard_normal((len(lens), ctx)).astype(np.float32) * 10
    sc[3, ::7] = sc[3, 0]  # a repeated value across the row
    for k, ns, win in [(1, 0, 0), (16, 4, 8), (512, 4, 64), (2048, 4, 128), (6554, 4, 256), (L, 0, 0)]:
        if k < 1 or ns + win > k:
            continue
        _select_case(sc, lens, k, ns, win)


def test_select_ties_zeros_and_infinities():
    rng = np.random.default_rng(5)
    ctx = 5000
    sc = rng.integers(-3, 4, size=(4, ctx)).astype(np.float32)     # heavy ties
    sc[1] = np.where(rng.random(ctx) < 0.5, 0.0, -0.0).astype(np.float32)  # only +-0
    sc[2, ::3] = -np.inf
    sc[3] = 1.0                                                    # all equal
    lens = [5000, 4000, 4999, 3000]
    for k, ns, win in [(7, 0, 0), (100, 4, 16), (1000, 10, 990), (1000, 0, 1000), (2500, 3, 5)]:
        _select_case(sc, lens, k, ns, win, stride=k + 7)
    # a long all-equal row (every radix pass keeps the whole bin) and a two-valued one
    sc3 = np.ones((2, 70000), np.float32)
    sc3[1, ::2] = 2.0
    for k, ns, win in [(3000, 4, 64), (40000, 0, 100)]:
        _select_case(sc3, [70000, 69999], k, ns, win)
    # -inf must rank below every finite score
    sc2 = np.full((1, 64), -np.inf, np.float32)
    sc2[0, 10] = -1e30
    _select_case(sc2, [64], 1, 0, 0)


@pytest.mark.parametrize("L,n_bin,k", [
    (32768, 200, 200),     # one round, bin of 200: ranked directly
    (32768, 500, 512),     # one round, bin above the direct-ranking cap: another radix pass
    (32768, 3000, 512),    # one round, bin of 3000: two more passes
    (100000, 600, 500),    # reloaded rounds, bin of 600: ranked directly
    (100000, 1000, 500),   # reloaded rounds, bin above that cap: another radix pass
])
def test_select_threshold_bin_sizes(L, n_bin, k):
    """The bin holding the threshold key has a chosen size: n_bin scores in
    [2.0, 2.2) share their top 12 key bits, 10 scores lie above them and the
    rest below, so the bin is ranked directly or refined by further radix
    passes depending on its size and on the row length."""
    rng = np.random.default_rng(L + n_bin)
    n_sink, window = 4, 64
    sc = rng.uniform(0.0, 0.5, size=(2, L)).astype(np.float32)
    for b in range(2):
        pos = rng.choice(np.arange(n_sink, L - window), size=n_bin + 10, replace=False)
        sc[b, pos[:n_bin]] = (2.0 + 0.2 * rng.random(n_bin)).astype(np.float32)
        sc[b, pos[n_bin:]] = (5.0 + rng.random(10)).astype(np.float32)
    assert (k - n_sink - window) - 10 < n_bin  # the threshold key lies in the bin
    _select_case(sc, [L, L - 1], k, n_sink, window)


@pytest.mark.parametrize("ctx", [65536, 65541])
def test_select_per_round_edge_rows(ctx):
    """Capacities above 1.5 rounds take the per-round selection (workspace):
    in one launch, an empty row, rows no longer than the budget, a row whose
    sinks and window fill the budget, rows of one and of two rounds; with
    aligned (16-byte loads) and unaligned capacities."""
    rng = np.random.default_rng(ctx)
    k, ns, win = 300, 4, 64
    lens = [0, 100, 300, 65536 if ctx >= 65536 else ctx, 32768, 40000, 50001, 65000]
    sc = (rng.standard_normal((len(lens), ctx)) * 10).astype(np.float32)
    sc[6, ::5] = 3.0  # a repeated value
    assert Bn.select_workspace_bytes(len(lens), ctx) > 0
    _select_case(sc, lens, k, ns, win, stride=k + 5)
    _select_case(sc, lens, ns + win, ns, win)  # r = 0: the forced positions only


# ------------------------------------------------------------------ hybrid selection
def _hybrid_case(tgt_h, drf_h, lens, k, m, n_sink, window, stride=None):
    tgt = torch.from_numpy(np.ascontiguousarray(tgt_h, dtype=np.float32)).cuda()
    drf = torch.from_numpy(np.ascontiguousarray(drf_h, dtype=np.float32)).cuda()
    idx, n = Bn.select_topk_hybrid(tgt, drf, dev_i32(lens), k, m, n_sink, window,
                                   idx_stride=stride or k)
    torch.cuda.synchronize()
    idx_h, n_h = idx.cpu().numpy(), n.cpu().numpy()
    for b, L in enumerate(lens):
        want = oracle.select_topk_hybrid(tgt_h[b], drf_h[b], int(L), k, m, n_sink, window)
        assert n_h[b] == len(want), (b, L, k, m, n_h[b], len(want))
        assert np.array_equal(idx_h[b, :n_h[b]], want), (b, L, k, m, n_sink, window)


@pytest.mark.parametrize("L", [1, 7, 1000, 4097, 32768, 40001, 131072, 262143])
def test_hybrid_select_random(L):
    """Both stages against the oracle: one round of keys in registers and
    reloaded rounds, aligned and unaligned rows, m from 0 past the free budget."""
    say(f"[hybrid select] L={L}")
    rng = np.random.default_rng(300 + L)
    for ctx in ((L + 3) // 4 * 4, L + 1):
        lens = [L, max(1, L // 3), max(1, L - 1)]
        tgt = rng.standard_normal((3, ctx)).astype(np.float32) * 10
        drf = rng.standard_normal((3, ctx)).astype(np.float32)
        for k, ns, win in [(1, 0, 0), (16, 4, 8), (512, 4, 64), (6554, 4, 256)]:
            if ns + win > k:
                continue
            r = k - ns - win
            for m in sorted({0, 1, r // 2, r, r + 5}):
                _hybrid_case(tgt, drf, lens, k, m, ns, win)


def test_hybrid_select_ties_and_overlap():
    """Tie-heavy and all-equal draft and target rows (every radix pass keeps
    the whole bin: the lowest positions win in each stage), the target's best
    positions taken by the draft stage first, and one signal for both stages."""
    rng = np.random.default_rng(17)
    ctx = 70000
    tgt = rng.integers(-3, 4, size=(4, ctx)).astype(np.float32)
    drf = rng.integers(-2, 3, size=(4, ctx)).astype(np.float32)
    drf[1] = 1.0                       # all equal: the draft stage takes the lowest free positions
    tgt[2] = 5.0
    drf[2] = tgt[2]                    # all equal in both
    drf[3] = tgt[3]                    # one signal for both stages
    lens = [70000, 69999, 50000, 65000]
    for k, m, ns, win in [(3000, 1500, 4, 64), (3000, 2932, 4, 64), (40000, 20000, 0, 100),
                          (100, 37, 10, 5)]:
        _hybrid_case(tgt, drf, lens, k, m, ns, win, stride=k + 3)
    # the draft signal favours exactly the target's top positions: the target
    # stage must skip them and take the next ones
    t2 = rng.standard_normal((1, 5000)).astype(np.float32)
    d2 = t2.copy()
    _hybrid_case(t2, d2, [5000], 300, 100, 4, 16)
    d3 = -t2
    _hybrid_case(t2, d3, [5000], 300, 100, 4, 16)


@pytest.mark.parametrize("name", ["g4t4_d128_ragged", "paged_g8t6_d64", "ctx2k_b1_h32kv8_d128"])
def test_hybrid_select_on_verify_scores(name):
    """The target signal as the verify pass writes it (the GPU's scores), the
    draft signal from the seeded generator; then sparse attention over the
    hybrid selection."""
    w = CASES[name]
    say(f"[hybrid pipeline] {name}")
    x = W.make_layer(w)
    d = to_device(x)
    _, _, lg = run_verify(d, w, "kvgroup_sum")
    sc = Bn.aggregate_scores(lg, d.seq_lens, w.num_q_heads, w.num_kv_heads)
    drf_h = W.draft_scores(w)
    drf = torch.from_numpy(drf_h).cuda()
    idx, n = Bn.select_topk_hybrid(sc, drf, d.seq_lens, w.budget, w.draft_m, w.n_sink, w.window)
    torch.cuda.synchronize()
    sc_h = sc.cpu().numpy()
    want = oracle.select_topk_hybrid_batch(sc_h, drf_h, x.seq_lens, w.budget, w.draft_m, w.n_sink,
                                           w.window)
    idx_h, n_h = idx.cpu().numpy(), n.cpu().numpy()
    for b in range(w.batch):
        assert n_h[b] == len(want[b])
        assert np.array_equal(idx_h[b, :n_h[b]], want[b]), f"{name} b={b}"
    out, lse = Bn.sparse_attention(d.q, d.k, d.v, d.seq_lens, idx, n, block_table=d.block_table,
                                   max_ctx=d.max_ctx)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_attention(x.q, x.k, x.v, x.seq_lens, want)
    assert_out_close(out, o_ref, f"{name} hybrid sparse out")
    assert_lse_close(lse, lse_ref, f"{name} hybrid sparse lse")


# ------------------------------------------------------------------ block selection
def _blocks_case(scores_h, lens, kb, block, n_sink, window, stride=None):
    """Block selection on the GPU against the oracle: the GPU's fp32 block
    sums against the exact fp64 sums (the scores tolerance, 1e-3 * max(1,
    sum of |members|); -inf blocks exactly), and the kept positions bit-exact
    against the oracle's selection ranking the GPU's own block sums (the same
    values compared on both sides)."""
    scores_h = np.ascontiguousarray(scores_h, dtype=np.float32)
    scores = torch.from_numpy(scores_h).cuda()
    nbs = -(-scores_h.shape[1] // block)
    sums = torch.full((scores_h.shape[0], nbs), float("nan"), dtype=torch.float32, device="cuda")
    idx, n = Bn.select_blocks(scores, dev_i32(lens), kb, block, n_sink, window,
                              idx_stride=stride or kb * block, block_sums=sums)
    torch.cuda.synchronize()
    idx_h, n_h, sums_h = idx.cpu().numpy(), n.cpu().numpy(), sums.cpu().numpy()
    out = []
    for b, L in enumerate(lens):
        nb = -(-int(L) // block)
        ref = oracle.block_sums(scores_h[b], int(L), block)
        got = sums_h[b, :nb].astype(np.float64)
        inf = np.isinf(ref)
        assert np.array_equal(got[inf], ref[inf]), (b, L, block, "infinite block sums")
        mag = np.array([np.abs(scores_h[b, i * block:min(int(L), (i + 1) * block)].astype(np.float64)).sum()
                        for i in range(nb)])
        err = np.abs(got[~inf] - ref[~inf])
        tol = 1e-3 * np.maximum(1.0, mag[~inf])
        assert np.all(err <= tol), (b, L, block, float(err.max(initial=0.0)))
        assert np.all(np.isnan(sums_h[b, nb:])), (b, L, block, "sums written past the length")
        want = oracle.select_blocks(scores_h[b], int(L), kb, block, n_sink, window, sums=got)
        assert n_h[b] == len(want), (b, L, kb, block, n_h[b], len(want))
        assert np.array_equal(idx_h[b, :n_h[b]], want), (b, L, kb, block, n_sink, window)
        out.append(want)
    return idx, n, out


@pytest.mark.parametrize("L", [1, 15, 16, 17, 1000, 4100, 32768, 40001, 131072])
def test_select_blocks_random(L):
    """Whole-block selection against the oracle: block sizes 16, 8, 4 and 5
    (unaligned rows read 4 bytes at a time), partial last blocks, sinks and
    windows that end mid-block, a budget covering every block."""
    say(f"[select blocks] L={L}")
    rng = np.random.default_rng(500 + L)
    for ctx in ((L + 15) // 16 * 16, L + 3):
        lens = [L, max(1, L // 3), max(1, L - 5)]
        sc = rng.standard_normal((3, ctx)).astype(np.float32) * 10
        for block, kb, ns, win in [(16, 32, 4, 64), (16, 8, 0, 0), (8, 64, 4, 100), (4, 410, 10, 256),
                                   (5, 20, 3, 7), (16, 8192, 4, 256)]:
            if -(-ctx // block) > 8704:
                continue
            _blocks_case(sc, lens, kb, block, ns, win)


def test_select_blocks_ties_and_infinities():
    rng = np.random.default_rng(23)
    ctx = 6000
    sc = rng.integers(-2, 3, size=(4, ctx)).astype(np.float32)   # block-sum ties
    sc[1] = 0.0
    sc[1, ::2] = -0.0                                            # all sums +-0: lowest blocks win
    sc[2, ::37] = -np.inf                                        # -inf sinks whole blocks
    sc[3] = 1.0
    lens = [6000, 5999, 5001, 4096]
    for block, kb, ns, win in [(16, 40, 4, 64), (16, 200, 0, 0), (32, 10, 33, 31), (1, 300, 4, 16)]:
        _blocks_case(sc, lens, kb, block, ns, win)


@pytest.mark.parametrize("name", ["paged_g8t6_d64", "ctx2k_b1_h32kv8_d128", "g4t4_d128_ragged"])
def test_select_blocks_on_verify_scores_then_sparse(name):
    """Block selection on the verify pass's own scores, then sparse attention
    over the kept blocks' positions (contiguous runs; with a paged cache a
    16-position block is one page)."""
    w = CASES[name]
    say(f"[block pipeline] {name}")
    x = W.make_layer(w)
    d = to_device(x)
    _, _, lg = run_verify(d, w, "kvgroup_sum")
    sc = Bn.aggregate_scores(lg, d.seq_lens, w.num_q_heads, w.num_kv_heads)
    kb = max(3, w.budget // 16)
    torch.cuda.synchronize()
    idx, n, want = _blocks_case(sc.cpu().numpy(), list(x.seq_lens), kb, 16, w.n_sink, w.window)
    out, lse = Bn.sparse_attention(d.q, d.k, d.v, d.seq_lens, idx, n, block_table=d.block_table,
                                   max_ctx=d.max_ctx)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_attention(x.q, x.k, x.v, x.seq_lens, want)
    assert_out_close(out, o_ref, f"{name} block sparse out")
    assert_lse_close(lse, lse_ref, f"{name} block sparse lse")


@pytest.mark.parametrize("name", ["g8t5_d128", "ctx2k_b1_h32kv8_d128", "paged_g8t6_d64"])
def test_determinism(name):
    """Two runs give bitwise identical logits, scores, selected positions and
    sparse outputs: every position's logit sum is computed by the same
    arithmetic whichever wavefront takes its tile.  The verify output and lse
    agree to within fp32 accumulation order (the tiles a wavefront takes are
    claimed at run time, so its order of accumulation may differ): at most one
    bf16 unit of the output, 1e-5 in lse."""
    w = CASES[name]
    x = W.make_layer(w)
    d = to_device(x)
    runs = []
    for _ in range(2):
        out, lse, lg = run_verify(d, w, "kvgroup_sum")
        sc = Bn.aggregate_scores(lg, d.seq_lens, w.num_q_heads, w.num_kv_heads)
        idx, n = Bn.select_topk(sc, d.seq_lens, w.budget, w.n_sink, w.window)
        so, sl = Bn.sparse_attention(d.q, d.k, d.v, d.seq_lens, idx, n, block_table=d.block_table,
                                     max_ctx=d.max_ctx)
        torch.cuda.synchronize()
        L = x.seq_lens
        lgv = np.concatenate([lg[b, :, :L[b]].cpu().numpy().ravel() for b in range(w.batch)])
        scv = np.concatenate([sc[b, :L[b]].cpu().numpy() for b in range(w.batch)])
        runs.append(dict(out=out.float().cpu().numpy(), lse=lse.cpu().numpy(), lg=lgv, sc=scv,
                         idx=np.concatenate([idx[b, :n[b]].cpu().numpy() for b in range(w.batch)]),
                         so=so.view(torch.int16).cpu().numpy(), sl=sl.cpu().numpy()))
    a, b = runs
    for key in ("lg", "sc", "idx", "so", "sl"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key
    np.testing.assert_allclose(a["out"], b["out"], atol=8e-3, rtol=1e-2)
    np.testing.assert_allclose(a["lse"], b["lse"], atol=1e-5, rtol=0)


@pytest.mark.parametrize("name", ["g4t5_d64", "ctx2k_b1_h32kv8_d128", "paged_g8t6_d64"])
def test_two_phase_api_matches_one_call(name):
    """partials + combine gives the same bytes as the one-call entry points, for
    one split (the one-call path then writes the output directly) and several."""
    w = CASES[name]
    x = W.make_layer(w)
    d = to_device(x)
    desc = Bn.make_desc(d.q, d.k, d.block_table, d.max_ctx)
    B, Hq, T, D = d.q.shape
    for layout, code in (("kvgroup_sum", Bn.LOGITS_KVGROUP_SUM), ("per_head", Bn.LOGITS_PER_HEAD)):
        out1, lse1, lg1 = run_verify(d, w, layout)
        ws = torch.empty(Bn.verify_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        lg2 = torch.empty_like(lg1)
        Bn.verify_partials(desc, d.q, d.k, d.v, d.seq_lens, d.block_table, w.collect_rows, code, lg2, ws)
        out2 = torch.empty_like(out1)
        lse2 = torch.empty_like(lse1)
        Bn.combine_partials(desc, d.max_ctx, d.seq_lens, ws, out2, lse2)
        torch.cuda.synchronize()
        assert_out_close(out2, oracle.verify_attention(x.q, x.k, x.v, x.seq_lens)[0], f"{name} two-phase")
        # same softmax merge order within a split; the direct path divides once
        np.testing.assert_allclose(out2.float().cpu().numpy(), out1.float().cpu().numpy(), atol=8e-3)
        np.testing.assert_allclose(lse2.cpu().numpy(), lse1.cpu().numpy(), atol=1e-5)
        for b in range(w.batch):
            L = int(x.seq_lens[b])
            assert torch.equal(lg1[b, ..., :L], lg2[b, ..., :L])
    idx, n = W.index_lists(w.seed + 1, x.seq_lens, count=max(1, w.budget // 2), stride=w.budget)
    idx_d, n_d = dev_i32(idx), dev_i32(n)
    so1, sl1 = Bn.sparse_attention(d.q, d.k, d.v, d.seq_lens, idx_d, n_d, block_table=d.block_table,
                                   max_ctx=d.max_ctx)
    ws = torch.empty(Bn.sparse_workspace_bytes(desc, idx.shape[1]), dtype=torch.uint8, device="cuda")
    Bn.sparse_partials(desc, d.q, d.k, d.v, d.seq_lens, d.block_table, idx_d, n_d, ws)
    so2, sl2 = torch.empty_like(so1), torch.empty_like(sl1)
    Bn.combine_partials(desc, idx.shape[1], n_d, ws, so2, sl2)
    torch.cuda.synchronize()
    np.testing.assert_allclose(so2.float().cpu().numpy(), so1.float().cpu().numpy(), atol=8e-3)
    np.testing.assert_allclose(sl2.cpu().numpy(), sl1.cpu().numpy(), atol=1e-5)


@pytest.mark.parametrize("name", ["g4t5_d64", "ctx2k_b1_h32kv8_d128", "paged_g8t6_d64"])
def test_sparse_one_launch_merge_repeats_and_resets(name):
    """The one-call sparse path splits each list over several workgroups and
    the last one to finish merges them: repeated calls on one workspace give
    the oracle's result each time (empty, short and full lists mixed), the
    counters are zero after every call, and the result matches the two-phase
    partials + combine form."""
    w = CASES[name]
    say(f"[sparse one-launch merge] {name}")
    x = W.make_layer(w)
    d = to_device(x)
    desc = Bn.make_desc(d.q, d.k, d.block_table, d.max_ctx)
    stride = 3000  # longer than one split: the splits merge in the launch
    nbytes = Bn.sparse_workspace_bytes(desc, stride)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sync_bytes = -(-w.batch * w.num_kv_heads * 4 // 256) * 256
    for rep, count in enumerate([stride, 5, 0, 1500, stride]):
        idx, n = W.index_lists(w.seed + 40 + rep, x.seq_lens, count=count, stride=stride)
        if rep == 3:
            n[0] = 0  # one empty list among full ones
        out, lse = Bn.sparse_attention(d.q, d.k, d.v, d.seq_lens, dev_i32(idx), dev_i32(n),
                                       block_table=d.block_table, max_ctx=d.max_ctx, workspace=ws)
        torch.cuda.synchronize()
        lists = [idx[b, :n[b]] for b in range(w.batch)]
        o_ref, lse_ref = oracle.sparse_attention(x.q, x.k, x.v, x.seq_lens, lists)
        assert_out_close(out, o_ref, f"{name} rep {rep} out")
        assert_lse_close(lse, lse_ref, f"{name} rep {rep} lse")
        assert int(ws[:sync_bytes].count_nonzero()) == 0, "counters not reset"
    # the two-phase form on its own workspace agrees
    ws2 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    idx_d, n_d = dev_i32(idx), dev_i32(n)
    Bn.sparse_partials(desc, d.q, d.k, d.v, d.seq_lens, d.block_table, idx_d, n_d, ws2)
    o2, l2 = torch.empty_like(out), torch.empty_like(lse)
    Bn.combine_partials(desc, stride, n_d, ws2, o2, l2)
    torch.cuda.synchronize()
    # different split plans: the fp32 merge order differs, so a bf16 output
    # may round one unit apart
    np.testing.assert_allclose(o2.float().cpu().numpy(), out.float().cpu().numpy(), atol=8e-3,
                               rtol=1e-2)
    np.testing.assert_allclose(l2.cpu().numpy(), lse.cpu().numpy(), atol=1e-5)


@pytest.mark.parametrize("count", [45, 700, 1500])
def test_sparse_paged_ignores_blocks_it_does_not_own(count):
    """A paged pool whose blocks outside the sequences' tables hold NaN (as a
    pool of freed or never-written blocks may): every gathered row, the
    padding of a list's last partial tile included, comes from a block the
    sequence owns, so the outputs stay finite and match the oracle.  Block
    ids are shifted by one so that pool block 0 is one of the NaN blocks."""
    w = CASES["paged_g8t6_d64"]
    say(f"[sparse paged NaN pool] count={count}")
    x = W.make_layer(w)
    nan_blk = np.full((1,) + x.k_pool.shape[1:], 0x7FC0, dtype=np.uint16)  # bf16 quiet NaN
    kp = np.concatenate([nan_blk, x.k_pool, nan_blk, nan_blk])
    vp = np.concatenate([nan_blk, x.v_pool, nan_blk, nan_blk])
    tab = x.block_table.copy()
    for b, L in enumerate(x.seq_lens):
        tab[b, :-(-int(L) // 16)] += 1
    q = dev_bf16(x.q)
    k, v, bt, lens = dev_bf16(kp), dev_bf16(vp), dev_i32(tab), dev_i32(x.seq_lens)
    idx, n = W.index_lists(w.seed + 90 + count, x.seq_lens, count=count, stride=count)
    for qrows in (w.q_len, 1):
        out, lse = Bn.sparse_attention(q[:, :, :qrows].contiguous(), k, v, lens, dev_i32(idx),
                                       dev_i32(n), block_table=bt, max_ctx=w.max_ctx())
        torch.cuda.synchronize()
        lists = [idx[b, :n[b]] for b in range(w.batch)]
        o_ref, lse_ref = oracle.sparse_attention(x.q[:, :, :qrows], x.k, x.v, x.seq_lens, lists)
        assert_out_close(out, o_ref, f"NaN pool count {count} rows {qrows} out")
        assert_lse_close(lse, lse_ref, f"NaN pool count {count} rows {qrows} lse")
    if count == 45:  # the verify pass reads owned blocks only, too
        out, lse, lg = Bn.verify_attention(q, k, v, lens, block_table=bt, max_ctx=w.max_ctx(),
                                           collect_rows=w.collect_rows, layout="kvgroup_sum")
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.verify_attention(x.q, x.k, x.v, x.seq_lens)
        assert_out_close(out, o_ref, "NaN pool verify out")
        assert_lse_close(lse, lse_ref, "NaN pool verify lse")
        for b, L in enumerate(x.seq_lens):
            assert np.all(~np.isnan(lg[b, :, :int(L)].cpu().numpy())), "NaN pool verify logits"


def test_sparse_workspace_reused_across_split_plans():
    """One zero-filled workspace, sized for the longest span, serves draft
    steps whose split plans differ: with 4093 listed positions the tails 1..6
    plan different split counts (the span crosses a chunk boundary), then
    tail 1 again.  Each call matches the oracle and leaves the counters
    zero."""
    w = W.small("reuse", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, gamma=0,
                lens=(6000,), budget=64, n_sink=4, window=16, seed=47)
    x = W.make_layer(w)
    d = to_device(x)
    count = 4093
    desc = Bn.make_desc(d.q, d.k, None, d.max_ctx)
    plans = {Bn.split_plan(desc, count + t) for t in range(1, 7)}
    assert len(plans) > 1, plans  # the case exercises a change of plan
    ws = torch.zeros(Bn.sparse_workspace_bytes(desc, count + 6), dtype=torch.uint8, device="cuda")
    sync_bytes = -(-w.batch * w.num_kv_heads * 4 // 256) * 256
    for tail in (1, 2, 3, 4, 5, 6, 1):
        say(f"[sparse workspace reuse] tail={tail}")
        lens = np.array([int(x.seq_lens[0]) - 6], np.int32)
        idx, n = W.index_lists(w.seed + 3, lens, count=count, stride=count)
        lens_t = lens + np.int32(tail)
        out, lse = Bn.sparse_attention(d.q, d.k, d.v, dev_i32(lens_t), dev_i32(idx), dev_i32(n),
                                       max_ctx=d.max_ctx, tail=tail, workspace=ws)
        torch.cuda.synchronize()
        lists = [np.concatenate([idx[0, :n[0]], np.arange(lens_t[0] - tail, lens_t[0])])]
        o_ref, lse_ref = oracle.sparse_attention(x.q, x.k, x.v, lens_t, lists)
        assert_out_close(out, o_ref, f"reuse tail {tail} out")
        assert_lse_close(lse, lse_ref, f"reuse tail {tail} lse")
        assert int(ws[:sync_bytes].count_nonzero()) == 0, f"counters not reset after tail {tail}"


@pytest.mark.parametrize("name", ["g4t5_d64", "ctx2k_b1_h32kv8_d128", "paged_g8t6_d64"])
@pytest.mark.parametrize("count", [20, 900, 2000])
def test_sparse_trailing_positions(name, count):
    """Trailing positions (the tokens drafted since the selection) attended
    after the list without appending them: against the oracle on the
    explicit lists, and equal to the appended form; one split and several."""
    w = CASES[name]
    say(f"[sparse tail] {name} count={count}")
    x = W.make_layer(w)
    d = to_device(x)
    for tail in (1, 3, 7):
        lens = np.array([max(int(L) - tail, 1) for L in x.seq_lens], np.int32)  # kept below L - tail
        idx, n = W.index_lists(w.seed + 70 + tail, lens, count=count, stride=count)
        lens_t = lens + np.int32(tail)
        qd = d.q[:, :, :1].contiguous()
        out, lse = Bn.sparse_attention(qd, d.k, d.v, dev_i32(lens_t), dev_i32(idx), dev_i32(n),
                                       block_table=d.block_table, max_ctx=d.max_ctx, tail=tail)
        lists = [np.concatenate([idx[b, :n[b]], np.arange(max(0, lens_t[b] - tail), lens_t[b])])
                 for b in range(w.batch)]
        ia = np.zeros((w.batch, count + tail), np.int32)
        for b, li in enumerate(lists):
            ia[b, :len(li)] = li
        na = np.array([len(li) for li in lists], np.int32)
        out2, lse2 = Bn.sparse_attention(qd, d.k, d.v, dev_i32(lens_t), dev_i32(ia), dev_i32(na),
                                         block_table=d.block_table, max_ctx=d.max_ctx)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.sparse_attention(x.q[:, :, :1], x.k, x.v, lens_t, lists)
        assert_out_close(out, o_ref, f"{name} tail {tail} out")
        assert_lse_close(lse, lse_ref, f"{name} tail {tail} lse")
        np.testing.assert_allclose(out.float().cpu().numpy(), out2.float().cpu().numpy(),
                                   atol=8e-3, rtol=1e-2)


@pytest.mark.parametrize("count,stride", [(1000, 1000), (3000, 3000), (700, 1024)])
def test_sparse_long_lists_many_tiles_per_wavefront(count, stride):
    """Lists long enough that every wavefront walks several tiles (one split
    with 8 wavefronts up to 1024 entries; several splits beyond), including
    tiles past the preloaded ones."""
    w = W.small("longlist", batch=2, num_q_heads=16, num_kv_heads=2, head_dim=64, gamma=4,
                lens=(4000, 3500), budget=64, n_sink=4, window=16, seed=21)
    say(f"[sparse long lists] count={count} stride={stride}")
    x = W.make_layer(w)
    d = to_device(x)
    idx, n = W.index_lists(31 + count, x.seq_lens, count=count, stride=stride)
    out, lse = Bn.sparse_attention(d.q, d.k, d.v, d.seq_lens, dev_i32(idx), dev_i32(n))
    torch.cuda.synchronize()
    lists = [idx[b, :n[b]] for b in range(w.batch)]
    o_ref, lse_ref = oracle.sparse_attention(x.q, x.k, x.v, x.seq_lens, lists)
    assert_out_close(out, o_ref, f"long list {count}")
    assert_lse_close(lse, lse_ref, f"long list {count} lse")


@pytest.mark.parametrize("name", ["g8t5_d128", "ctx2k_b1_h32kv8_d128", "paged_g8t6_d64"])
def test_verify_finish_equals_combine_and_aggregate(name):
    """The fused combine + aggregate launch gives the same bytes as the two
    separate calls (same per-element code and summation order)."""
    w = CASES[name]
    x = W.make_layer(w)
    d = to_device(x)
    desc = Bn.make_desc(d.q, d.k, d.block_table, d.max_ctx)
    for layout, code in (("kvgroup_sum", Bn.LOGITS_KVGROUP_SUM), ("per_head", Bn.LOGITS_PER_HEAD)):
        ws = torch.empty(Bn.verify_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        shape = (w.batch, w.num_kv_heads, d.max_ctx) if code == Bn.LOGITS_KVGROUP_SUM else \
            (w.batch, 2, w.num_q_heads, d.max_ctx)
        lg = torch.empty(shape, dtype=torch.float32, device="cuda")
        Bn.verify_partials(desc, d.q, d.k, d.v, d.seq_lens, d.block_table, w.collect_rows, code, lg, ws)
        o1, l1 = torch.empty_like(d.q), torch.empty(d.q.shape[:3], dtype=torch.float32, device="cuda")
        Bn.combine_partials(desc, d.max_ctx, d.seq_lens, ws, o1, l1)
        s1 = Bn.aggregate_scores(lg, d.seq_lens, w.num_q_heads, w.num_kv_heads, layout=layout)
        o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
        s2 = torch.full_like(s1, 7.0)
        Bn.verify_finish(desc, d.seq_lens, ws, o2, l2, code, lg, s2)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)
        for b in range(w.batch):
            L = int(x.seq_lens[b])
            assert torch.equal(s1[b, :L], s2[b, :L])
            assert torch.all(s2[b, L:] == 7.0)  # positions past the length are untouched
        o3 = torch.empty_like(o1)
        Bn.verify_finish(desc, d.seq_lens, ws, o3, None)  # combine only
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def _row_set(kind, T):
    return {"all": tuple(range(T)), "first": (0,), "bonus": (T - 1,),
            "even": tuple(range(0, T, 2)), "mid": tuple(range(1, T - 1)) or (0,)}[kind]


@pytest.mark.parametrize("kind", ["all", "first", "bonus", "even", "mid"])
@pytest.mark.parametrize("name", ["g4t5_d64", "g8t8_d64", "paged_g8t6_d64", "chunk4224_g1t3_d64"])
def test_collect_any_row_set(name, kind):
    """Logits of any subset of the verify rows (all of them is the full score
    sum over every verify row): logits and scores against the oracle in both
    layouts, through the one-call and the partials + finish entry points; the
    attention output does not depend on which rows are collected."""
    w = CASES[name]
    T = w.gamma + 1
    rows = _row_set(kind, T)
    say(f"[collect rows] {name} rows={rows}")
    x = W.make_layer(w)
    d = to_device(x)
    o_ref, lse_ref = oracle.verify_attention(x.q, x.k, x.v, x.seq_lens)
    l_ref = oracle.collected_logits(x.q, x.k, x.seq_lens, rows)
    absl = np.where(np.isneginf(l_ref), 0.0, np.abs(l_ref))
    s_ref, s_floor = oracle.aggregate_scores(l_ref), oracle.aggregate_scores(absl)
    desc = Bn.make_desc(d.q, d.k, d.block_table, d.max_ctx)
    for layout, code in (("per_head", Bn.LOGITS_PER_HEAD), ("kvgroup_sum", Bn.LOGITS_KVGROUP_SUM)):
        out, lse, lg = Bn.verify_attention(d.q, d.k, d.v, d.seq_lens, block_table=d.block_table,
                                           max_ctx=d.max_ctx, collect_rows=rows, layout=layout)
        torch.cuda.synchronize()
        assert_out_close(out, o_ref, f"{name}/{layout}/{kind} out")
        assert_lse_close(lse, lse_ref, f"{name}/{layout}/{kind} lse")
        if layout == "per_head":
            assert lg.shape[1] == len(rows)
            assert_logits_close(lg.cpu().numpy(), l_ref, f"{name}/{kind} per-head logits")
        else:
            assert_logits_close(lg.cpu().numpy(), oracle.kvgroup_sum(l_ref, w.num_kv_heads),
                                f"{name}/{kind} group logits",
                                floor=oracle.kvgroup_sum(absl, w.num_kv_heads))
        sc = Bn.aggregate_scores(lg, d.seq_lens, w.num_q_heads, w.num_kv_heads, layout=layout)
        # two-phase: partials, then combine + aggregate in one launch
        ws = torch.empty(Bn.verify_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        lg2 = torch.empty_like(lg)
        Bn.verify_partials(desc, d.q, d.k, d.v, d.seq_lens, d.block_table, rows, code, lg2, ws)
        o2, l2 = torch.empty_like(out), torch.empty_like(lse)
        s2 = torch.empty_like(sc)
        Bn.verify_finish(desc, d.seq_lens, ws, o2, l2, code, lg2, s2)
        torch.cuda.synchronize()
        assert_logits_close(sc.cpu().numpy(), s_ref, f"{name}/{layout}/{kind} scores", floor=s_floor)
        for b in range(w.batch):
            L = int(x.seq_lens[b])
            assert torch.equal(lg[b, ..., :L], lg2[b, ..., :L])
            assert torch.equal(sc[b, :L], s2[b, :L])


def _head_set(kind, Hq, G):
    return {"one": (Hq - 1,), "first_group": tuple(range(G)),
            "scattered": tuple(range(1, Hq, 3)), "one_per_group": tuple(range(0, Hq, G))}[kind]


@pytest.mark.parametrize("kind", ["one", "first_group", "scattered", "one_per_group"])
@pytest.mark.parametrize("name", ["g4t5_d64", "g8t8_d64", "paged_g8t6_d64", "chunk4224_g1t3_d64"])
def test_head_subset_scoring(name, kind):
    """Scores on a subset of the query heads (online semantic-retrieval-head
    scoring): per-head logits of the chosen heads only ([B, R, H, ctx]),
    kv-group sums over the chosen heads (0 for a kv-head with none), scores,
    through both entry-point forms; attention output unchanged."""
    w = CASES[name]
    T, Hq, Hkv = w.gamma + 1, w.num_q_heads, w.num_kv_heads
    heads = _head_set(kind, Hq, Hq // Hkv)
    rows = (0, T - 1)
    say(f"[head subset] {name} heads={heads}")
    x = W.make_layer(w)
    d = to_device(x)
    o_ref, lse_ref = oracle.verify_attention(x.q, x.k, x.v, x.seq_lens)
    l_ref = oracle.collected_logits(x.q, x.k, x.seq_lens, rows, heads=heads)
    absl = np.where(np.isneginf(l_ref), 0.0, np.abs(l_ref))
    s_ref, s_floor = oracle.aggregate_scores(l_ref), oracle.aggregate_scores(absl)
    desc = Bn.make_desc(d.q, d.k, d.block_table, d.max_ctx)
    for layout, code in (("per_head", Bn.LOGITS_PER_HEAD), ("kvgroup_sum", Bn.LOGITS_KVGROUP_SUM)):
        out, lse, lg = Bn.verify_attention(d.q, d.k, d.v, d.seq_lens, block_table=d.block_table,
                                           max_ctx=d.max_ctx, collect_rows=rows, heads=heads,
                                           layout=layout)
        torch.cuda.synchronize()
        assert_out_close(out, o_ref, f"{name}/{layout}/{kind} out")
        assert_lse_close(lse, lse_ref, f"{name}/{layout}/{kind} lse")
        if layout == "per_head":
            assert lg.shape[2] == len(heads)
            assert_logits_close(lg.cpu().numpy(), l_ref, f"{name}/{kind} per-head logits")
        else:
            gs = oracle.kvgroup_sum(l_ref, Hkv, heads=heads, num_q_heads=Hq)
            gf = oracle.kvgroup_sum(absl, Hkv, heads=heads, num_q_heads=Hq)
            for b, L in enumerate(x.seq_lens):
                gs[b, :, int(L):] = np.nan  # past the length: not written (an empty group's 0 too)
            assert_logits_close(lg.cpu().numpy(), gs, f"{name}/{kind} group logits", floor=gf)
        sc = Bn.aggregate_scores(lg, d.seq_lens, Hq, Hkv, layout=layout)
        ws = torch.empty(Bn.verify_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        lg2 = torch.empty_like(lg)
        Bn.verify_partials(desc, d.q, d.k, d.v, d.seq_lens, d.block_table, rows, code, lg2, ws,
                           heads=heads)
        o2, l2, s2 = torch.empty_like(out), torch.empty_like(lse), torch.empty_like(sc)
        Bn.verify_finish(desc, d.seq_lens, ws, o2, l2, code, lg2, s2)
        torch.cuda.synchronize()
        assert_logits_close(sc.cpu().numpy(), s_ref, f"{name}/{layout}/{kind} scores", floor=s_floor)
        for b in range(w.batch):
            L = int(x.seq_lens[b])
            assert torch.equal(lg[b, ..., :L], lg2[b, ..., :L])
            assert torch.equal(sc[b, :L], s2[b, :L])


def test_scores_accumulate_over_layers():
    """Scores summed over several layers' calls (the layers whose heads are
    scored): aggregate and finish add to the scores already there."""
    w = CASES["g4t5_d64"]
    heads = (1, 6, 11)
    rows = (0, w.gamma)
    say("[accumulate over layers]")
    layers = [W.make_layer(w, layer=l) for l in (0, 3)]
    want = sum(oracle.aggregate_scores(oracle.collected_logits(x.q, x.k, x.seq_lens, rows, heads=heads))
               for x in layers)
    floor = sum(oracle.aggregate_scores(np.abs(np.nan_to_num(
        oracle.collected_logits(x.q, x.k, x.seq_lens, rows, heads=heads), neginf=0.0)))
        for x in layers)
    for layout, code in (("kvgroup_sum", Bn.LOGITS_KVGROUP_SUM), ("per_head", Bn.LOGITS_PER_HEAD)):
        s_agg, s_fin = None, None
        for i, x in enumerate(layers):
            d = to_device(x)
            _, _, lg = Bn.verify_attention(d.q, d.k, d.v, d.seq_lens, max_ctx=d.max_ctx,
                                           collect_rows=rows, heads=heads, layout=layout)
            s_agg = Bn.aggregate_scores(lg, d.seq_lens, w.num_q_heads, w.num_kv_heads, layout=layout,
                                        scores=s_agg, accumulate=i > 0)
            desc = Bn.make_desc(d.q, d.k, None, d.max_ctx)
            ws = torch.empty(Bn.verify_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
            lg2 = torch.empty_like(lg)
            Bn.verify_partials(desc, d.q, d.k, d.v, d.seq_lens, None, rows, code, lg2, ws, heads=heads)
            if s_fin is None:
                s_fin = torch.empty_like(s_agg)
            Bn.verify_finish(desc, d.seq_lens, ws, torch.empty_like(d.q),
                             torch.empty(d.q.shape[:3], dtype=torch.float32, device="cuda"), code,
                             lg2, s_fin, accumulate=i > 0)
        torch.cuda.synchronize()
        assert_logits_close(s_agg.cpu().numpy(), want, f"{layout} accumulated scores", floor=floor)
        for b in range(w.batch):
            L = int(layers[0].seq_lens[b])
            assert torch.equal(s_agg[b, :L], s_fin[b, :L])


def test_append_positions_for_draft_steps():
    """Draft-step lists: the selected positions followed by the drafted ones,
    appended in place; entries past the stride are dropped."""
    lens = np.array([100, 7, 50], np.int32)
    idx_h, n_h = W.index_lists(3, lens, count=5, stride=9)
    idx, n = dev_i32(idx_h), dev_i32(n_h)
    Bn.append_positions(dev_i32(lens), 0, 2, idx, n)      # draft step 1 and 2 at once
    Bn.append_positions(dev_i32(lens), 2, 3, idx, n)      # 3 more: the third list overflows
    torch.cuda.synchronize()
    got, cnt = idx.cpu().numpy(), n.cpu().numpy()
    for b, L in enumerate(lens):
        want = np.concatenate([idx_h[b, :n_h[b]], np.arange(L, L + 5)])[:9]
        assert cnt[b] == len(want)
        assert np.array_equal(got[b, :cnt[b]], want)
