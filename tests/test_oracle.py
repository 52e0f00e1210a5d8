"""Pins of the fp64 oracle against facts fixed outside it.

Each test ties an oracle function to something other than its own formula:
a library routine it must reduce to (torch CPU fp64 scaled_dot_product_attention),
a closed form, an invariant of the definitions, or brute force over every
subset on tiny inputs (the argmax of Vegas, "A. aggregated attention-logit
selection", restricted by the protected sinks/window of Dustin, "1. hybrid
attention aggregation").
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_long_amd import workloads as W


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def causal_mask(T, L):
    """bool [T, L]: row t sees j <= L - T + t (bottom-right aligned)."""
    j = np.arange(L)[None, :]
    t = np.arange(T)[:, None]
    return j <= (L - T + t)


# ------------------------------------------------------------------ verify attention
@pytest.mark.parametrize("T", [1, 4])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2)])
def test_verify_equals_torch_sdpa_fp64(T, Hq, Hkv):
    B, d, ctx = 3, 16, 40
    lens = [40, 23, T]  # full, ragged, minimal (only the verify tokens)
    q, k, v = rnd((B, Hq, T, d), 1), rnd((B, Hkv, ctx, d), 2), rnd((B, Hkv, ctx, d), 3)
    o, lse = oracle.verify_attention(q, k, v, lens)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        qt = torch.from_numpy(q[b])
        kt = torch.from_numpy(k[b, :, :L]).repeat_interleave(G, dim=0)
        vt = torch.from_numpy(v[b, :, :L]).repeat_interleave(G, dim=0)
        mask = torch.from_numpy(causal_mask(T, L))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        np.testing.assert_allclose(o[b], ref.numpy(), rtol=0, atol=1e-12)
        # lse against torch.logsumexp of the library's own masked score matrix
        s = (qt @ kt.transpose(-1, -2)) / math.sqrt(d)
        s = s.masked_fill(~mask, float("-inf"))
        np.testing.assert_allclose(lse[b], torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_softmax_weights_sum_to_one():
    # V = identity rows: o[r] is the weight vector itself.
    d, L, T = 64, 50, 5
    q, k = rnd((1, 2, T, d), 4), rnd((1, 1, L, d), 5)
    v = np.zeros((1, 1, L, L))
    v[0, 0] = np.eye(L)
    o, _ = oracle.verify_attention(q, k, v, [L], scale=0.3)
    w = o[0].reshape(-1, L)
    assert np.all(w >= 0)
    assert np.max(np.abs(w.sum(axis=1) - 1.0)) < 1e-12
    # causally hidden positions carry zero weight
    for t in range(T):
        assert np.all(o[0, :, t, L - T + t + 1:] == 0.0)


def test_constant_values_and_identical_keys():
    d, L, T = 32, 70, 3
    q, k = rnd((2, 4, T, d), 6), rnd((2, 2, L, d), 7)
    vrow = rnd(d, 8)
    v = np.broadcast_to(vrow, (2, 2, L, d)).copy()
    o, _ = oracle.verify_attention(q, k, v, [L, 41])
    np.testing.assert_allclose(o, np.broadcast_to(vrow, o.shape), rtol=0, atol=1e-13)
    # identical keys: uniform weights -> mean of the visible values; lse = s + ln(n)
    k_same = np.broadcast_to(rnd(d, 9), (2, 2, L, d)).copy()
    v2 = rnd((2, 2, L, d), 10)
    o2, lse2 = oracle.verify_attention(q, k_same, v2, [L, 41])
    for b, Lb in enumerate([L, 41]):
        for h in range(4):
            g = h // 2
            for t in range(T):
                n = Lb - T + t + 1
                np.testing.assert_allclose(o2[b, h, t], v2[b, g, :n].mean(axis=0), atol=1e-12)
                s = q[b, h, t] @ k_same[b, g, 0] / math.sqrt(d)
                assert abs(lse2[b, h, t] - (s + math.log(n))) < 1e-12


def test_single_visible_position():
    # L == T: row 0 sees only position 0 -> o = v_0, lse = s_0
    d, T = 16, 4
    q, k, v = rnd((1, 2, T, d), 11), rnd((1, 1, T, d), 12), rnd((1, 1, T, d), 13)
    o, lse = oracle.verify_attention(q, k, v, [T], scale=0.5)
    np.testing.assert_array_equal(o[0, :, 0], np.broadcast_to(v[0, 0, 0], (2, d)))
    np.testing.assert_allclose(lse[0, :, 0], 0.5 * (q[0, :, 0] @ k[0, 0, 0]), atol=1e-14)


# ------------------------------------------------------------------ collected logits
@pytest.mark.parametrize("rows", [(0, 4), (0, 1, 2, 3, 4), (2,), (1, 3)])
def test_logits_closed_form_basis_keys(rows):
    # k[g, j] = (g + 1) * e_{(j + g) mod d}  =>  l[c, h, j] = scale * (g+1) * q[h, r_c][(j+g) mod d]
    B, Hq, Hkv, T, d, ctx = 2, 6, 3, 5, 8, 30
    lens = [30, 17]
    q = rnd((B, Hq, T, d), 14)
    k = np.zeros((B, Hkv, ctx, d))
    for g in range(Hkv):
        for j in range(ctx):
            k[:, g, j, (j + g) % d] = g + 1
    sc = 0.25
    l = oracle.collected_logits(q, k, lens, rows, scale=sc)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        for c, r in enumerate(rows):
            for h in range(Hq):
                g = h // G
                for j in range(L):
                    want = sc * (g + 1) * q[b, h, r, (j + g) % d] if j <= L - T + r else -np.inf
                    assert l[b, c, h, j] == want
            assert np.all(np.isnan(l[b, c, :, L:]))


def test_logits_depend_only_on_collected_rows():
    B, Hq, Hkv, T, d, L = 1, 4, 2, 5, 16, 25
    q, k = rnd((B, Hq, T, d), 15), rnd((B, Hkv, L, d), 16)
    l1 = oracle.collected_logits(q, k, [L], (0, 4))
    q2 = q.copy()
    q2[:, :, 1:4] += 3.0  # rows that are not collected
    assert np.array_equal(l1, oracle.collected_logits(q2, k, [L], (0, 4)), equal_nan=True)
    q3 = q.copy()
    q3[:, :, 4] += 1.0    # the bonus row
    l3 = oracle.collected_logits(q3, k, [L], (0, 4))
    assert np.array_equal(l1[:, 0], l3[:, 0], equal_nan=True)
    assert not np.allclose(l1[:, 1, :, :L - T + 4], l3[:, 1, :, :L - T + 4])


def test_scores_per_head_equal_regrouped_sum():
    B, Hq, Hkv, T, d, L = 2, 8, 2, 4, 16, 33
    q, k = rnd((B, Hq, T, d), 17), rnd((B, Hkv, L, d), 18)
    l = oracle.collected_logits(q, k, [L, L], (0, 3))
    s1 = oracle.aggregate_scores(l)
    s2 = oracle.aggregate_scores(oracle.kvgroup_sum(l, Hkv))
    fin = np.isfinite(s1)
    np.testing.assert_allclose(s1[fin], s2[fin], rtol=1e-13, atol=1e-12)
    assert np.array_equal(np.isneginf(s1), np.isneginf(s2))
    # linearity: the score of position j is the sum of its 2*Hq logits
    b, j = 1, 7
    assert abs(s1[b, j] - sum(l[b, c, h, j] for c in range(2) for h in range(Hq))) < 1e-12


def test_scores_all_rows_closed_form():
    # Collecting every verify row (the full sum of Vegas "A."): for a position
    # every row sees, the score is scale * k_g[j] . (sum over rows and the
    # group's heads of q), one dot product per kv-head; the last T - 1
    # positions are hidden from row 0 and score -inf.
    B, Hq, Hkv, T, d = 2, 8, 2, 5, 16
    lens = [40, 23]
    q, k = rnd((B, Hq, T, d), 19), rnd((B, Hkv, 40, d), 20)
    sc = 0.3
    l = oracle.collected_logits(q, k, lens, range(T), scale=sc)
    assert l.shape == (B, T, Hq, 40)
    s = oracle.aggregate_scores(oracle.kvgroup_sum(l, Hkv))
    G = Hq // Hkv
    for b, L in enumerate(lens):
        qsum = [q[b, g * G:(g + 1) * G].sum(axis=(0, 1)) for g in range(Hkv)]
        want = sc * sum(k[b, g, :L - T + 1] @ qsum[g] for g in range(Hkv))
        np.testing.assert_allclose(s[b, :L - T + 1], want, rtol=1e-12, atol=1e-12)
        assert np.all(np.isneginf(s[b, L - T + 1:L]))
    # the Collect-2 rows are a subset: their per-head logits are the same values
    l2 = oracle.collected_logits(q, k, lens, (0, T - 1), scale=sc)
    assert np.array_equal(l2, l[:, [0, T - 1]], equal_nan=True)


@pytest.mark.parametrize("heads", [(1, 4), (0,), (5,), (0, 1, 2, 3, 4, 5)])
def test_logits_head_subset_closed_form(heads):
    # basis keys again: l[c, i, j] = scale * (g+1) * q[heads[i], r_c][(j+g) mod d], g = heads[i] // G
    B, Hq, Hkv, T, d, ctx = 2, 6, 3, 4, 8, 30
    lens = [30, 19]
    rows = (0, 3)
    q = rnd((B, Hq, T, d), 21)
    k = np.zeros((B, Hkv, ctx, d))
    for g in range(Hkv):
        for j in range(ctx):
            k[:, g, j, (j + g) % d] = g + 1
    sc = 0.5
    l = oracle.collected_logits(q, k, lens, rows, scale=sc, heads=heads)
    assert l.shape == (B, len(rows), len(heads), ctx)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        for c, r in enumerate(rows):
            for i, h in enumerate(heads):
                g = h // G
                for j in range(L):
                    want = sc * (g + 1) * q[b, h, r, (j + g) % d] if j <= L - T + r else -np.inf
                    assert l[b, c, i, j] == want


def test_head_subset_group_sums_closed_form():
    """Scores restricted to a head subset (Dustin's online SRH scoring): per
    kv-head, scale * k_g[j] . (sum of the collected rows of its selected
    heads' queries); a kv-head with no selected head contributes 0."""
    B, Hq, Hkv, T, d, L = 1, 8, 4, 3, 16, 50
    q, k = rnd((B, Hq, T, d), 22), rnd((B, Hkv, L, d), 23)
    heads = [1, 2, 7]          # groups 0, 1, 3 (G = 2); group 2 has none
    rows = (0, 2)
    sc = 0.25
    l = oracle.collected_logits(q, k, [L], rows, scale=sc, heads=heads)
    gs = oracle.kvgroup_sum(l, Hkv, heads=heads, num_q_heads=Hq)
    G = Hq // Hkv
    vis = L - T + 1  # positions every collected row sees (row 0's limit)
    for g in range(Hkv):
        qs = sum(q[0, h, t] for h in heads if h // G == g for t in rows)
        want = sc * (k[0, g, :vis] @ qs) if np.ndim(qs) else np.zeros(vis)
        np.testing.assert_allclose(gs[0, g, :vis], want, rtol=1e-12, atol=1e-12)
    assert np.all(gs[0, 2] == 0)
    assert np.all(np.isneginf(gs[0, [0, 1, 3], vis:L]))
    # the subset is the restriction of the all-heads logits
    full = oracle.collected_logits(q, k, [L], rows, scale=sc)
    assert np.array_equal(l, full[:, :, heads], equal_nan=True)


# ------------------------------------------------------------------ selection
def brute_force_best(scores, L, k, n_sink, window):
    forced = set(range(min(n_sink, L))) | set(range(max(0, L - window), L))
    rest = [j for j in range(L) if j not in forced]
    best, best_sets = -np.inf, []
    for extra in itertools.combinations(rest, k - len(forced)):
        tot = sum(scores[j] for j in extra)
        if tot > best:
            best, best_sets = tot, [set(extra) | forced]
        elif tot == best:
            best_sets.append(set(extra) | forced)
    return best, best_sets, forced


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("L,k,n_sink,window", [(10, 5, 1, 2), (12, 7, 2, 3), (14, 6, 0, 0),
                                               (13, 4, 4, 0), (11, 5, 0, 5), (9, 3, 1, 1)])
def test_select_attains_bruteforce_argmax(seed, L, k, n_sink, window):
    rng = np.random.default_rng(seed)
    # integer-valued, tie-heavy scores
    scores = rng.integers(-3, 4, size=L).astype(np.float64)
    got = oracle.select_topk(scores, L, k, n_sink, window)
    best, best_sets, forced = brute_force_best(scores, L, k, n_sink, window)
    gs = set(int(x) for x in got)
    assert gs in best_sets
    assert forced <= gs and len(gs) == k and list(got) == sorted(gs)
    # among equal scores the lower positions win
    free_sel = [j for j in gs if j not in forced]
    free_out = [j for j in range(L) if j not in gs]
    for i in free_sel:
        for j in free_out:
            assert scores[i] > scores[j] or (scores[i] == scores[j] and i < j)


def test_select_edge_cases():
    s = np.array([5.0, -0.0, 0.0, -np.inf, 2.0, 0.0, -np.inf, 1.0])
    # k >= L keeps everything
    assert list(oracle.select_topk(s, 8, 8, 1, 1)) == list(range(8))
    assert list(oracle.select_topk(s, 5, 9, 1, 1)) == list(range(5))
    # -0.0 == +0.0: ties go to the lower position; -inf ranks last, ties by position
    assert list(oracle.select_topk(s, 8, 3, 0, 0)) == [0, 4, 7]
    assert list(oracle.select_topk(s, 8, 5, 0, 0)) == [0, 1, 2, 4, 7]
    assert list(oracle.select_topk(s, 8, 7, 0, 0)) == [0, 1, 2, 3, 4, 5, 7]
    # sinks + window == k: exactly the forced set
    assert list(oracle.select_topk(s, 8, 4, 2, 2)) == [0, 1, 6, 7]
    # L shorter than sinks + window (so k >= L as well): every position is kept
    assert list(oracle.select_topk(s, 5, 6, 3, 3)) == [0, 1, 2, 3, 4]
    # sinks and window overlapping inside L: forced set is their union
    assert list(oracle.select_topk(s, 6, 5, 2, 3)) == [0, 1, 3, 4, 5]
    assert list(oracle.select_topk(s, 0, 4, 1, 1)) == []
    with pytest.raises(ValueError):
        oracle.select_topk(s, 8, 3, 2, 2)


def _lexmin_best(values, cands, size):
    """Brute force: the size-`size` subsets of `cands` with the largest value
    sum; of those, the one whose sorted positions come first."""
    best, best_set = -np.inf, None
    for sub in itertools.combinations(sorted(cands), size):
        tot = sum(values[j] for j in sub)
        if tot > best or (tot == best and (best_set is None or sub < best_set)):
            best, best_set = tot, sub
    return set(best_set if best_set is not None else ())


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("L,k,m,n_sink,window", [(10, 6, 2, 1, 2), (12, 7, 3, 2, 1), (11, 5, 5, 0, 0),
                                                 (12, 6, 0, 1, 1), (9, 5, 9, 1, 1), (13, 8, 4, 0, 3)])
def test_hybrid_select_bruteforce(seed, L, k, m, n_sink, window):
    """Dustin "1.": sinks + window, then the best min(m, r) free positions by
    the draft signal, then the best of the rest by the target signal: each
    stage checked by brute force over all subsets (tie-heavy integer scores;
    among equal sums the lowest positions)."""
    rng = np.random.default_rng(100 + seed)
    tgt = rng.integers(-2, 3, size=L).astype(np.float64)
    drf = rng.integers(-2, 3, size=L).astype(np.float64)
    got = set(int(x) for x in oracle.select_topk_hybrid(tgt, drf, L, k, m, n_sink, window))
    forced = set(range(min(n_sink, L))) | set(range(max(0, L - window), L))
    r = k - len(forced)
    m_eff = min(m, r)
    free = [j for j in range(L) if j not in forced]
    from_draft = _lexmin_best(drf, free, m_eff)
    rest = [j for j in free if j not in from_draft]
    from_target = _lexmin_best(tgt, rest, r - m_eff)
    assert got == forced | from_draft | from_target
    assert len(got) == k


def test_hybrid_select_reductions():
    rng = np.random.default_rng(7)
    L, k, n_sink, window = 300, 40, 4, 16
    tgt = rng.standard_normal(L)
    drf = rng.standard_normal(L)
    plain_t = oracle.select_topk(tgt, L, k, n_sink, window)
    plain_d = oracle.select_topk(drf, L, k, n_sink, window)
    # m = 0: the target signal alone; m >= r: the draft signal alone
    assert np.array_equal(oracle.select_topk_hybrid(tgt, drf, L, k, 0, n_sink, window), plain_t)
    for m in (k - n_sink - window, k, 10 ** 6):
        assert np.array_equal(oracle.select_topk_hybrid(tgt, drf, L, k, m, n_sink, window), plain_d)
    # one signal for both stages: the hierarchy is the plain top-k, for every m
    for m in (0, 1, 7, 20, 25):
        assert np.array_equal(oracle.select_topk_hybrid(tgt, tgt, L, k, m, n_sink, window), plain_t)
    # the draft stage's picks are the top-m of the draft signal among the free positions
    got = oracle.select_topk_hybrid(tgt, drf, L, k, 9, n_sink, window)
    free = np.arange(n_sink, L - window)
    top_d = free[np.argsort(-drf[free], kind="stable")[:9]]
    assert set(top_d.tolist()) <= set(got.tolist())
    # k >= L, L = 0, and a budget the protected ranges exceed
    assert list(oracle.select_topk_hybrid(tgt, drf, 30, 30, 5, 1, 1)) == list(range(30))
    assert list(oracle.select_topk_hybrid(tgt, drf, 0, 4, 1, 1, 1)) == []
    with pytest.raises(ValueError):
        oracle.select_topk_hybrid(tgt, drf, L, 10, 2, 6, 6)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("L,kb,block,n_sink,window", [(23, 3, 4, 1, 2), (32, 4, 4, 0, 0), (30, 4, 4, 5, 3),
                                                      (17, 3, 2, 2, 1), (40, 3, 8, 0, 9), (21, 5, 3, 0, 0)])
def test_select_blocks_bruteforce(seed, L, kb, block, n_sink, window):
    """Whole blocks kept: brute force over every set of free blocks (tie-heavy
    integer scores, exact in float32): the chosen blocks have the largest
    summed member score, the lowest blocks among equal sums, and the output
    is every position below L of the forced and chosen blocks."""
    rng = np.random.default_rng(200 + seed)
    sc = rng.integers(-3, 4, size=L).astype(np.float64)
    got = [int(x) for x in oracle.select_blocks(sc, L, kb, block, n_sink, window)]
    nb = -(-L // block)
    members = [list(range(i * block, min(L, (i + 1) * block))) for i in range(nb)]
    forced = set(range(min(-(-n_sink // block), nb)))
    if window > 0:
        forced |= set(range(max(0, L - window) // block, nb))
    free = [i for i in range(nb) if i not in forced]
    best, best_set = -np.inf, None
    for sub in itertools.combinations(free, kb - len(forced)):
        tot = sum(sc[j] for i in sub for j in members[i])
        if tot > best or (tot == best and sub < best_set):
            best, best_set = tot, sub
    want = sorted(j for i in sorted(forced | set(best_set)) for j in members[i])
    assert got == want
    # every sink and window position is kept
    assert set(range(min(n_sink, L))) | set(range(max(0, L - window), L)) <= set(got)


def test_select_blocks_reductions_and_edges():
    rng = np.random.default_rng(9)
    L = 500
    sc = rng.standard_normal(L).astype(np.float32)
    # block 1 is the position-level selection
    for k, ns, win in [(40, 4, 16), (1, 0, 0), (100, 0, 99)]:
        assert np.array_equal(oracle.select_blocks(sc, L, k, 1, ns, win),
                              oracle.select_topk(sc, L, k, ns, win))
    # block sums: the partial last block holds positions 32..36 only; on
    # integer scores they equal the integer sums (python ints, exact)
    si = rng.integers(-50, 50, size=37).astype(np.float32)
    bs = oracle.block_sums(si, 37, 16)
    assert bs.dtype == np.float64 and bs.shape == (3,)
    ints = [int(x) for x in si]
    assert list(bs) == [sum(ints[0:16]), sum(ints[16:32]), sum(ints[32:37])]
    # block 1: every block sum is its one score
    assert np.array_equal(oracle.block_sums(sc, 37, 1), sc[:37].astype(np.float64))
    # exact, not float32 in position order: 2^24 + 1 + 1 + 1 + 1 is 2^24 + 4
    # (a float32 running sum stays at 2^24), and 1e8 - 1e8 + 0.5 keeps the 0.5
    big = np.array([2.0 ** 24, 1, 1, 1, 1, 1e8, -1e8, 0.5], dtype=np.float32)
    assert list(oracle.block_sums(big, 8, 5)) == [2.0 ** 24 + 4, 0.5]
    # the block sums of a row add up to its total (dyadic scores: exact)
    dy = rng.integers(-1000, 1000, size=500).astype(np.float32) / np.float32(64)
    assert oracle.block_sums(dy, 500, 16).sum() == float(dy.astype(np.float64).sum())
    # a -inf member makes its block -inf
    sinf = np.ones(40, np.float32)
    sinf[17] = -np.inf
    assert list(oracle.block_sums(sinf, 40, 16)) == [16.0, -np.inf, 8.0]
    # ranking given sums: the sums decide, not the scores
    given = np.array([0.0, 5.0, 1.0, 9.0, 2.0])
    assert list(oracle.select_blocks(si, 37, 2, 8, 0, 0, sums=given)) == list(range(8, 16)) + list(range(24, 32))
    with pytest.raises(ValueError):
        oracle.select_blocks(si, 37, 2, 8, 0, 0, sums=given[:3])
    # k_blocks covering every block keeps everything; L = 0 keeps nothing
    assert list(oracle.select_blocks(sc, 37, 3, 16, 1, 1)) == list(range(37))
    assert list(oracle.select_blocks(sc, 0, 3, 16, 1, 1)) == []
    # a window across a block boundary forces both blocks
    got = oracle.select_blocks(sc, 64, 3, 16, 0, 20)
    assert set(range(32, 64)) <= set(got.tolist()) and len(got) == 48
    with pytest.raises(ValueError):
        oracle.select_blocks(sc, 64, 2, 16, 1, 20)
    # a -inf member sinks its whole block
    s2 = np.ones(64, np.float32)
    s2[20] = -np.inf
    assert 20 not in oracle.select_blocks(s2, 64, 3, 16, 0, 0).tolist()


def test_select_planted_positions_win_on_small_workload():
    """Planted keys (aligned with the group's queries) must be selected: their
    summed logit is far above the spread of the unplanted ones."""
    w = W.WORKLOADS["ctx2k_b1_h32kv8_d128"]
    x = W.make_layer(w)
    l = oracle.collected_logits(x.q, x.k, x.seq_lens, w.collect_rows)
    scores = oracle.aggregate_scores(l)
    sel = oracle.select_topk(scores[0], int(x.seq_lens[0]), w.budget, w.n_sink, w.window)
    assert len(sel) == w.budget
    assert set(x.planted[0].tolist()) <= set(sel.tolist())


# ------------------------------------------------------------------ sparse attention
def test_sparse_with_every_position_equals_verify():
    B, Hq, Hkv, T, d, ctx = 2, 4, 2, 3, 16, 45
    lens = [45, 29]
    q, k, v = rnd((B, Hq, T, d), 19), rnd((B, Hkv, ctx, d), 20), rnd((B, Hkv, ctx, d), 21)
    o1, l1 = oracle.verify_attention(q, k, v, lens)
    o2, l2 = oracle.sparse_attention(q, k, v, lens, [np.arange(L) for L in lens])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_sparse_equals_torch_sdpa_on_gathered_subset():
    B, Hq, Hkv, T, d, L = 1, 6, 3, 4, 32, 80
    q, k, v = rnd((B, Hq, T, d), 22), rnd((B, Hkv, L, d), 23), rnd((B, Hkv, L, d), 24)
    idx = np.sort(np.random.default_rng(25).choice(L, 20, replace=False))
    idx[-1] = L - 1
    o, lse = oracle.sparse_attention(q, k, v, [L], [idx])
    G = Hq // Hkv
    qt = torch.from_numpy(q[0])
    kt = torch.from_numpy(k[0][:, idx]).repeat_interleave(G, dim=0)
    vt = torch.from_numpy(v[0][:, idx]).repeat_interleave(G, dim=0)
    mask = torch.from_numpy(idx[None, :] <= (L - T + np.arange(T))[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    np.testing.assert_allclose(o[0], ref.numpy(), atol=1e-12)


def test_sparse_single_index_and_empty_rows():
    d, T, L = 16, 3, 50
    q, k, v = rnd((1, 2, T, d), 26), rnd((1, 1, L, d), 27), rnd((1, 1, L, d), 28)
    o, lse = oracle.sparse_attention(q, k, v, [L], [np.array([17])], scale=0.5)
    for t in range(T):
        np.testing.assert_array_equal(o[0, :, t], np.broadcast_to(v[0, 0, 17], (2, d)))
        np.testing.assert_allclose(lse[0, :, t], 0.5 * (q[0, :, t] @ k[0, 0, 17]), atol=1e-14)
    # only the last position listed: rows that cannot see it get o = 0, lse = -inf
    o, lse = oracle.sparse_attention(q, k, v, [L], [np.array([L - 1])])
    assert np.all(o[0, :, :T - 1] == 0) and np.all(np.isneginf(lse[0, :, :T - 1]))
    np.testing.assert_array_equal(o[0, :, T - 1], np.broadcast_to(v[0, 0, L - 1], (2, d)))
    # empty list
    o, lse = oracle.sparse_attention(q, k, v, [L], [np.zeros(0, dtype=np.int64)])
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], dtype=np.uint16)
    want = [1.0, -1.0, 0.0, -0.0, 3.3895313892515355e38, 9.183549615799121e-41, 3.140625]
    got = oracle.widen_bf16(bits)
    assert list(got) == want
    assert math.copysign(1.0, got[3]) == -1.0


def test_block_positions_expands_block_lists():
    """Block lists stand for whole blocks of positions, clipped to the length
    (closed forms), and the positions block selection keeps are exactly the
    expansion of the blocks they fall in."""
    assert list(oracle.block_positions([0, 2], 16, 40)) == list(range(16)) + list(range(32, 40))
    assert list(oracle.block_positions([1, 3], 5, 100)) == [5, 6, 7, 8, 9, 15, 16, 17, 18, 19]
    assert list(oracle.block_positions([], 16, 40)) == []
    assert list(oracle.block_positions([2], 16, 32)) == []          # a block wholly past the length
    assert list(oracle.block_positions([0, 1, 2], 1, 3)) == [0, 1, 2]  # block 1: the ids themselves
    rng = np.random.default_rng(4)
    for L, kb, block, ns, win in [(500, 7, 16, 4, 40), (37, 2, 8, 0, 0), (1000, 30, 5, 3, 17)]:
        sc = rng.standard_normal(L).astype(np.float32)
        pos = oracle.select_blocks(sc, L, kb, block, ns, win)
        ids = np.unique(pos // block)
        assert np.array_equal(oracle.block_positions(ids, block, L), pos)
