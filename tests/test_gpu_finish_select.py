"""vgsa_verify_finish_select: combine + aggregate + top-k selection in one
launch, against the separate calls (vgsa_verify_finish, then vgsa_select_topk
on the scores it wrote) and against the oracle's selection on the GPU's own
scores.  Outputs, lse, scores, index lists and counts must be identical
(same per-element code; the selection is exact), positions past a length
untouched, and the selection workspace zero again after every call."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_long_amd import binding as Bn
from sparse_attention_long_amd import workloads as W
from tests.gpu_helpers import dev_i32, say, to_device

pytestmark = pytest.mark.gpu

CASES = {
    # unaligned capacity (4-byte score loads); a row no longer than the budget
    "g4t4_d128_ragged": W.small("fs_g4t4", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                gamma=3, lens=(301, 4, 128), budget=40, n_sink=4, window=8,
                                cap_align=1),
    "g4t5_d64": W.small("fs_g4t5", batch=2, num_q_heads=16, num_kv_heads=4, head_dim=64, gamma=4,
                        lens=(33, 257), budget=24, n_sink=2, window=6, seed=11),
    "paged_g8t6_d64": W.small("fs_pg", batch=3, num_q_heads=16, num_kv_heads=2, head_dim=64,
                              gamma=5, ctx=None, ctx_range=(40, 300), paged=True, budget=48,
                              n_sink=4, window=12, seed=15),
    # rows of one and two rounds of 32768 positions, several pieces each
    "two_rounds_g4t3_d64": W.small("fs_c2r", batch=4, num_q_heads=8, num_kv_heads=2, head_dim=64,
                                   gamma=2, lens=(65536, 32769, 20000, 4097), budget=300,
                                   n_sink=4, window=32, planted=40, seed=16),
}


def _finish_separately(desc, d, ws, code, lg, k, n_sink, window, stride, scores0=None):
    o = torch.empty_like(d.q)
    lse = torch.empty(d.q.shape[:3], dtype=torch.float32, device="cuda")
    s = torch.full((d.q.shape[0], d.max_ctx), 7.0, dtype=torch.float32, device="cuda") \
        if scores0 is None else scores0.clone()
    Bn.verify_finish(desc, d.seq_lens, ws, o, lse, code, lg, s, accumulate=scores0 is not None)
    idx, n = Bn.select_topk(s, d.seq_lens, k, n_sink, window, idx_stride=stride)
    return o, lse, s, idx, n


def _finish_fused(desc, d, ws, code, lg, k, n_sink, window, stride, sws, scores0=None):
    B = d.q.shape[0]
    o = torch.empty_like(d.q)
    lse = torch.empty(d.q.shape[:3], dtype=torch.float32, device="cuda")
    s = torch.full((B, d.max_ctx), 7.0, dtype=torch.float32, device="cuda") \
        if scores0 is None else scores0.clone()
    idx = torch.full((B, stride), -5, dtype=torch.int32, device="cuda")
    n = torch.full((B,), -5, dtype=torch.int32, device="cuda")
    Bn.verify_finish_select(desc, d.seq_lens, ws, o, lse, code, lg, s, k, n_sink, window, idx, n,
                            sws, accumulate=scores0 is not None)
    return o, lse, s, idx, n


def _assert_same(sep, fus, lens, k, n_sink, window, sws, what):
    torch.cuda.synchronize()
    o1, l1, s1, i1, n1 = sep
    o2, l2, s2, i2, n2 = fus
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), what
    assert torch.equal(l1, l2), what
    n1h, n2h = n1.cpu().numpy(), n2.cpu().numpy()
    assert np.array_equal(n1h, n2h), (what, n1h, n2h)
    s2h, i2h = s2.cpu().numpy(), i2.cpu().numpy()
    for b, L in enumerate(lens):
        L = int(L)
        assert torch.equal(s1[b, :L], s2[b, :L]), (what, b)
        assert np.all(s2h[b, L:] == s1[b, L:].cpu().numpy()), (what, b)  # untouched past L
        n = int(n2h[b])
        assert torch.equal(i1[b, :n], i2[b, :n]), (what, b)
        assert np.all(i2h[b, n:] == -5), (what, b)  # entries past the count untouched
        want = oracle.select_topk(s2h[b], L, k, n_sink, window)
        assert n == len(want) and np.array_equal(i2h[b, :n], want), (what, b, L)
    # the workspace opens with the histograms ([B][4096] u32) and the arrival
    # counters ([B] i32), each part 256-byte aligned: left zero for the next
    # call (the candidate lists after them are scratch)
    al = lambda n: -(-n // 256) * 256
    n_zero = al(len(lens) * 4096 * 4) + al(len(lens) * 4)
    assert int(torch.count_nonzero(sws[:n_zero])) == 0, f"{what}: histograms and counters not left zero"


@pytest.mark.parametrize("name", list(CASES))
def test_finish_select_matches_separate_calls(name):
    w = CASES[name]
    k, n_sink, window = w.budget, w.n_sink, w.window
    stride = k + 3
    sws = torch.zeros(Bn.finish_select_workspace_bytes(w.batch, w.max_ctx()), dtype=torch.uint8, device="cuda")
    for layer in (0, 1):  # the second call reuses the selection workspace
        x = W.make_layer(w, layer=layer)
        d = to_device(x)
        desc = Bn.make_desc(d.q, d.k, d.block_table, d.max_ctx)
        for layout, code in (("kvgroup_sum", Bn.LOGITS_KVGROUP_SUM), ("per_head", Bn.LOGITS_PER_HEAD)):
            say(f"[finish+select] {name} layer {layer} {layout}")
            ws = torch.empty(Bn.verify_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
            shape = (w.batch, w.num_kv_heads, d.max_ctx) if code == Bn.LOGITS_KVGROUP_SUM else \
                (w.batch, 2, w.num_q_heads, d.max_ctx)
            lg = torch.empty(shape, dtype=torch.float32, device="cuda")
            Bn.verify_partials(desc, d.q, d.k, d.v, d.seq_lens, d.block_table, w.collect_rows, code,
                               lg, ws)
            sep = _finish_separately(desc, d, ws, code, lg, k, n_sink, window, stride)
            fus = _finish_fused(desc, d, ws, code, lg, k, n_sink, window, stride, sws)
            _assert_same(sep, fus, x.seq_lens, k, n_sink, window, sws, f"{name} {layout} {layer}")


class _Dev:
    """A contiguous verify input (q, k, v, lengths) built from seeded randoms."""

    def __init__(self, seed, lens, max_ctx, hq=8, hkv=2, d=64, T=2):
        g = torch.Generator().manual_seed(seed)
        B = len(lens)
        self.q = torch.randn((B, hq, T, d), generator=g).to(torch.bfloat16).cuda()
        self.k = torch.randn((B, hkv, max_ctx, d), generator=g).to(torch.bfloat16).cuda()
        self.v = torch.randn((B, hkv, max_ctx, d), generator=g).to(torch.bfloat16).cuda()
        self.seq_lens = dev_i32(lens)
        self.block_table = None
        self.max_ctx = max_ctx


def _crafted_logits(kind, rng, B, hkv, M, lens):
    if kind == "normal":
        return (rng.standard_normal((B, hkv, M)) * 10).astype(np.float32)
    if kind == "integer_ties":  # scores of few distinct values: huge threshold bins
        return rng.integers(-3, 4, size=(B, hkv, M)).astype(np.float32)
    if kind == "all_zero":  # every score equal: the lowest positions win
        return np.zeros((B, hkv, M), np.float32)
    if kind == "threshold_bin":
        # 600 positions share the top 12 key bits of the threshold score, 10 lie
        # above them: the bin is ranked directly or refined by further passes
        lg = rng.uniform(0.0, 0.25, size=(B, hkv, M)).astype(np.float32)
        for b, L in enumerate(lens):
            if L > 800:
                pos = rng.choice(np.arange(4, L - 64), size=610, replace=False)
                lg[b, :, pos[:600]] = (1.0 + 0.1 * rng.random((600, 1))).astype(np.float32)
                lg[b, :, pos[600:]] = (3.0 + rng.random((10, 1))).astype(np.float32)
        return lg
    if kind == "minus_inf":  # -inf scores rank below every finite one
        lg = (rng.standard_normal((B, hkv, M)) * 10).astype(np.float32)
        lg[:, 0, ::3] = -np.inf
        return lg
    raise ValueError(kind)


KINDS = ["normal", "integer_ties", "all_zero", "threshold_bin", "minus_inf"]


@pytest.mark.parametrize("kind", KINDS)
def test_finish_select_crafted_scores(kind):
    """Scores built from chosen logits (the partials come from a real verify
    pass): two full rounds, one round plus one position, a row no longer than
    the budget and short rows; budgets with and without free positions; the
    scores accumulated onto earlier ones."""
    lens = [65536, 32769, 40, 1000, 2]
    M = 65536
    dv = _Dev(3, lens, M)
    desc = Bn.make_desc(dv.q, dv.k, None, M)
    ws = torch.empty(Bn.verify_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    lg0 = torch.empty((len(lens), 2, M), dtype=torch.float32, device="cuda")
    Bn.verify_partials(desc, dv.q, dv.k, dv.v, dv.seq_lens, None, (0, 1), Bn.LOGITS_KVGROUP_SUM,
                       lg0, ws)
    rng = np.random.default_rng(KINDS.index(kind))
    lg = torch.from_numpy(_crafted_logits(kind, rng, len(lens), 2, M, lens)).cuda()
    sws = torch.zeros(Bn.finish_select_workspace_bytes(len(lens), M), dtype=torch.uint8, device="cuda")
    base = torch.from_numpy(rng.standard_normal((len(lens), M)).astype(np.float32)).cuda()
    for k, n_sink, window in [(512, 4, 64), (68, 4, 64), (6000, 4, 256), (1, 0, 0)]:
        for acc in (None, base):
            what = f"{kind} k={k} sinks={n_sink} window={window} acc={acc is not None}"
            say(f"[finish+select crafted] {what}")
            sep = _finish_separately(desc, dv, ws, Bn.LOGITS_KVGROUP_SUM, lg, k, n_sink, window,
                                     k + 1, scores0=acc)
            fus = _finish_fused(desc, dv, ws, Bn.LOGITS_KVGROUP_SUM, lg, k, n_sink, window, k + 1,
                                sws, scores0=acc)
            _assert_same(sep, fus, lens, k, n_sink, window, sws, what)


@pytest.mark.parametrize("M,lens", [
    (131088, [131088, 100001, 65537, 700]),   # five rounds (16-byte loads)
    (131078, [131078, 99999, 32768]),          # unaligned capacity (4-byte loads)
    (262144, [262144, 200000]),                # eight rounds
])
def test_finish_select_long_rows(M, lens):
    """Rows of up to eight rounds of 32768 positions: the selecting workgroup
    reloads the row per pass; threshold bins above the reloaded-row cap take
    further radix passes."""
    dv = _Dev(5, lens, M, hq=4, hkv=1, d=64, T=2)
    desc = Bn.make_desc(dv.q, dv.k, None, M)
    ws = torch.empty(Bn.verify_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    lg0 = torch.empty((len(lens), 1, M), dtype=torch.float32, device="cuda")
    Bn.verify_partials(desc, dv.q, dv.k, dv.v, dv.seq_lens, None, (0, 1), Bn.LOGITS_KVGROUP_SUM,
                       lg0, ws)
    sws = torch.zeros(Bn.finish_select_workspace_bytes(len(lens), M), dtype=torch.uint8, device="cuda")
    for kind in ("normal", "integer_ties", "threshold_bin"):
        rng = np.random.default_rng(KINDS.index(kind) + 7)
        lg = torch.from_numpy(_crafted_logits(kind, rng, len(lens), 1, M, lens)).cuda()
        for k, n_sink, window in [(6554, 4, 256), (512, 4, 64)]:
            what = f"M={M} {kind} k={k}"
            say(f"[finish+select long rows] {what}")
            sep = _finish_separately(desc, dv, ws, Bn.LOGITS_KVGROUP_SUM, lg, k, n_sink, window, k)
            fus = _finish_fused(desc, dv, ws, Bn.LOGITS_KVGROUP_SUM, lg, k, n_sink, window, k, sws)
            _assert_same(sep, fus, lens, k, n_sink, window, sws, what)
