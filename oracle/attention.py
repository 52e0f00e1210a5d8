"""Plain fp64 CPU oracle of verification-guided sparse attention.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package.  The product path (the HIP library and
its Python binding) never calls it, links it or shares code with it.

Everything is computed in float64 from the plain definitions, with matrix
products, sums, exp/log and a sort as the only library steps.  bf16 inputs
arrive as uint16 bit patterns and are widened exactly.

Sources (pages are cited by title and section):
  * Vegas, section 2 "core mechanism", step 1: the verify pass is a standard
    forward pass with full attention, so it computes the attention logits of
    every KV entry.  -> verify_attention
  * Vegas, section 2, "A. aggregated attention-logit selection": the selected
    prefix set T (|T| = k) maximises the sum, over the gamma+1 draft/bonus
    tokens and all query heads, of the logits l_ti^(h) of its members.
    -> aggregate_scores, select_topk
  * Vegas, "B. Collect-2-Query": logits are collected only for the first draft
    token and the bonus token.  -> collected_logits
  * Vegas, section 3 "implementation": the logits written out are the ones
    before softmax normalisation; drafting runs a page-size-1 paged attention
    whose page indices are the selected token indices.  -> sparse_attention
  * Dustin, "1. hybrid attention aggregation": a few attention-sink prefix
    tokens and a local window of recent tokens are protected first, and the
    remaining budget is filled by score.  -> select_topk
  * Dustin, "1. hybrid attention aggregation": the two signals (target
    historical attention from the previous forward pass, draft lookahead
    attention from drafting) fill that budget hierarchically, the top-m by the
    draft signal first, the rest by the target signal.  -> select_topk_hybrid
  * The euno.news summary of arXiv 2512.21911, "3. sparse verification
    engine": attention keeps the top keys in structured blocks.  -> select_blocks

Readings where the pages are silent (each one is listed with its reason in
the design notes):
  * Row t of the T = gamma+1 verify rows sits at absolute position L-T+t, where
    L counts the cached positions including the T verify tokens themselves; it
    sees positions j <= L-T+t (causal, bottom-right aligned).  Masked logits
    are -inf.
  * The collected rows are row 0 (first draft token) and row gamma (bonus)
    unless a caller names others (every row: the full sum of "A.").
  * A logit is scale * q.k with scale = 1/sqrt(d), the quantity softmax reads.
  * The budget k includes sinks and window; if k >= L every position is kept.
  * Ties in score are broken by the lower position; -0.0 equals +0.0.
  * Hybrid selection: m counts the draft-chosen positions among those not
    protected, clamped to the remaining budget; the draft scores are an input
    array of the same shape as the target scores.
  * Selected indices are returned in ascending order.
  * Sparse attention applies the same causal rule to the absolute positions in
    the index list; a row with no visible index yields o = 0, lse = -inf.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------- inputs
def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("expected uint16 bf16 bit patterns")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


# --------------------------------------------------------------------------- attention core
def attend(q_rows: np.ndarray, keys: np.ndarray, values: np.ndarray,
           visible: Sequence[int], scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of R query rows over N ordered keys.

    Row r sees the first visible[r] keys.  With s_j = scale * q.k_j:
        m = max_j s_j,  p_j = exp(s_j - m),  Z = sum_j p_j,
        o = sum_j p_j v_j / Z,  lse = m + ln Z.
    A row that sees nothing gets o = 0 and lse = -inf.
    Returns o [R, d] and lse [R] in float64.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    R, d = q_rows.shape
    N = keys.shape[0]
    o = np.zeros((R, values.shape[1] if values.ndim == 2 else d), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if N == 0:
        return o, lse
    s = scale * (q_rows @ keys.T)                     # [R, N]
    for r in range(R):
        n = int(min(max(visible[r], 0), N))
        if n == 0:
            continue
        sr = s[r, :n]
        m = sr.max()
        p = np.exp(sr - m)
        z = p.sum()
        o[r] = (p @ values[:n]) / z
        lse[r] = m + math.log(z)
    return o, lse


# --------------------------------------------------------------------------- verify
def verify_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens: Sequence[int],
                     scale: Optional[float] = None,
                     heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Full-attention verify pass (Vegas, section 2 "core mechanism", step 1).

    q [B, Hq, T, d]; k, v logical caches [B, Hkv, ctx, d] (float64 or bf16 bits);
    seq_lens [B] counts the T verify tokens.  GQA: q-head h reads kv-head
    h // (Hq / Hkv).  Returns o [B, Hq, T, d] and lse [B, Hq, T]; heads not in
    `heads` (when given) are left as NaN.
    """
    q = _f64(q)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = default_scale(d) if scale is None else scale
    o = np.full((B, Hq, T, v.shape[3]), np.nan)
    lse = np.full((B, Hq, T), np.nan)
    want = set(range(Hq)) if heads is None else set(heads)
    for b in range(B):
        L = int(seq_lens[b])
        for g in range(Hkv):
            hs = [h for h in range(g * G, (g + 1) * G) if h in want]
            if not hs:
                continue
            rows = q[b, hs].reshape(-1, d)                       # (h, t) row-major
            vis = [L - T + t + 1 for _ in hs for t in range(T)]  # row t sees j <= L-T+t
            ob, lb = attend(rows, _f64(k[b, g, :L]), _f64(v[b, g, :L]), vis, sc)
            o[b, hs] = ob.reshape(len(hs), T, -1)
            lse[b, hs] = lb.reshape(len(hs), T)
    return o, lse


# --------------------------------------------------------------------------- logits
def collected_logits(q: np.ndarray, k: np.ndarray, seq_lens: Sequence[int],
                     rows: Sequence[int], scale: Optional[float] = None,
                     heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """Pre-softmax logits of the collected rows (Vegas, section 3: written
    before softmax normalisation).  "A." sums its score over every verify row
    t = 1..gamma+1; "B. Collect-2-Query" keeps only the first draft row and
    the bonus row.  `rows` names the collected rows (0-based, ascending), so
    both readings are this one function.

    `heads` restricts collection to a subset of the query heads (Dustin,
    "2. ... semantic retrieval heads", online part: scores are computed on the
    chosen heads only); default all heads, in order.

    Returns l [B, R, H, ctx], R = len(rows), H = len(heads):
    l[b, c, i, j] = scale * q[b, heads[i], rows[c]] . k[b, g, j] (g the kv-head
    of heads[i]) for j <= L_b - T + rows[c], -inf for the causally hidden
    positions up to L_b, NaN beyond L_b (undefined).
    """
    q = _f64(q)
    B, Hq, T, d = q.shape
    Hkv, ctx = k.shape[1], k.shape[2]
    G = Hq // Hkv
    sc = default_scale(d) if scale is None else scale
    rows = [int(t) for t in rows]
    heads = list(range(Hq)) if heads is None else [int(h) for h in heads]
    out = np.full((B, len(rows), len(heads), ctx), np.nan)
    for b in range(B):
        L = int(seq_lens[b])
        for i, h in enumerate(heads):
            kg = _f64(k[b, h // G, :L])
            for c, t in enumerate(rows):
                row = sc * (kg @ q[b, h, t])
                row[L - T + t + 1:] = -np.inf
                out[b, c, i, :L] = row
    return out


def kvgroup_sum(logits: np.ndarray, num_kv_heads: int, heads: Optional[Sequence[int]] = None,
                num_q_heads: Optional[int] = None) -> np.ndarray:
    """Collected logits summed over the collected rows and over the collected
    q-heads of each kv-head: [B, R, H, ctx] -> [B, Hkv, ctx].  With a head
    subset, `heads` and `num_q_heads` give each logit row's head and the group
    size; a kv-head none of whose heads is collected sums to 0."""
    B, _, H, ctx = logits.shape
    if heads is None:
        heads, num_q_heads = list(range(H)), H
    G = num_q_heads // num_kv_heads
    out = np.zeros((B, num_kv_heads, ctx))
    for g in range(num_kv_heads):
        sel = [i for i, h in enumerate(heads) if h // G == g]
        if sel:
            out[:, g] = logits[:, :, sel, :].sum(axis=(1, 2))
    return out


def aggregate_scores(logits: np.ndarray) -> np.ndarray:
    """One importance score per KV position (Vegas, "A.", the summand of the
    argmax: sum over the collected draft/bonus rows and all query heads).
    Accepts per-head logits [B, R, Hq, ctx] or kv-group sums [B, Hkv, ctx]."""
    if logits.ndim == 4:
        return logits.sum(axis=(1, 2))
    return logits.sum(axis=1)


# --------------------------------------------------------------------------- selection
def select_topk(scores: np.ndarray, length: int, k: int, n_sink: int, window: int) -> np.ndarray:
    """Positions kept for the next step (Vegas, "A."; Dustin, "1. hybrid attention
    aggregation" for the protected sinks and window).

    F = [0, min(n_sink, L)) U [max(0, L - window), L) is always kept; the
    remaining k - |F| slots go to the other positions in order of descending
    score, lower position first among equal scores.  If k >= L all positions
    are kept.  Returns ascending int64 positions.
    """
    L = int(length)
    if L <= 0:
        return np.zeros(0, dtype=np.int64)
    if k >= L:
        return np.arange(L, dtype=np.int64)
    forced = np.zeros(L, dtype=bool)
    forced[:min(n_sink, L)] = True
    forced[max(0, L - window):] = True
    nf = int(forced.sum())
    if nf > k:
        raise ValueError("sinks and window exceed the budget")
    rest = np.flatnonzero(~forced)
    vals = np.asarray(scores[:L], dtype=np.float64)[rest]
    # lexsort: last key is primary -> descending score, then ascending position
    order = np.lexsort((rest, -vals))
    chosen = rest[order[:k - nf]]
    keep = forced.copy()
    keep[chosen] = True
    return np.flatnonzero(keep).astype(np.int64)


def _top_by(values: np.ndarray, candidates: np.ndarray, count: int) -> np.ndarray:
    """`count` candidates of largest value, lower position first among equals."""
    order = np.lexsort((candidates, -np.asarray(values, dtype=np.float64)[candidates]))
    return candidates[order[:count]]


def select_topk_hybrid(target: np.ndarray, draft: np.ndarray, length: int, k: int, m: int,
                       n_sink: int, window: int) -> np.ndarray:
    """Hierarchical selection from two signals (Dustin, "1. hybrid attention
    aggregation"): the sink prefix and the recent window are protected first;
    of the remaining budget r = k - |F|, min(m, r) positions go to the largest
    draft-lookahead scores, then the other r - min(m, r) to the largest
    target-historical scores among the positions still free.  Ties: lower
    position first.  If k >= L all positions are kept.  Returns ascending
    int64 positions.
    """
    L = int(length)
    if L <= 0:
        return np.zeros(0, dtype=np.int64)
    if k >= L:
        return np.arange(L, dtype=np.int64)
    forced = np.zeros(L, dtype=bool)
    forced[:min(n_sink, L)] = True
    forced[max(0, L - window):] = True
    nf = int(forced.sum())
    if nf > k:
        raise ValueError("sinks and window exceed the budget")
    r = k - nf
    m_eff = min(max(int(m), 0), r)
    free = np.flatnonzero(~forced)
    by_draft = _top_by(draft[:L], free, m_eff)
    keep = forced.copy()
    keep[by_draft] = True
    by_target = _top_by(target[:L], np.flatnonzero(~keep), r - m_eff)
    keep[by_target] = True
    return np.flatnonzero(keep).astype(np.int64)


def select_topk_hybrid_batch(target: np.ndarray, draft: np.ndarray, seq_lens: Sequence[int], k: int,
                             m: int, n_sink: int, window: int) -> List[np.ndarray]:
    return [select_topk_hybrid(target[b], draft[b], int(seq_lens[b]), k, m, n_sink, window)
            for b in range(target.shape[0])]


def block_sums(scores: np.ndarray, length: int, block: int) -> np.ndarray:
    """Score of each `block`-position block of [0, L): the sum of its members'
    scores (the last block may be partial), from the definition: the members
    widened to float64 and summed exactly (math.fsum, correctly rounded)."""
    L = int(length)
    nb = -(-L // block)
    x = np.asarray(scores[:L], dtype=np.float64)
    return np.array([math.fsum(x[i * block:min(L, (i + 1) * block)].tolist()) for i in range(nb)],
                    dtype=np.float64)


def select_blocks(scores: np.ndarray, length: int, k_blocks: int, block: int, n_sink: int,
                  window: int, sums: Optional[np.ndarray] = None) -> np.ndarray:
    """Block-granular selection (structured block sparsity, the euno.news
    summary of arXiv 2512.21911, "3. sparse verification engine"; Quest's
    page-level selection in Dustin's comparison): whole blocks of `block`
    positions are kept.  Under Vegas "A."'s summed-logit objective the best
    k_blocks blocks are those of largest block sum.  The blocks holding the
    sink prefix [0, n_sink) and the recent window [L - window, L) are kept
    first; the rest of the k_blocks go to the largest block sums, lower block
    first among equals.  If k_blocks covers every block all positions are
    kept.  Returns the kept positions ascending (every member of a kept
    block below L).

    `sums` (optional, one value per block of [0, L)) are the block sums to
    rank, compared as given: e.g. another implementation's own rounded sums,
    so that a selection made from them can be checked exactly.  Default: the
    exact sums of block_sums."""
    L = int(length)
    if L <= 0:
        return np.zeros(0, dtype=np.int64)
    nb = -(-L // block)
    if k_blocks >= nb:
        return np.arange(L, dtype=np.int64)
    forced = np.zeros(nb, dtype=bool)
    forced[:min(-(-n_sink // block), nb)] = True
    if window > 0:
        forced[max(0, L - window) // block:] = True
    nf = int(forced.sum())
    if nf > k_blocks:
        raise ValueError("sink and window blocks exceed the block budget")
    rank = block_sums(scores, L, block) if sums is None else np.asarray(sums, dtype=np.float64)[:nb]
    if rank.shape[0] != nb:
        raise ValueError("one block sum per block of [0, L) is needed")
    chosen = _top_by(rank, np.flatnonzero(~forced), k_blocks - nf)
    keep = forced.copy()
    keep[chosen] = True
    pos = np.arange(L, dtype=np.int64)
    return pos[keep[pos // block]]


def block_positions(ids: Sequence[int], block: int, length: int) -> np.ndarray:
    """The positions a list of block ids stands for (structured block
    sparsity: block i is positions [i * block, (i + 1) * block)), clipped to
    [0, length), in list order.  Returns int64 positions."""
    L = int(length)
    out = [p for i in ids for p in range(int(i) * block, min((int(i) + 1) * block, L))]
    return np.asarray(out, dtype=np.int64)


def select_blocks_batch(scores: np.ndarray, seq_lens: Sequence[int], k_blocks: int, block: int,
                        n_sink: int, window: int,
                        sums: Optional[np.ndarray] = None) -> List[np.ndarray]:
    return [select_blocks(scores[b], int(seq_lens[b]), k_blocks, block, n_sink, window,
                          None if sums is None else sums[b])
            for b in range(scores.shape[0])]


def select_topk_batch(scores: np.ndarray, seq_lens: Sequence[int], k: int, n_sink: int,
                      window: int) -> List[np.ndarray]:
    return [select_topk(scores[b], int(seq_lens[b]), k, n_sink, window)
            for b in range(scores.shape[0])]


# --------------------------------------------------------------------------- sparse
def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens: Sequence[int],
                     idx: Sequence[np.ndarray], scale: Optional[float] = None,
                     heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention restricted to the selected positions (Vegas, section 2 step 3
    and section 3: page size 1, the selected indices are the pages).

    idx[b] holds ascending absolute positions.  Row t of T' rows sees the
    listed positions j <= L'_b - T' + t, L'_b = seq_lens[b].
    """
    q = _f64(q)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = default_scale(d) if scale is None else scale
    o = np.full((B, Hq, T, v.shape[3]), np.nan)
    lse = np.full((B, Hq, T), np.nan)
    want = set(range(Hq)) if heads is None else set(heads)
    for b in range(B):
        L = int(seq_lens[b])
        pos = np.asarray(idx[b], dtype=np.int64)
        for g in range(Hkv):
            hs = [h for h in range(g * G, (g + 1) * G) if h in want]
            if not hs:
                continue
            rows = q[b, hs].reshape(-1, d)
            vis = [int(np.count_nonzero(pos <= L - T + t)) for _ in hs for t in range(T)]
            ob, lb = attend(rows, _f64(k[b, g, pos]), _f64(v[b, g, pos]), vis, sc)
            o[b, hs] = ob.reshape(len(hs), T, -1)
            lse[b, hs] = lb.reshape(len(hs), T)
    return o, lse


def _f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    return widen_bf16(x) if x.dtype == np.uint16 else x.astype(np.float64, copy=False)
