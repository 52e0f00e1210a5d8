"""Seeded synthetic workloads for verification-guided sparse attention.

This module only builds inputs: shapes, seeded bf16 tensors, planted salient
keys, ragged lengths and paged block tables.  It holds none of the method's
arithmetic (no attention, no logits, no selection), so that both the fp64
oracle and the GPU path can be fed from it without sharing any computation.

Shapes follow the problem statement of the pages:
  * Vegas (gist.science 2602.07223), section 2 "core mechanism": the verify
    pass runs over the gamma draft tokens plus the bonus token, i.e.
    T = gamma + 1 query rows per sequence, against the whole KV cache.
  * Vegas section 3 "implementation": the KV cache is addressed through
    pages (a paged pool with a block table is the PagedAttention layout).
  * Dustin (gist.science 2606.24957), "experiments": batch 16 at 32K context
    is the shape of the headline self-attention measurement.

Input recipe (the same for every workload):
  * Q, K and V are i.i.d. N(0, 1) in float32, drawn from numpy's PCG64 with a
    seed tuple (seed, layer, b, g, tensor-tag) per (sequence, kv-head) slice,
    then rounded to bfloat16 with round-to-nearest-even.  A slice can
    therefore be regenerated on its own, bit-identically.
  * "Planted" salient keys stand in for the few key KV entries that real
    attention concentrates on (Vegas section 1).  For each sequence a set of
    positions is drawn from [n_sink, L - window) without replacement, shared
    by all kv-heads.  At a planted position j of kv-head g the key is
    replaced by 4 * ||k_j|| * u, where u is the unit vector along the sum of
    the group's query rows (the heads that share g, all T rows), and the
    result is rounded to bfloat16.
  * Ragged lengths are integers drawn uniformly from an inclusive range.
  * Paged caches use 16-position blocks; physical block ids are one seeded
    random permutation, shared by all layers.
  * Draft-lookahead scores (the second signal of hybrid selection; the draft
    model that would produce them is not part of this path) are i.i.d.
    N(0, 1) float32 per position below the length, with the planted
    positions raised by 8 (the draft also attends the salient entries), and 0
    past the length.  The draft share m is half of the budget left after the
    sinks and the window.

bf16 tensors are returned as uint16 numpy arrays holding the raw bits.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

TAG_Q, TAG_K, TAG_V, TAG_QDRAFT, TAG_PLANT, TAG_LEN, TAG_BLOCKS, TAG_DRAFTSC = 1, 2, 3, 4, 5, 6, 7, 8
PAGE_BLOCK = 16


@dataclass(frozen=True)
class Workload:
    """One synthetic per-layer decode workload."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    ctx: Optional[int]                    # fixed context length L (incl. the T verify tokens)
    gamma: int                            # draft tokens; T = gamma + 1 verify rows
    budget: int                           # k, number of selected positions
    n_sink: int
    window: int
    planted: Optional[int] = None         # fixed planted count per sequence ...
    planted_frac: Optional[float] = None  # ... or a fraction of L (rounded)
    draft_steps: int = 0                  # sparse steps of one query each after selection
    sparse_verify: bool = True            # sparse attention over the same T rows
    ctx_range: Optional[Tuple[int, int]] = None  # ragged: inclusive uniform range
    paged: bool = False
    layers: int = 1
    seed: int = 1
    lens: Optional[Tuple[int, ...]] = None       # explicit per-sequence lengths (tests)
    cap_align: int = 16                          # row capacity rounded up to this many positions

    # ---- derived sizes ----
    @property
    def q_len(self) -> int:
        return self.gamma + 1

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def collect_rows(self) -> Tuple[int, int]:
        # first draft token's row and the bonus token's row (Vegas, "Collect-2-Query")
        return (0, self.gamma)

    @property
    def draft_m(self) -> int:
        # hybrid selection: positions picked by the draft signal (half the free budget)
        return max(0, self.budget - self.n_sink - self.window) // 2

    def max_len(self) -> int:
        if self.lens is not None:
            return max(self.lens)
        if self.ctx is not None:
            return self.ctx
        return self.ctx_range[1]

    def max_ctx(self) -> int:
        """Row capacity: the longest context plus headroom for draft-step tokens,
        rounded up to whole 16-position blocks for paged caches, and to
        `cap_align` positions otherwise (16: fp32 logit and score rows start
        64-byte aligned, so they are read and written as 16-byte vectors)."""
        cap = self.max_len() + self.draft_steps
        align = PAGE_BLOCK if self.paged else max(1, self.cap_align)
        return -(-cap // align) * align

    def planted_count(self, length: int) -> int:
        if self.planted is not None:
            return self.planted
        if self.planted_frac is not None:
            return int(round(self.planted_frac * length))
        return 0


# The five workloads, named by what they are.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("ctx2k_b1_h32kv8_d128", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 ctx=2048, gamma=3, budget=256, n_sink=4, window=64, planted=8,
                 draft_steps=1, sparse_verify=True, seed=1001),
        Workload("ctx32k_b1_h32kv8_d128_draft4", batch=1, num_q_heads=32, num_kv_heads=8,
                 head_dim=128, ctx=32768, gamma=4, budget=2048, n_sink=4, window=128,
                 planted_frac=0.01, draft_steps=4, sparse_verify=False, seed=1002),
        Workload("ctx32k_b16_h64kv8_d128", batch=16, num_q_heads=64, num_kv_heads=8,
                 head_dim=128, ctx=32768, gamma=4, budget=512, n_sink=4, window=64,
                 planted_frac=0.01, draft_steps=0, sparse_verify=True, seed=1003),
        Workload("ctx128k_b8_h32kv8_d128_draft6", batch=8, num_q_heads=32, num_kv_heads=8,
                 head_dim=128, ctx=131072, gamma=6, budget=6554, n_sink=4, window=256,
                 planted_frac=0.005, draft_steps=6, sparse_verify=False, seed=1004),
        Workload("ragged8k-64k_b4_h64kv8_d64_paged16_l24", batch=4, num_q_heads=64,
                 num_kv_heads=8, head_dim=64, ctx=None, ctx_range=(8192, 65536), gamma=5,
                 budget=1024, n_sink=4, window=128, planted_frac=0.01, draft_steps=0,
                 sparse_verify=True, paged=True, layers=24, seed=1005),
    ]
}

# The workload the throughput figure is quoted on: batch 16, 32K context.
HEADLINE = "ctx32k_b16_h64kv8_d128"


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits.
    Inputs here are finite, so no NaN special case is needed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(w: Workload, layer: int, b: int, g: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([w.seed, layer, b, g, tag])


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(int(np.prod(shape)), dtype=np.float32)).reshape(shape)


# ---------------------------------------------------------------- lengths
def seq_lens(w: Workload) -> np.ndarray:
    """Verify-time context length per sequence (it counts the T verify tokens)."""
    if w.lens is not None:
        return np.asarray(w.lens, dtype=np.int32)
    if w.ctx is not None:
        return np.full(w.batch, w.ctx, dtype=np.int32)
    lo, hi = w.ctx_range
    rng = _rng(w, 0, 0, 0, TAG_LEN)
    return rng.integers(lo, hi + 1, size=w.batch, dtype=np.int64).astype(np.int32)


def planted_positions(w: Workload, layer: int, b: int, length: int) -> np.ndarray:
    n = w.planted_count(length)
    lo, hi = w.n_sink, length - w.window
    if n <= 0 or hi <= lo:
        return np.zeros(0, dtype=np.int64)
    n = min(n, hi - lo)
    rng = _rng(w, layer, b, 0, TAG_PLANT)
    return np.sort(rng.choice(np.arange(lo, hi), size=n, replace=False))


# ---------------------------------------------------------------- per-slice generation
def q_group(w: Workload, layer: int, b: int, g: int) -> np.ndarray:
    """Verify query rows of the heads of kv-head g: uint16 [G, T, d]."""
    return _normal_bf16(_rng(w, layer, b, g, TAG_Q), (w.group, w.q_len, w.head_dim))


def q_draft_group(w: Workload, layer: int, b: int, g: int) -> np.ndarray:
    """One fresh query per draft step for the heads of kv-head g: uint16 [steps, G, d]."""
    return _normal_bf16(_rng(w, layer, b, g, TAG_QDRAFT), (w.draft_steps, w.group, w.head_dim))


def kv_slice(w: Workload, layer: int, b: int, g: int, length: int,
             qg: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Logical K and V rows of (sequence b, kv-head g): uint16 [max_ctx, d] each.
    Rows at and beyond `length + draft_steps` are zero (never read)."""
    cap, d = w.max_ctx(), w.head_dim
    n = min(cap, length + w.draft_steps)
    k = np.zeros((cap, d), dtype=np.uint16)
    v = np.zeros((cap, d), dtype=np.uint16)
    k[:n] = _normal_bf16(_rng(w, layer, b, g, TAG_K), (n, d))
    v[:n] = _normal_bf16(_rng(w, layer, b, g, TAG_V), (n, d))
    pos = planted_positions(w, layer, b, length)
    if pos.size:
        if qg is None:
            qg = q_group(w, layer, b, g)
        u = bf16_bits_to_f32(qg).astype(np.float64).reshape(-1, d).sum(axis=0)
        u /= np.linalg.norm(u)
        kj = bf16_bits_to_f32(k[pos]).astype(np.float64)
        norms = np.linalg.norm(kj, axis=1, keepdims=True)
        k[pos] = f32_to_bf16_bits((4.0 * norms * u[None, :]).astype(np.float32))
    return k, v


@dataclass
class LayerInputs:
    """Host-side inputs of one layer.  bf16 tensors are uint16 bit arrays."""

    workload: Workload
    layer: int
    seq_lens: np.ndarray                  # int32 [B]
    q: np.ndarray                         # [B, Hq, T, d]
    k: np.ndarray                         # logical [B, Hkv, max_ctx, d]
    v: np.ndarray                         # logical [B, Hkv, max_ctx, d]
    q_draft: Optional[np.ndarray]         # [steps, B, Hq, 1, d] or None
    planted: List[np.ndarray] = field(default_factory=list)
    # paged layout (only when workload.paged)
    k_pool: Optional[np.ndarray] = None   # [num_blocks, Hkv, 16, d]
    v_pool: Optional[np.ndarray] = None
    block_table: Optional[np.ndarray] = None  # int32 [B, max_blocks]


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_layer(w: Workload, layer: int = 0, batches: Optional[List[int]] = None) -> LayerInputs:
    """Generate every tensor of one layer (only sequences in `batches`, others zero)."""
    B, Hq, Hkv, G, T, d = w.batch, w.num_q_heads, w.num_kv_heads, w.group, w.q_len, w.head_dim
    cap = w.max_ctx()
    lens = seq_lens(w)
    bsel = list(range(B)) if batches is None else list(batches)
    q = np.zeros((B, Hq, T, d), dtype=np.uint16)
    k = np.zeros((B, Hkv, cap, d), dtype=np.uint16)
    v = np.zeros((B, Hkv, cap, d), dtype=np.uint16)
    qd = np.zeros((w.draft_steps, B, Hq, 1, d), dtype=np.uint16) if w.draft_steps else None

    def fill(bg):
        b, g = bg
        qg = q_group(w, layer, b, g)
        q[b, g * G:(g + 1) * G] = qg
        kk, vv = kv_slice(w, layer, b, g, int(lens[b]), qg)
        k[b, g] = kk
        v[b, g] = vv
        if qd is not None:
            qd[:, b, g * G:(g + 1) * G, 0, :] = q_draft_group(w, layer, b, g)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, [(b, g) for b in bsel for g in range(Hkv)]))
    planted = [planted_positions(w, layer, b, int(lens[b])) for b in range(B)]
    out = LayerInputs(w, layer, lens, q, k, v, qd, planted)
    if w.paged:
        out.block_table, need = block_table(w)
        out.k_pool = to_paged(k, out.block_table, need)
        out.v_pool = to_paged(v, out.block_table, need)
    return out


# ---------------------------------------------------------------- paged layout
def block_table(w: Workload) -> Tuple[np.ndarray, List[int]]:
    """int32 [B, max_blocks] table of physical block ids.  Each sequence owns
    ceil((L_b + steps) / 16) blocks; ids are one seeded permutation of all of
    them (shared by every layer).  Unused entries hold 0."""
    lens = seq_lens(w)
    cap_blocks = w.max_ctx() // PAGE_BLOCK
    need = [-(-(int(L) + w.draft_steps) // PAGE_BLOCK) for L in lens]
    total = int(sum(need))
    perm = _rng(w, 0, 0, 0, TAG_BLOCKS).permutation(total).astype(np.int32)
    table = np.zeros((w.batch, cap_blocks), dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, need


def to_paged(logical: np.ndarray, table: np.ndarray, need: List[int]) -> np.ndarray:
    """Scatter logical [B, Hkv, cap, d] rows into a pool [num_blocks, Hkv, 16, d];
    sequence b owns the first need[b] entries of its table row."""
    B, Hkv, cap, d = logical.shape
    pool = np.zeros((int(sum(need)), Hkv, PAGE_BLOCK, d), dtype=logical.dtype)
    for b in range(B):
        for i in range(need[b]):
            pool[int(table[b, i])] = logical[b, :, i * PAGE_BLOCK:(i + 1) * PAGE_BLOCK, :]
    return pool


def draft_scores(w: Workload, layer: int = 0) -> np.ndarray:
    """Synthetic draft-lookahead scores: float32 [B, max_ctx] (recipe in the
    module docstring)."""
    lens = seq_lens(w)
    out = np.zeros((w.batch, w.max_ctx()), dtype=np.float32)
    for b, L in enumerate(lens):
        L = int(L)
        out[b, :L] = _rng(w, layer, b, 0, TAG_DRAFTSC).standard_normal(L, dtype=np.float32)
        pos = planted_positions(w, layer, b, L)
        out[b, pos] += np.float32(8.0)
    return out


def small(name: str = "small", **kw) -> Workload:
    """A custom workload for tests; defaults span several tiles with a ragged tail."""
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx=301, gamma=3,
                budget=48, n_sink=4, window=16, planted=4, draft_steps=0,
                sparse_verify=True, seed=7)
    base.update(kw)
    return Workload(name, **base)


def index_lists(seed: int, lens, count: int, stride: int) -> Tuple[np.ndarray, np.ndarray]:
    """Seeded ascending index lists: for each sequence, min(count, L) distinct
    positions drawn uniformly from [0, L), padded to `stride` with zeros.
    Returns (idx int32 [B, stride], n_idx int32 [B])."""
    rng = np.random.default_rng([seed, TAG_PLANT, 99])
    B = len(lens)
    idx = np.zeros((B, stride), dtype=np.int32)
    n = np.zeros(B, dtype=np.int32)
    for b, L in enumerate(lens):
        m = min(count, int(L), stride)
        pos = np.sort(rng.choice(int(L), size=m, replace=False)) if m > 0 else np.zeros(0, np.int64)
        idx[b, :m] = pos
        n[b] = m
    return idx, n
