"""Thin Python binding of libvgsa.so (the C ABI declared in include/vgsa.h).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is not built, or no GPU is
visible, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvgsa.so")

LOGITS_NONE, LOGITS_PER_HEAD, LOGITS_KVGROUP_SUM = 0, 1, 2
_LAYOUTS = {"none": LOGITS_NONE, "per_head": LOGITS_PER_HEAD, "kvgroup_sum": LOGITS_KVGROUP_SUM}

c_i32, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
c_u32, c_u64 = ctypes.c_uint32, ctypes.c_uint64
ALL_HEADS = (1 << 64) - 1
P_i32 = ctypes.POINTER(ctypes.c_int32)


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32), ("num_q_heads", c_i32), ("num_kv_heads", c_i32), ("head_dim", c_i32),
        ("q_len", c_i32), ("max_ctx", c_i32), ("block_size", c_i32),
        ("max_blocks_per_seq", c_i32), ("num_blocks", c_i32), ("softmax_scale", c_f32),
    ]


# name -> (restype, argtypes); every symbol the header declares
SIGNATURES = {
    "vgsa_status_string": (ctypes.c_char_p, [c_i32]),
    "vgsa_version": (ctypes.c_char_p, []),
    "vgsa_split_plan": (c_i32, [ctypes.POINTER(AttnDesc), c_i32, P_i32, P_i32]),
    "vgsa_verify_workspace_bytes": (c_sz, [ctypes.POINTER(AttnDesc)]),
    "vgsa_sparse_workspace_bytes": (c_sz, [ctypes.POINTER(AttnDesc), c_i32]),
    "vgsa_verify_attention": (c_i32, [ctypes.POINTER(AttnDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_u32,
                                      c_u64, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "vgsa_aggregate_scores": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp,
                                      c_vp, c_vp]),
    "vgsa_select_topk": (c_i32, [c_i32, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_i32,
                                 c_vp, c_vp]),
    "vgsa_select_workspace_bytes": (c_sz, [c_i32, c_i32]),
    "vgsa_select_topk_ws": (c_i32, [c_i32, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_i32,
                                    c_vp, c_vp, c_sz, c_vp]),
    "vgsa_select_topk_hybrid": (c_i32, [c_i32, c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                        c_vp, c_i32, c_vp, c_vp]),
    "vgsa_select_topk_hybrid_ws": (c_i32, [c_i32, c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32,
                                           c_i32, c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]),
    "vgsa_select_blocks": (c_i32, [c_i32, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_i32,
                                   c_vp, c_vp, c_vp]),
    "vgsa_sparse_attention": (c_i32, [ctypes.POINTER(AttnDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                      c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "vgsa_select_block_ids": (c_i32, [c_i32, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp,
                                      c_i32, c_vp, c_vp, c_vp]),
    "vgsa_sparse_attention_blocks": (c_i32, [ctypes.POINTER(AttnDesc), c_vp, c_vp, c_vp, c_vp, c_vp,
                                             c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                                             c_sz, c_vp]),
    "vgsa_verify_partials": (c_i32, [ctypes.POINTER(AttnDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_u32,
                                     c_u64, c_i32, c_vp, c_vp, c_sz, c_vp]),
    "vgsa_sparse_partials": (c_i32, [ctypes.POINTER(AttnDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                     c_vp, c_i32, c_vp, c_sz, c_vp]),
    "vgsa_combine_partials": (c_i32, [ctypes.POINTER(AttnDesc), c_i32, c_vp, c_vp, c_sz, c_vp,
                                      c_vp, c_vp]),
    "vgsa_verify_finish": (c_i32, [ctypes.POINTER(AttnDesc), c_vp, c_vp, c_sz, c_vp, c_vp, c_i32,
                                   c_i32, c_i32, c_vp, c_vp, c_vp]),
    "vgsa_finish_select_workspace_bytes": (c_sz, [c_i32, c_i32]),
    "vgsa_verify_finish_select": (c_i32, [ctypes.POINTER(AttnDesc), c_vp, c_vp, c_sz, c_vp, c_vp,
                                          c_i32, c_i32, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32,
                                          c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]),
    "vgsa_append_positions": (c_i32, [c_i32, c_vp, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp]),
    "vgsa_noalloc_scratch_bytes": (c_sz, []),
    "vgsa_verify_attention_noalloc": (c_i32, [ctypes.POINTER(AttnDesc), c_vp, c_vp, c_vp, c_vp,
                                              c_vp, c_u32, c_u64, c_i32, c_vp, c_vp, c_vp, c_vp]),
}

_lib: Optional[ctypes.CDLL] = None


class VgsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (no compute happens here)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sparse_attention_long_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().vgsa_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise VgsaError(status, where)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: Optional[int] = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_desc(q: torch.Tensor, k_cache: torch.Tensor, block_table: Optional[torch.Tensor] = None,
              max_ctx: Optional[int] = None, scale: float = 0.0) -> AttnDesc:
    """Describe an attention call from the tensors' shapes.
    Contiguous cache: k_cache [B, Hkv, max_ctx, d].  Paged: k_cache
    [num_blocks, Hkv, 16, d] with block_table [B, max_blocks]."""
    B, Hq, T, d = q.shape
    if block_table is None:
        _, Hkv, cap, _ = k_cache.shape
        return AttnDesc(B, Hq, Hkv, d, T, cap if max_ctx is None else max_ctx, 0, 0, 0, scale)
    nb, Hkv, bs, _ = k_cache.shape
    mb = block_table.shape[1]
    return AttnDesc(B, Hq, Hkv, d, T, 16 * mb if max_ctx is None else max_ctx, bs, mb, nb, scale)


def split_plan(desc: AttnDesc, span: int) -> Tuple[int, int]:
    s, c = c_i32(0), c_i32(0)
    _check(load().vgsa_split_plan(ctypes.byref(desc), span, ctypes.byref(s), ctypes.byref(c)),
           "vgsa_split_plan")
    return s.value, c.value


def verify_workspace_bytes(desc: AttnDesc) -> int:
    return int(load().vgsa_verify_workspace_bytes(ctypes.byref(desc)))


def sparse_workspace_bytes(desc: AttnDesc, idx_stride: int) -> int:
    return int(load().vgsa_sparse_workspace_bytes(ctypes.byref(desc), idx_stride))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is None:
        # zero-filled: the one-call sparse path keeps self-resetting counters in it
        return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)
    _need(workspace, "workspace", torch.uint8)
    return workspace


def _check_attn(q, k_cache, v_cache, seq_lens, block_table):
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if q.shape[3] != k_cache.shape[3]:
        raise ValueError("head_dim of q and the cache differ")
    if seq_lens.shape[0] != q.shape[0]:
        raise ValueError("seq_lens must have one entry per sequence")
    if block_table is not None:
        _need(block_table, "block_table", torch.int32, 2)
        if block_table.shape[0] != q.shape[0]:
            raise ValueError("block_table must have one row per sequence")
    elif k_cache.shape[0] != q.shape[0]:
        raise ValueError("contiguous cache must have one row per sequence")


# --------------------------------------------------------------------------- entry points
def row_mask(rows: Sequence[int], q_len: int) -> int:
    """Collect mask from row indices: bit t set collects row t.  Rows must be
    distinct, ascending and below q_len (the logits are stored in row order)."""
    rows = [int(r) for r in rows]
    if not rows or any(r < 0 or r >= q_len for r in rows) or sorted(set(rows)) != rows:
        raise ValueError(f"collect rows {rows} must be distinct, ascending and in [0, {q_len})")
    m = 0
    for r in rows:
        m |= 1 << r
    return m


def head_mask(heads: Optional[Sequence[int]], num_q_heads: int) -> int:
    """Head mask from head indices (None: every head).  Heads must be
    distinct, ascending and below num_q_heads."""
    if heads is None:
        return ALL_HEADS
    heads = [int(h) for h in heads]
    if not heads or any(h < 0 or h >= num_q_heads or h >= 64 for h in heads) or \
            sorted(set(heads)) != heads:
        raise ValueError(f"heads {heads} must be distinct, ascending and in [0, {min(num_q_heads, 64)})")
    m = 0
    for h in heads:
        m |= 1 << h
    return m


def verify_attention(q, k_cache, v_cache, seq_lens, *, block_table=None, max_ctx=None,
                     collect_rows: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None,
                     layout: str = "kvgroup_sum", logits=None, out=None, lse=None, workspace=None,
                     scale: float = 0.0):
    """vgsa_verify_attention.  Returns (out bf16 [B,Hq,T,d], lse fp32 [B,Hq,T], logits);
    per-head logits are [B, R, H, max_ctx] for R collected rows and H collected heads."""
    _check_attn(q, k_cache, v_cache, seq_lens, block_table)
    desc = make_desc(q, k_cache, block_table, max_ctx, scale)
    lay = _LAYOUTS[layout]
    B, Hq, T, d = q.shape
    dev = q.device
    mask = row_mask((0, T - 1) if collect_rows is None else collect_rows, T)
    hmask = head_mask(heads, Hq)
    if lay != LOGITS_NONE and logits is None:
        R = bin(mask).count("1")
        H = Hq if heads is None else len(heads)
        shape = (B, R, H, desc.max_ctx) if lay == LOGITS_PER_HEAD else (B, desc.num_kv_heads, desc.max_ctx)
        logits = torch.empty(shape, dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((B, Hq, T, d), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws = _workspace(verify_workspace_bytes(desc), dev, workspace)
    _check(load().vgsa_verify_attention(
        ctypes.byref(desc), _p(q), _p(k_cache), _p(v_cache), _p(block_table), _p(seq_lens), mask,
        hmask, lay, _p(logits) if lay != LOGITS_NONE else None, _p(out), _p(lse), _p(ws), ws.numel(),
        _stream(dev)), "vgsa_verify_attention")
    return out, lse, logits


def verify_attention_noalloc(q, k_cache, v_cache, seq_lens, out, lse, logits=None, *,
                             block_table=None, max_ctx=None,
                             collect_rows: Optional[Sequence[int]] = None,
                             heads: Optional[Sequence[int]] = None, layout: str = "kvgroup_sum",
                             scale: float = 0.0):
    """vgsa_verify_attention_noalloc: vgsa_verify_attention with the library's
    static scratch as the workspace.  The caller passes every output (out,
    lse, and logits unless layout is "none"); nothing is allocated here or in
    the library."""
    _check_attn(q, k_cache, v_cache, seq_lens, block_table)
    desc = make_desc(q, k_cache, block_table, max_ctx, scale)
    lay = _LAYOUTS[layout]
    T = q.shape[2]
    mask = row_mask((0, T - 1) if collect_rows is None else collect_rows, T)
    if lay != LOGITS_NONE and logits is None:
        raise ValueError("logits must be given unless layout is 'none'")
    _check(load().vgsa_verify_attention_noalloc(
        ctypes.byref(desc), _p(q), _p(k_cache), _p(v_cache), _p(block_table), _p(seq_lens), mask,
        head_mask(heads, q.shape[1]), lay, _p(logits) if lay != LOGITS_NONE else None, _p(out),
        _p(lse), _stream(q.device)), "vgsa_verify_attention_noalloc")
    return out, lse, logits


def noalloc_scratch_bytes() -> int:
    return int(load().vgsa_noalloc_scratch_bytes())


def aggregate_scores(logits, seq_lens, num_q_heads: int, num_kv_heads: int, *,
                     layout: str = "kvgroup_sum", scores=None, accumulate: bool = False):
    """vgsa_aggregate_scores.  Returns scores fp32 [B, max_ctx] (added to
    `scores` when accumulating); per-head logits are [B, R, H, max_ctx]."""
    if accumulate and scores is None:
        raise ValueError("accumulate needs the scores to add to")
    _need(logits, "logits", torch.float32)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    lay = _LAYOUTS[layout]
    B, max_ctx = logits.shape[0], logits.shape[-1]
    n_rows = logits.shape[1] * logits.shape[2] if lay == LOGITS_PER_HEAD and logits.dim() == 4 else 0
    if scores is None:
        scores = torch.empty((B, max_ctx), dtype=torch.float32, device=logits.device)
    _check(load().vgsa_aggregate_scores(B, num_q_heads, num_kv_heads, max_ctx, lay, n_rows,
                                        int(bool(accumulate)), _p(logits),
                                        _p(seq_lens), _p(scores), _stream(logits.device)),
           "vgsa_aggregate_scores")
    return scores


def select_workspace_bytes(batch: int, max_ctx: int) -> int:
    return int(load().vgsa_select_workspace_bytes(batch, max_ctx))


def select_topk(scores, seq_lens, k: int, n_sink: int, window: int, *, idx_stride=None,
                idx=None, n_idx=None, workspace=None):
    """vgsa_select_topk_ws (vgsa_select_topk when the row needs no workspace).
    Returns (idx int32 [B, idx_stride], n_idx int32 [B])."""
    _need(scores, "scores", torch.float32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, max_ctx = scores.shape
    stride = k if idx_stride is None else idx_stride
    if idx is None:
        idx = torch.empty((B, stride), dtype=torch.int32, device=scores.device)
    if n_idx is None:
        n_idx = torch.empty((B,), dtype=torch.int32, device=scores.device)
    nbytes = select_workspace_bytes(B, max_ctx) if B > 0 else 0
    if nbytes and workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=scores.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    _check(load().vgsa_select_topk_ws(B, max_ctx, _p(scores), _p(seq_lens), k, n_sink, window,
                                      _p(idx), idx.shape[1], _p(n_idx), _p(workspace),
                                      0 if workspace is None else workspace.numel(),
                                      _stream(scores.device)),
           "vgsa_select_topk_ws")
    return idx, n_idx


def select_topk_hybrid(target_scores, draft_scores, seq_lens, k: int, m: int, n_sink: int,
                       window: int, *, idx_stride=None, idx=None, n_idx=None, workspace=None):
    """vgsa_select_topk_hybrid_ws (vgsa_select_topk_hybrid when the row needs no
    workspace).  Returns (idx int32 [B, idx_stride], n_idx int32 [B])."""
    _need(target_scores, "target_scores", torch.float32, 2)
    _need(draft_scores, "draft_scores", torch.float32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if draft_scores.shape != target_scores.shape:
        raise ValueError("draft_scores must have the shape of target_scores")
    B, max_ctx = target_scores.shape
    stride = k if idx_stride is None else idx_stride
    if idx is None:
        idx = torch.empty((B, stride), dtype=torch.int32, device=target_scores.device)
    if n_idx is None:
        n_idx = torch.empty((B,), dtype=torch.int32, device=target_scores.device)
    nbytes = select_workspace_bytes(B, max_ctx) if B > 0 else 0
    if nbytes and workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=target_scores.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    _check(load().vgsa_select_topk_hybrid_ws(
        B, max_ctx, _p(target_scores), _p(draft_scores), _p(seq_lens), k, m, n_sink, window,
        _p(idx), idx.shape[1], _p(n_idx), _p(workspace),
        0 if workspace is None else workspace.numel(), _stream(target_scores.device)),
        "vgsa_select_topk_hybrid_ws")
    return idx, n_idx


def select_blocks(scores, seq_lens, k_blocks: int, block: int, n_sink: int, window: int, *,
                  idx_stride=None, idx=None, n_idx=None, block_sums=None):
    """vgsa_select_blocks.  Returns (idx int32 [B, idx_stride] positions of the
    kept blocks, n_idx int32 [B]).  `block_sums` (fp32 [B, ceil(max_ctx /
    block)], optional) receives the block sums the ranking compared."""
    _need(scores, "scores", torch.float32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, max_ctx = scores.shape
    stride = k_blocks * block if idx_stride is None else idx_stride
    if idx is None:
        idx = torch.empty((B, stride), dtype=torch.int32, device=scores.device)
    if n_idx is None:
        n_idx = torch.empty((B,), dtype=torch.int32, device=scores.device)
    if block_sums is not None:
        _need(block_sums, "block_sums", torch.float32, 2)
        if tuple(block_sums.shape) != (B, -(-max_ctx // block)):
            raise ValueError(f"block_sums must be [{B}, {-(-max_ctx // block)}]")
    _check(load().vgsa_select_blocks(B, max_ctx, _p(scores), _p(seq_lens), k_blocks, block, n_sink,
                                     window, _p(idx), idx.shape[1], _p(n_idx), _p(block_sums),
                                     _stream(scores.device)), "vgsa_select_blocks")
    return idx, n_idx


def select_block_ids(scores, seq_lens, k_blocks: int, block: int, n_sink: int, window: int, *,
                     ids_stride=None, ids=None, n_ids=None, block_sums=None):
    """vgsa_select_block_ids.  Returns (ids int32 [B, ids_stride] kept block
    ids ascending, n_ids int32 [B])."""
    _need(scores, "scores", torch.float32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, max_ctx = scores.shape
    stride = k_blocks if ids_stride is None else ids_stride
    if ids is None:
        ids = torch.empty((B, stride), dtype=torch.int32, device=scores.device)
    if n_ids is None:
        n_ids = torch.empty((B,), dtype=torch.int32, device=scores.device)
    if block_sums is not None:
        _need(block_sums, "block_sums", torch.float32, 2)
        if tuple(block_sums.shape) != (B, -(-max_ctx // block)):
            raise ValueError(f"block_sums must be [{B}, {-(-max_ctx // block)}]")
    _check(load().vgsa_select_block_ids(B, max_ctx, _p(scores), _p(seq_lens), k_blocks, block,
                                        n_sink, window, _p(ids), ids.shape[1], _p(n_ids),
                                        _p(block_sums), _stream(scores.device)),
           "vgsa_select_block_ids")
    return ids, n_ids


def sparse_attention_blocks(q, k_cache, v_cache, seq_lens, ids, n_ids, block: int, *,
                            block_table=None, max_ctx=None, tail: int = 0, out=None, lse=None,
                            workspace=None, scale: float = 0.0):
    """vgsa_sparse_attention_blocks: sparse attention over whole blocks of
    `block` positions (ids ascending).  Returns (out, lse) as sparse_attention."""
    _check_attn(q, k_cache, v_cache, seq_lens, block_table)
    _need(ids, "ids", torch.int32, 2)
    _need(n_ids, "n_ids", torch.int32, 1)
    desc = make_desc(q, k_cache, block_table, max_ctx, scale)
    B, Hq, T, d = q.shape
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, T, d), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws = _workspace(sparse_workspace_bytes(desc, ids.shape[1] * block + tail), dev, workspace)
    _check(load().vgsa_sparse_attention_blocks(
        ctypes.byref(desc), _p(q), _p(k_cache), _p(v_cache), _p(block_table), _p(seq_lens), _p(ids),
        _p(n_ids), ids.shape[1], block, tail, _p(out), _p(lse), _p(ws), ws.numel(), _stream(dev)),
        "vgsa_sparse_attention_blocks")
    return out, lse


def sparse_attention(q, k_cache, v_cache, seq_lens, idx, n_idx, *, block_table=None, max_ctx=None,
                     tail: int = 0, out=None, lse=None, workspace=None, scale: float = 0.0):
    """vgsa_sparse_attention.  Returns (out bf16 [B,Hq,T',d], lse fp32 [B,Hq,T']).
    `tail`: the last `tail` positions below each length are attended after the list."""
    _check_attn(q, k_cache, v_cache, seq_lens, block_table)
    _need(idx, "idx", torch.int32, 2)
    _need(n_idx, "n_idx", torch.int32, 1)
    desc = make_desc(q, k_cache, block_table, max_ctx, scale)
    B, Hq, T, d = q.shape
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, T, d), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws = _workspace(sparse_workspace_bytes(desc, idx.shape[1] + tail), dev, workspace)
    _check(load().vgsa_sparse_attention(
        ctypes.byref(desc), _p(q), _p(k_cache), _p(v_cache), _p(block_table), _p(seq_lens), _p(idx),
        _p(n_idx), idx.shape[1], tail, _p(out), _p(lse), _p(ws), ws.numel(), _stream(dev)),
        "vgsa_sparse_attention")
    return out, lse


def append_positions(base, first: int, count: int, idx, n_idx) -> None:
    """vgsa_append_positions: idx[b][n_idx[b] + i] = base[b] + first + i for
    i < count, n_idx[b] += count (in place)."""
    _need(base, "base", torch.int32, 1)
    _need(idx, "idx", torch.int32, 2)
    _need(n_idx, "n_idx", torch.int32, 1)
    _check(load().vgsa_append_positions(idx.shape[0], _p(base), first, count, _p(idx), idx.shape[1],
                                        _p(n_idx), _stream(idx.device)), "vgsa_append_positions")


# --------------------------------------------------------------------------- two-phase form
def verify_partials(desc: AttnDesc, q, k_cache, v_cache, seq_lens, block_table, rows, layout: int,
                    logits, workspace, heads: Optional[Sequence[int]] = None) -> None:
    """vgsa_verify_partials; `rows` / `heads` are the collected row and head
    indices (ascending; heads None: every head)."""
    _check(load().vgsa_verify_partials(
        ctypes.byref(desc), _p(q), _p(k_cache), _p(v_cache), _p(block_table), _p(seq_lens),
        row_mask(rows, desc.q_len), head_mask(heads, desc.num_q_heads), layout, _p(logits) if layout != LOGITS_NONE else None, _p(workspace),
        workspace.numel(), _stream(q.device)), "vgsa_verify_partials")


def sparse_partials(desc: AttnDesc, q, k_cache, v_cache, seq_lens, block_table, idx, n_idx,
                    workspace) -> None:
    _check(load().vgsa_sparse_partials(
        ctypes.byref(desc), _p(q), _p(k_cache), _p(v_cache), _p(block_table), _p(seq_lens), _p(idx),
        _p(n_idx), idx.shape[1], _p(workspace), workspace.numel(), _stream(q.device)),
        "vgsa_sparse_partials")


def combine_partials(desc: AttnDesc, span: int, lengths, workspace, out, lse) -> None:
    _check(load().vgsa_combine_partials(
        ctypes.byref(desc), span, _p(lengths), _p(workspace), workspace.numel(), _p(out), _p(lse),
        _stream(out.device)), "vgsa_combine_partials")


def verify_finish(desc: AttnDesc, seq_lens, workspace, out, lse, layout: int = LOGITS_NONE,
                  logits=None, scores=None, accumulate: bool = False) -> None:
    """vgsa_verify_finish: combine the verify partials and (with `scores`)
    aggregate the collected logits, in one launch (added to `scores` when
    accumulating).  Per-head logits are [B, R, H, max_ctx]."""
    num_rows = 0
    if layout == LOGITS_PER_HEAD and logits is not None and logits.dim() == 4:
        num_rows = logits.shape[1] * logits.shape[2]
    _check(load().vgsa_verify_finish(
        ctypes.byref(desc), _p(seq_lens), _p(workspace), workspace.numel(), _p(out), _p(lse),
        layout, num_rows, int(bool(accumulate)), _p(logits), _p(scores), _stream(out.device)), "vgsa_verify_finish")


def finish_select_workspace_bytes(batch: int, max_ctx: int) -> int:
    return int(load().vgsa_finish_select_workspace_bytes(batch, max_ctx))


def verify_finish_select(desc: AttnDesc, seq_lens, workspace, out, lse, layout: int, logits,
                         scores, k: int, n_sink: int, window: int, idx, n_idx, select_workspace,
                         accumulate: bool = False) -> None:
    """vgsa_verify_finish_select: verify_finish (with scores) and the top-k
    selection on those scores in one launch.  `select_workspace` (uint8,
    finish_select_workspace_bytes(B, max_ctx) bytes) must be zero before its
    first use; every call leaves it ready for the next.  Per-head logits are
    [B, R, H, max_ctx]."""
    _need(idx, "idx", torch.int32, 2)
    _need(n_idx, "n_idx", torch.int32, 1)
    _need(select_workspace, "select_workspace", torch.uint8)
    num_rows = 0
    if layout == LOGITS_PER_HEAD and logits is not None and logits.dim() == 4:
        num_rows = logits.shape[1] * logits.shape[2]
    _check(load().vgsa_verify_finish_select(
        ctypes.byref(desc), _p(seq_lens), _p(workspace), workspace.numel(), _p(out), _p(lse),
        layout, num_rows, int(bool(accumulate)), _p(logits), _p(scores), k, n_sink, window,
        _p(idx), idx.shape[1], _p(n_idx), _p(select_workspace), select_workspace.numel(),
        _stream(out.device)), "vgsa_verify_finish_select")
