"""The C-ABI library loads, exports every declared symbol, and rejects invalid
arguments on the host before anything is launched (no GPU needed: every call
here fails validation, so no HIP call is reached)."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_attention_long_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vgsa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: each call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vgsa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from sparse_attention_long_amd import build
        build.build()
    return B.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = declared_functions()
    assert len(names) == 25
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.SIGNATURES)
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (vgsa_\w+)", out))
    assert set(names) <= exported


def test_desc_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "vgsa.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu\\n\", sizeof(vgsa_attn_desc),"
        " offsetof(vgsa_attn_desc, num_blocks), offsetof(vgsa_attn_desc, softmax_scale),"
        " sizeof(vgsa_status));return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    size, off_nb, off_scale, st = map(int, subprocess.run([str(exe)], capture_output=True, text=True).stdout.split())
    assert size == ctypes.sizeof(B.AttnDesc)
    assert off_nb == B.AttnDesc.num_blocks.offset and off_scale == B.AttnDesc.softmax_scale.offset
    assert st == 4


def test_status_strings_and_version(lib):
    assert B.status_string(0) == "ok"
    assert "invalid" in B.status_string(1)
    assert lib.vgsa_version().decode().startswith("vgsa")


ALL = B.ALL_HEADS


def desc(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, q_len=4, max_ctx=1000,
                block_size=0, max_blocks_per_seq=0, num_blocks=0, softmax_scale=0.0)
    base.update(kw)
    return B.AttnDesc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), INVALID),
    (dict(num_q_heads=0), INVALID),
    (dict(num_kv_heads=0), INVALID),
    (dict(num_q_heads=6, num_kv_heads=4), INVALID),
    (dict(head_dim=0), INVALID),
    (dict(head_dim=96), UNSUPPORTED),
    (dict(q_len=0), INVALID),
    (dict(q_len=17), UNSUPPORTED),
    (dict(num_q_heads=64, num_kv_heads=4, q_len=5), UNSUPPORTED),  # 16 * 5 rows > 64
    (dict(max_ctx=0), INVALID),
    (dict(block_size=8), UNSUPPORTED),
    (dict(block_size=-16), INVALID),
    (dict(block_size=16, max_blocks_per_seq=0, num_blocks=4), INVALID),
    (dict(block_size=16, max_blocks_per_seq=10, num_blocks=4, max_ctx=161), INVALID),
    (dict(softmax_scale=float("nan")), INVALID),
    (dict(batch=70000), UNSUPPORTED),
])
def test_bad_desc_rejected_everywhere(lib, kw, code):
    d = ctypes.byref(desc(**kw))
    assert lib.vgsa_verify_attention(d, FAKE, FAKE, FAKE, FAKE, FAKE, 9, ALL, 2, FAKE, FAKE, None,
                                     FAKE, 1 << 40, None) == code
    assert lib.vgsa_sparse_attention(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 0, FAKE, None,
                                     FAKE, 1 << 40, None) == code
    assert lib.vgsa_verify_workspace_bytes(d) == 0
    s, c = ctypes.c_int32(), ctypes.c_int32()
    assert lib.vgsa_split_plan(d, 100, ctypes.byref(s), ctypes.byref(c)) == code


def test_verify_argument_checks(lib):
    d = desc()
    dp = ctypes.byref(d)
    ws = lib.vgsa_verify_workspace_bytes(dp)
    assert ws > 0
    V = lib.vgsa_verify_attention
    # null q / cache / seq_lens / out
    assert V(dp, None, FAKE, FAKE, None, FAKE, 9, ALL, 0, None, FAKE, None, FAKE, ws, None) == INVALID
    assert V(dp, FAKE, FAKE, FAKE, None, None, 9, ALL, 0, None, FAKE, None, FAKE, ws, None) == INVALID
    assert V(dp, FAKE, FAKE, FAKE, None, FAKE, 9, ALL, 0, None, None, None, FAKE, ws, None) == INVALID
    # block table given for a contiguous cache
    assert V(dp, FAKE, FAKE, FAKE, FAKE, FAKE, 9, ALL, 0, None, FAKE, None, FAKE, ws, None) == INVALID
    # logits requested but missing; collect mask empty or naming a row >= q_len; bad layout
    assert V(dp, FAKE, FAKE, FAKE, None, FAKE, 9, ALL, 1, None, FAKE, None, FAKE, ws, None) == INVALID
    for mask in [0, 1 << 4, 0x11, 0xFFFFFFFF]:
        for lay in (1, 2):
            assert V(dp, FAKE, FAKE, FAKE, None, FAKE, mask, ALL, lay, FAKE, FAKE, None, FAKE, ws,
                     None) == INVALID
    assert V(dp, FAKE, FAKE, FAKE, None, FAKE, 9, ALL, 7, FAKE, FAKE, None, FAKE, ws, None) == INVALID
    # head mask: empty, or naming a head >= Hq; subsets need Hq <= 64
    for hm in (0, 1 << 8, 0x1FF):
        assert V(dp, FAKE, FAKE, FAKE, None, FAKE, 9, hm, 2, FAKE, FAKE, None, FAKE, ws, None) == INVALID
    d128 = desc(num_q_heads=128, num_kv_heads=32, q_len=4)
    w128 = lib.vgsa_verify_workspace_bytes(ctypes.byref(d128))
    assert V(ctypes.byref(d128), FAKE, FAKE, FAKE, None, FAKE, 9, 3, 2, FAKE, FAKE, None, FAKE, w128,
             None) == UNSUPPORTED
    # workspace missing or one byte short
    assert V(dp, FAKE, FAKE, FAKE, None, FAKE, 9, ALL, 2, FAKE, FAKE, None, None, ws, None) == WORKSPACE
    assert V(dp, FAKE, FAKE, FAKE, None, FAKE, 9, ALL, 2, FAKE, FAKE, None, FAKE, ws - 1, None) == WORKSPACE
    # misaligned q / cache / out; misaligned workspace
    ODD = ctypes.c_void_p(0x1008)
    assert V(dp, ODD, FAKE, FAKE, None, FAKE, 9, ALL, 2, FAKE, FAKE, None, FAKE, ws, None) == INVALID
    assert V(dp, FAKE, ODD, FAKE, None, FAKE, 9, ALL, 2, FAKE, FAKE, None, FAKE, ws, None) == INVALID
    assert V(dp, FAKE, FAKE, ODD, None, FAKE, 9, ALL, 2, FAKE, FAKE, None, FAKE, ws, None) == INVALID
    assert V(dp, FAKE, FAKE, FAKE, None, FAKE, 9, ALL, 2, FAKE, ODD, None, FAKE, ws, None) == INVALID
    assert V(dp, FAKE, FAKE, FAKE, None, FAKE, 9, ALL, 2, FAKE, FAKE, None, ctypes.c_void_p(0x1010),
             ws, None) == WORKSPACE
    # paged cache without a block table
    dpg = desc(block_size=16, max_blocks_per_seq=63, num_blocks=100, max_ctx=1000)
    wsp = lib.vgsa_verify_workspace_bytes(ctypes.byref(dpg))
    assert V(ctypes.byref(dpg), FAKE, FAKE, FAKE, None, FAKE, 9, ALL, 2, FAKE, FAKE, None, FAKE, wsp,
             None) == INVALID


def test_sparse_and_combine_argument_checks(lib):
    d = desc()
    dp = ctypes.byref(d)
    ws = lib.vgsa_sparse_workspace_bytes(dp, 64)
    assert ws > 0 and lib.vgsa_sparse_workspace_bytes(dp, 0) == 0
    S = lib.vgsa_sparse_attention
    assert S(dp, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 64, 0, FAKE, None, FAKE, ws, None) == INVALID
    assert S(dp, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 64, 0, FAKE, None, FAKE, ws, None) == INVALID
    assert S(dp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 0, 0, FAKE, None, FAKE, ws, None) == INVALID
    assert S(dp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 64, 0, FAKE, None, FAKE, ws - 1, None) == WORKSPACE
    assert S(dp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 64, -1, FAKE, None, FAKE, ws, None) == INVALID  # tail < 0
    C = lib.vgsa_combine_partials
    assert C(dp, 0, FAKE, FAKE, ws, FAKE, None, None) == INVALID
    F = lib.vgsa_verify_finish
    wv = lib.vgsa_verify_workspace_bytes(dp)
    assert F(dp, None, FAKE, wv, FAKE, None, 2, 2, 0, FAKE, FAKE, None) == INVALID
    assert F(dp, FAKE, FAKE, wv, None, None, 2, 2, 0, FAKE, FAKE, None) == INVALID
    assert F(dp, FAKE, FAKE, wv, FAKE, None, 0, 2, 0, FAKE, FAKE, None) == INVALID   # scores need a layout
    assert F(dp, FAKE, FAKE, wv, FAKE, None, 2, 2, 0, None, FAKE, None) == INVALID   # ... and logits
    assert F(dp, FAKE, FAKE, wv - 1, FAKE, None, 2, 2, 0, FAKE, FAKE, None) == WORKSPACE
    for nr in (0, 33):  # per-head logit rows outside 1..q_len*Hq
        assert F(dp, FAKE, FAKE, wv, FAKE, None, 1, nr, 0, FAKE, FAKE, None) == INVALID
    assert F(ctypes.byref(desc(head_dim=96)), FAKE, FAKE, wv, FAKE, None, 2, 2, 0, FAKE, FAKE, None) == UNSUPPORTED
    assert C(dp, 64, None, FAKE, ws, FAKE, None, None) == INVALID
    assert C(dp, 64, FAKE, FAKE, ws, None, None, None) == INVALID
    assert C(dp, 64, FAKE, FAKE, 256, FAKE, None, None) == WORKSPACE  # header only


def test_aggregate_and_select_argument_checks(lib):
    A = lib.vgsa_aggregate_scores
    assert A(-1, 8, 2, 100, 2, 2, 0, FAKE, FAKE, FAKE, None) == INVALID
    assert A(2, 6, 4, 100, 2, 2, 0, FAKE, FAKE, FAKE, None) == INVALID
    assert A(2, 8, 2, 0, 2, 2, 0, FAKE, FAKE, FAKE, None) == INVALID
    assert A(2, 8, 2, 100, 0, 2, 0, FAKE, FAKE, FAKE, None) == INVALID   # layout NONE has nothing to sum
    assert A(2, 8, 2, 100, 2, 2, 0, None, FAKE, FAKE, None) == INVALID
    for nr in (0, 129):  # per-head logit rows outside 1..16*Hq
        assert A(2, 8, 2, 100, 1, nr, 0, FAKE, FAKE, FAKE, None) == INVALID
    assert A(0, 8, 2, 100, 2, 2, 0, FAKE, FAKE, FAKE, None) == OK        # empty batch: nothing launched
    T = lib.vgsa_select_topk
    assert T(2, 100, FAKE, FAKE, 0, 0, 0, FAKE, 8, FAKE, None) == INVALID     # k < 1
    assert T(2, 100, FAKE, FAKE, 8, -1, 0, FAKE, 8, FAKE, None) == INVALID
    assert T(2, 100, FAKE, FAKE, 8, 4, 5, FAKE, 8, FAKE, None) == INVALID     # sinks + window > k
    assert T(2, 100, FAKE, FAKE, 8, 4, 4, FAKE, 7, FAKE, None) == INVALID     # idx_stride < k
    assert T(2, 100, None, FAKE, 8, 4, 4, FAKE, 8, FAKE, None) == INVALID
    assert T(2, 0, FAKE, FAKE, 8, 4, 4, FAKE, 8, FAKE, None) == INVALID
    assert T(0, 100, FAKE, FAKE, 8, 4, 4, FAKE, 8, FAKE, None) == OK
    H = lib.vgsa_select_topk_hybrid
    assert H(0, 100, FAKE, FAKE, FAKE, 8, 2, 2, 2, FAKE, 8, FAKE, None) == OK   # empty batch
    assert H(2, 100, FAKE, None, FAKE, 8, 2, 2, 2, FAKE, 8, FAKE, None) == INVALID  # no draft scores
    assert H(2, 100, None, FAKE, FAKE, 8, 2, 2, 2, FAKE, 8, FAKE, None) == INVALID
    assert H(2, 100, FAKE, FAKE, FAKE, 8, -1, 2, 2, FAKE, 8, FAKE, None) == INVALID   # m < 0
    assert H(2, 100, FAKE, FAKE, FAKE, 8, 2, 4, 5, FAKE, 8, FAKE, None) == INVALID    # sinks + window > k
    assert H(2, 100, FAKE, FAKE, FAKE, 8, 2, 2, 2, FAKE, 7, FAKE, None) == INVALID    # idx_stride < k
    assert H(2, 100, FAKE, FAKE, FAKE, 0, 0, 0, 0, FAKE, 8, FAKE, None) == INVALID    # k < 1
    assert H(2, 262145, FAKE, FAKE, FAKE, 8, 2, 2, 2, FAKE, 8, FAKE, None) == UNSUPPORTED
    K = lib.vgsa_select_blocks
    assert K(0, 100, FAKE, FAKE, 8, 16, 4, 16, FAKE, 128, FAKE, None, None) == OK        # empty batch
    assert K(2, 100, FAKE, FAKE, 8, 0, 4, 16, FAKE, 128, FAKE, None, None) == INVALID     # block < 1
    assert K(2, 100, FAKE, FAKE, 8, 2048, 4, 16, FAKE, 16384, FAKE, None, None) == INVALID  # block > 1024
    assert K(2, 100, FAKE, FAKE, 2, 16, 4, 16, FAKE, 128, FAKE, None, None) == INVALID    # 1 + 1 + 1 > 2
    assert K(2, 100, FAKE, FAKE, 3, 16, 4, 16, FAKE, 47, FAKE, None, None) == INVALID     # idx_stride < 48
    assert K(2, 100, None, FAKE, 8, 16, 4, 16, FAKE, 128, FAKE, None, None) == INVALID
    assert K(2, 100, FAKE, FAKE, 8, 16, -1, 16, FAKE, 128, FAKE, None, None) == INVALID
    assert K(2, 16 * 8704 + 1, FAKE, FAKE, 8, 16, 4, 16, FAKE, 128, FAKE, None, None) == UNSUPPORTED


def test_append_argument_checks(lib):
    P = lib.vgsa_append_positions
    assert P(-1, FAKE, 0, 1, FAKE, 8, FAKE, None) == INVALID
    assert P(2, FAKE, -1, 1, FAKE, 8, FAKE, None) == INVALID
    assert P(2, FAKE, 0, -1, FAKE, 8, FAKE, None) == INVALID
    assert P(2, FAKE, 0, 1, FAKE, 0, FAKE, None) == INVALID
    assert P(2, None, 0, 1, FAKE, 8, FAKE, None) == INVALID
    assert P(2, FAKE, 0, 1, FAKE, 8, None, None) == INVALID
    assert P(2, None, 0, 0, None, 8, None, None) == OK   # nothing to append: nothing launched
    assert P(0, None, 0, 3, None, 8, None, None) == OK


def test_split_plan_covers_span(lib):
    # wide layout (one 8-wavefront workgroup per CU): chunks of 256 .. 16640
    for B_, Hkv, span in [(16, 8, 32768), (1, 8, 32768), (8, 8, 131078), (4, 8, 65536), (1, 1, 5),
                          (16, 8, 512), (1, 8, 2049), (64, 8, 131088), (64, 8, 9216), (64, 8, 9217),
                          (512, 8, 1 << 20)]:
        d = desc(batch=B_, num_kv_heads=Hkv, num_q_heads=Hkv, q_len=1, max_ctx=span)
        s, c = B.split_plan(d, span)
        assert s >= 1 and c % 256 == 0 and c <= 16640 and s * c >= span and (s - 1) * c < span
    # narrow layout (d = 128 with four 16-row blocks): chunks of 128 .. 9216
    for B_, span in [(16, 32768), (1, 32768), (8, 131078), (64, 131088), (2, 5000)]:
        d = desc(batch=B_, num_kv_heads=8, num_q_heads=64, q_len=8, max_ctx=span)
        s, c = B.split_plan(d, span)
        assert s >= 1 and c % 128 == 0 and c <= 9216 and s * c >= span and (s - 1) * c < span
    # one round of 256 wide workgroups (one per CU) at the 32K x b16 shape ...
    d = desc(batch=16, num_q_heads=64, num_kv_heads=8, q_len=5, max_ctx=32768)
    assert B.split_plan(d, 32768) == (2, 16384)
    # ... of 512 narrow ones (two per CU) with four row blocks
    d = desc(batch=16, num_q_heads=64, num_kv_heads=8, q_len=8, max_ctx=32768)
    assert B.split_plan(d, 32768) == (4, 8192)
    # chunks are capped at 16384 positions ...
    d = desc(batch=1, num_q_heads=8, num_kv_heads=1, q_len=2, head_dim=64, max_ctx=1 << 24)
    assert B.split_plan(d, 1 << 24) == (1024, 16384)
    d = desc(batch=8, num_q_heads=32, num_kv_heads=8, q_len=7, max_ctx=145000)
    assert B.split_plan(d, 145000) == (9, 16384)
    # ... except that a last sliver of at most 256 positions (one step of
    # every wavefront) is spread over the other splits (chunks of 16640)
    for span in (131078, 131088, 131072 + 256):
        d = desc(batch=8, num_q_heads=32, num_kv_heads=8, q_len=7, max_ctx=span)
        assert B.split_plan(d, span) == (8, 16640)
    d = desc(batch=8, num_q_heads=32, num_kv_heads=8, q_len=7, max_ctx=131072 + 257)
    assert B.split_plan(d, 131072 + 257) == (9, 16384)
    d = desc(batch=2, num_q_heads=8, num_kv_heads=1, q_len=2, max_ctx=2 * 8192 + 100)
    assert B.split_plan(d, 2 * 8192 + 100) == (65, 256)   # not capped: no widening
    # narrow: slivers up to 1024 positions are spread (chunks of at most 9216)
    d = desc(batch=8, num_q_heads=64, num_kv_heads=8, q_len=8, max_ctx=131088)
    assert B.split_plan(d, 131088) == (16, 8320)


def test_select_workspace_sizes_and_validation(lib):
    """The per-round selection needs a workspace only for capacities of 49153 ..
    262144 positions; a missing or small workspace is refused before any launch."""
    ws = lib.vgsa_select_workspace_bytes
    assert ws(4, 32768) == 0 and ws(4, 1000) == 0 and ws(4, 262145) == 0 and ws(0, 65536) == 0
    assert ws(4, 32772) == 0 and ws(4, 49152) == 0  # up to 1.5 rounds: one workgroup per row
    w2, w8 = ws(4, 49153), ws(4, 262144)
    assert 0 < w2 < w8 and w2 % 256 == 0 and w8 % 256 == 0
    assert ws(8, 131072) > ws(4, 131072)
    fake = ctypes.c_void_p(0x1000)
    # missing workspace -> VGSA_ERR_WORKSPACE (3); bad arguments -> VGSA_ERR_INVALID_ARG (1)
    assert lib.vgsa_select_topk_ws(4, 131072, fake, fake, 512, 4, 64, fake, 512, fake,
                                   None, 0, None) == 3
    assert lib.vgsa_select_topk_ws(4, 131072, fake, fake, 512, 4, 64, fake, 512, fake,
                                   fake, w2 - 1, None) == 3
    assert lib.vgsa_select_topk_ws(4, 131072, fake, fake, 512, 400, 200, fake, 512, fake,
                                   fake, ws(4, 131072), None) == 1
    assert lib.vgsa_select_topk_ws(4, 131072, fake, fake, 512, 4, 64, fake, 100, fake,
                                   fake, ws(4, 131072), None) == 1
    # the hybrid form takes the same workspace
    assert lib.vgsa_select_topk_hybrid_ws(4, 131072, fake, fake, fake, 512, 100, 4, 64, fake, 512,
                                          fake, None, 0, None) == 3
    assert lib.vgsa_select_topk_hybrid_ws(4, 131072, fake, None, fake, 512, 100, 4, 64, fake, 512,
                                          fake, fake, ws(4, 131072), None) == 1


def test_finish_select_argument_checks(lib):
    """vgsa_verify_finish_select validates as vgsa_verify_finish plus
    vgsa_select_topk, refuses rows past 262144 positions, and checks its
    selection workspace; all before any launch."""
    d = desc()
    dp = ctypes.byref(d)
    ws = lib.vgsa_verify_workspace_bytes(dp)
    sws = lib.vgsa_finish_select_workspace_bytes(2, d.max_ctx)
    pieces = -(-d.max_ctx // 4096)
    assert sws >= 2 * 4096 * 4 + 2 * 4 + 2 * pieces * (4 + 4096 * 8) and sws % 256 == 0
    assert lib.vgsa_finish_select_workspace_bytes(0, d.max_ctx) == 0
    assert lib.vgsa_finish_select_workspace_bytes(2, 0) == 0
    assert lib.vgsa_finish_select_workspace_bytes(2, 262145) == 0
    F = lib.vgsa_verify_finish_select

    def call(**kw):
        a = dict(d=dp, lens=FAKE, ws=FAKE, ws_bytes=ws, out=FAKE, lse=None, layout=2, rows=0, acc=0,
                 logits=FAKE, scores=FAKE, k=64, sink=4, window=16, idx=FAKE, stride=64, n_idx=FAKE,
                 sws=FAKE, sws_bytes=sws)
        a.update(kw)
        return F(a["d"], a["lens"], a["ws"], a["ws_bytes"], a["out"], a["lse"], a["layout"],
                 a["rows"], a["acc"], a["logits"], a["scores"], a["k"], a["sink"], a["window"],
                 a["idx"], a["stride"], a["n_idx"], a["sws"], a["sws_bytes"], None)

    assert call(scores=None) == INVALID      # the scores are required
    assert call(logits=None) == INVALID
    assert call(layout=0) == INVALID         # no logits layout
    assert call(k=0) == INVALID
    assert call(sink=50, window=20) == INVALID  # forced positions exceed the budget
    assert call(stride=63) == INVALID
    assert call(idx=None) == INVALID
    assert call(n_idx=None) == INVALID
    assert call(lens=None) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(ws_bytes=ws - 1) == WORKSPACE
    assert call(sws=None) == WORKSPACE
    assert call(sws_bytes=sws - 1) == WORKSPACE
    assert call(sws=ctypes.c_void_p(0x1010)) == WORKSPACE
    big = desc(max_ctx=262145)
    assert F(ctypes.byref(big), FAKE, FAKE, lib.vgsa_verify_workspace_bytes(ctypes.byref(big)), FAKE,
             None, 2, 0, 0, FAKE, FAKE, 64, 4, 16, FAKE, 64, FAKE, FAKE, sws, None) == UNSUPPORTED
    bad = desc(head_dim=96)
    assert F(ctypes.byref(bad), FAKE, FAKE, 1 << 40, FAKE, None, 2, 0, 0, FAKE, FAKE, 64, 4, 16, FAKE,
             64, FAKE, FAKE, sws, None) == UNSUPPORTED


def test_block_list_argument_checks(lib):
    """vgsa_select_block_ids validates as vgsa_select_blocks but needs only
    k_blocks entries per row; vgsa_sparse_attention_blocks refuses a block
    outside 1 .. 1024 and checks its workspace against ids_stride * block +
    tail entries."""
    S = lib.vgsa_select_block_ids
    assert S(2, 1000, FAKE, FAKE, 8, 16, 4, 16, FAKE, 7, FAKE, None, None) == INVALID   # stride < k
    assert S(2, 1000, FAKE, FAKE, 8, 0, 4, 16, FAKE, 8, FAKE, None, None) == INVALID    # block 0
    assert S(2, 1000, FAKE, FAKE, 8, 1025, 4, 16, FAKE, 8, FAKE, None, None) == INVALID
    assert S(2, 1000, FAKE, FAKE, 2, 16, 4, 40, FAKE, 8, FAKE, None, None) == INVALID   # forced > k
    assert S(2, 1000, None, FAKE, 8, 16, 4, 16, FAKE, 8, FAKE, None, None) == INVALID
    assert S(2, 1 << 20, FAKE, FAKE, 8, 16, 4, 16, FAKE, 8, FAKE, None, None) == UNSUPPORTED
    assert S(0, 1000, FAKE, FAKE, 8, 16, 4, 16, FAKE, 8, FAKE, None, None) == OK      # nothing to do
    d = desc()
    dp = ctypes.byref(d)
    SA = lib.vgsa_sparse_attention_blocks
    ws = lib.vgsa_sparse_workspace_bytes(dp, 8 * 16 + 3)
    assert SA(dp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 8, 0, 3, FAKE, None, FAKE, ws, None) == INVALID
    assert SA(dp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 8, 1025, 3, FAKE, None, FAKE, ws,
              None) == INVALID
    assert SA(dp, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 8, 16, 3, FAKE, None, FAKE, ws,
              None) == INVALID
    assert SA(dp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 8, 16, -1, FAKE, None, FAKE, ws,
              None) == INVALID
    assert SA(dp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 8, 16, 3, None, None, FAKE, ws,
              None) == INVALID
    assert SA(dp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 8, 16, 3, FAKE, None, FAKE, ws - 1,
              None) == WORKSPACE
    assert SA(dp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 22, 1024, 3, FAKE, None, FAKE,
              1 << 40, None) == UNSUPPORTED  # ids_stride * block past int32


def test_binding_refuses_accumulate_without_scores():
    """aggregate_scores(accumulate=True) needs the scores to add to: the
    binding raises before allocating anything or calling the library."""
    import torch
    with pytest.raises(ValueError, match="accumulate"):
        B.aggregate_scores(torch.zeros(1, 8, 16), torch.zeros(1, dtype=torch.int32), 8, 8,
                           accumulate=True)


def test_noalloc_verify_rejects_requests_beyond_its_scratch(lib):
    """vgsa_verify_attention_noalloc refuses, before any HIP call, a desc whose
    split partials exceed the static scratch, and reports an invalid desc as
    the workspace form does."""
    scratch = lib.vgsa_noalloc_scratch_bytes()
    assert scratch == 64 << 20
    N = lib.vgsa_verify_attention_noalloc
    # batch 64 x 64 q-heads x 5 rows at 32K: 4 x the headline's partials
    big = B.AttnDesc(64, 64, 8, 128, 5, 32768, 0, 0, 0, 0.0)
    assert lib.vgsa_verify_workspace_bytes(ctypes.byref(big)) > scratch
    assert N(ctypes.byref(big), FAKE, FAKE, FAKE, None, FAKE, 17, B.ALL_HEADS, 2, FAKE, FAKE, FAKE,
             None) == 5
    assert B.status_string(5) == "request exceeds the library's static scratch"
    bad = B.AttnDesc(2, 6, 4, 128, 5, 1000, 0, 0, 0, 0.0)   # Hq not a multiple of Hkv
    assert N(ctypes.byref(bad), FAKE, FAKE, FAKE, None, FAKE, 17, B.ALL_HEADS, 2, FAKE, FAKE, FAKE,
             None) == INVALID
    odd = B.AttnDesc(2, 8, 4, 96, 5, 1000, 0, 0, 0, 0.0)    # head_dim 96
    assert N(ctypes.byref(odd), FAKE, FAKE, FAKE, None, FAKE, 17, B.ALL_HEADS, 2, FAKE, FAKE, FAKE,
             None) == UNSUPPORTED
