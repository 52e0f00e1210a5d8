#!/usr/bin/env python3
"""Throughput of one per-layer decode iteration of verification-guided sparse
attention on one MI355X.

A step is the whole hot path over one batch of synthetic, HBM-resident input:
  verify (split-KV attention of the T = gamma+1 rows + kv-group-summed
  pre-softmax logits of the first-draft and bonus rows) -> combine ->
  aggregate scores -> top-k select (sinks + window kept) -> sparse attention
  over the selected positions (sparse verify over the T rows, and/or
  single-query draft steps) -> combine.

Prints one JSON line.  `value` is iterations per second; `roofline` is the
verify kernel (the dominant one) against the 8 TB/s HBM peak, timed with HIP
events on the stream it runs on; `cpu_baseline` is the fp64 oracle on a
bounded sample of the same workload on this host's cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--layers N]
                    [--logits kvgroup_sum|per_head] [--collect two|all]
                    [--select plain|hybrid|blocks]

--layers N runs N layers per step, each with its own queries and cache (the
ragged paged workload defines 24); `value` stays iterations/s per layer.

The defaults are the kv-group-summed layout and the two Collect-2-Query rows;
the JSON also reports the verify kernel with every row collected and the
hybrid (draft signal first) selection on the same scores.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify+topk+sparse-attn iters/s per layer at 32K, b16; % of HBM peak BW"
HBM_PEAK_GBS = 8000.0
OVERHEAD_ROUNDS = 6  # alternating rounds of the logit-overhead measurement
# K/V smaller than this rotate through copies (twice the 256 MB Infinity Cache)
ROTATE_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(w, lens, layout="kvgroup_sum", n_rows=2, n_heads=None, k_sel=None):
    """Algorithmic HBM bytes of one iteration, by stage (what the method must
    move: every K/V row read once, the collected logits written once, scores
    and indices once; split partials are implementation overhead and excluded).
    Logits are one fp32 per (kv-head, position), or per (collected row,
    collected q-head, position) in the per-head layout."""
    B, Hq, Hkv, d, T = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.q_len
    k = w.budget if k_sel is None else k_sel
    Ls = [int(L) for L in lens]
    kv = sum(Hkv * L * d * 2 * 2 for L in Ls)
    q_in = B * Hq * T * d * 2
    o_out = B * Hq * T * d * 2
    per_pos = Hkv if layout == "kvgroup_sum" else n_rows * (Hq if n_heads is None else n_heads)
    emit = sum(per_pos * L * 4 for L in Ls)
    agg = emit + sum(L * 4 for L in Ls)
    sel = sum(L * 4 for L in Ls) + B * k * 4
    n_sel = [min(k, L) for L in Ls]
    sparse = 0
    if w.sparse_verify:
        sparse += sum(Hkv * n * d * 2 * 2 for n in n_sel) + q_in + o_out + B * k * 4
    for s in range(1, w.draft_steps + 1):
        sparse += sum(Hkv * (n + s) * d * 2 * 2 for n in n_sel) + 2 * (B * Hq * d * 2) + B * k * 4
    return {
        "verify_kernel": kv + q_in + emit,  # the split-KV kernel: K, V, Q read; logits written
        "verify": kv + q_in + o_out + emit,
        "aggregate": agg,
        "select": sel,
        "sparse": sparse,
        "iteration": kv + q_in + o_out + emit + agg + sel + sparse,
        "sparse_kernel_kv": sum(Hkv * n * d * 2 * 2 for n in n_sel) + q_in if w.sparse_verify else 0,
    }


def counter_traffic(workload_name):
    """HBM bytes per verify launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy kernel), or None when the
    kernel source has changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"verify_{workload_name}.md")
    src = os.path.join(ROOT, "sparse_attention_long_amd", "csrc", "attention.hip")
    try:
        text = open(path).read()
        m = re.search(r"traffic_bytes=(\d+) source_sha256_prefix=([0-9a-f]+)", text)
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if not m or not digest.startswith(m.group(2)):
        return None
    return int(m.group(1))


def host_cpu():
    """Model name and usable core count of this host."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        nproc = os.cpu_count() or 1
    return model, nproc


def cpu_baseline(w, x, seconds, rows, heads=None, gpu_idx=None):
    """The fp64 oracle, as it stands, on whole sequences of the workload until
    `seconds` have passed; scaled to iterations/s of the full batch.

    Also reports, for the sequences it ran, how many of the positions the GPU
    selected from its fp32 scores the oracle selects from its fp64 scores
    (informational: the parity bar compares selections on the same scores)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    model, nproc = host_cpu()
    t0 = time.perf_counter()
    done = 0
    overlap = []
    for b in range(w.batch):
        sl = slice(b, b + 1)
        lens = x.seq_lens[sl]
        oracle.verify_attention(x.q[sl], x.k[sl], x.v[sl], lens)
        lg = oracle.collected_logits(x.q[sl], x.k[sl], lens, rows, heads=heads)
        sc = oracle.aggregate_scores(oracle.kvgroup_sum(lg, w.num_kv_heads, heads=heads,
                                                        num_q_heads=w.num_q_heads))
        idx = oracle.select_topk(sc[0], int(lens[0]), w.budget, w.n_sink, w.window)
        if gpu_idx is not None:
            g_idx, g_n = gpu_idx
            mine = set(g_idx[b, :g_n[b]].tolist())
            overlap.append(len(mine & set(idx.tolist())) / max(1, len(idx)))
        if w.sparse_verify:
            oracle.sparse_attention(x.q[sl], x.k[sl], x.v[sl], lens, [idx])
        for s in range(1, w.draft_steps + 1):
            li = np.concatenate([idx, np.arange(int(lens[0]), int(lens[0]) + s)])
            oracle.sparse_attention(x.q_draft[s - 1][sl], x.k[sl], x.v[sl], lens + s, [li])
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    per_seq = el / done
    out = {
        "value": 1.0 / (per_seq * w.batch),
        "unit": "iters/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{done} of {w.batch} sequences (full iteration each: verify, logits, scores, "
                  f"select, sparse) in {el:.1f} s, fp64 numpy; value scaled to the whole batch",
        "cpu_model": model,
        "nproc": int(nproc),
        "threading": f"matrix products on {blas_threads} BLAS threads; the per-row softmax, "
                     "sums, sort and gathers single-threaded numpy",
    }
    if overlap:
        out["selection_overlap_vs_fp64_scores"] = {
            "sequences": len(overlap), "mean": float(np.mean(overlap)), "min": float(np.min(overlap)),
            "note": "fraction of the oracle's fp64-score selection that the GPU's fp32-score "
                    "selection also keeps (layer 0)"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--logits", choices=("kvgroup_sum", "per_head"), default="kvgroup_sum",
                    help="layout of the collected logits")
    ap.add_argument("--collect", choices=("two", "all"), default="two",
                    help="collected verify rows: first draft + bonus (Collect-2-Query), or every row")
    ap.add_argument("--score-heads", type=int, default=0,
                    help="score on this many q-heads only, spread evenly (0: every head)")
    ap.add_argument("--select", choices=("plain", "hybrid", "blocks"), default="plain",
                    help="top-k by the verify scores; hybrid: top-m by a draft-lookahead score "
                         "first (synthetic draft scores); blocks: whole 16-position blocks")
    ap.add_argument("--finish-select", choices=("fused", "separate"), default="fused",
                    help="plain selection on rows of up to 65536 positions: the finish and the "
                         "selection in one launch (fused) or two")
    ap.add_argument("--layers", type=int, default=1,
                    help="a step runs this many layers in turn, each with its own cache and queries "
                         "(up to the workload's layer count); value stays iterations/s per layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", type=int, default=0,
                    help="1: capture one step as a HIP graph and time its replays")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain fp32 copy of this many MiB three times (a kernel of "
                         "known traffic, for scaling HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(sequences shard across GPUs with no exchange; run one process per GPU).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_attention_long_amd import binding as Bn
    from sparse_attention_long_amd import workloads as W

    name = args.workload or W.HEADLINE
    w = W.WORKLOADS[name]
    n_layers = args.layers
    if not 1 <= n_layers <= w.layers:
        print(f"--layers must be 1..{w.layers} for {name}", file=sys.stderr)
        sys.exit(2)
    if n_layers > 1 and args.graph:
        print("--graph captures one layer's step; use it with --layers 1", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    Bn.load()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x {args.copy_calibration_mib} MiB read + written")
        del src, dst

    log(f"[bench] generating {name}")
    t0 = time.perf_counter()
    x = W.make_layer(w, 0)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f}s")

    def d_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q = d_bf16(x.q)
    if w.paged:
        k, v = d_bf16(x.k_pool), d_bf16(x.v_pool)
        bt = torch.from_numpy(x.block_table).to(dev)
    else:
        k, v, bt = d_bf16(x.k), d_bf16(x.v), None
    q_layers = [q]
    if n_layers > 1:
        # layers 1 .. n-1: their own queries and caches (the block table and
        # lengths are shared by all layers)
        k_copies, v_copies = [k], [v]
        for layer in range(1, n_layers):
            xl = W.make_layer(w, layer)
            q_layers.append(d_bf16(xl.q))
            k_copies.append(d_bf16(xl.k_pool if w.paged else xl.k))
            v_copies.append(d_bf16(xl.v_pool if w.paged else xl.v))
            del xl
        log(f"[bench] {n_layers} layers generated in {time.perf_counter() - t0:.1f}s")
        n_copies = n_layers
    else:
        # Cold caches: K/V below 512 MiB would stay in the 256 MB Infinity
        # Cache from one launch to the next, so such workloads rotate through
        # copies of K/V (same values, other addresses) whose sizes add up to at
        # least 512 MiB; every launch that reads K/V takes the next copy.
        kv_bytes = (k.numel() + v.numel()) * 2
        n_copies = 1 if kv_bytes >= ROTATE_BYTES else min(64, -(-ROTATE_BYTES // kv_bytes))
        k_copies, v_copies = [k], [v]
        for _ in range(n_copies - 1):
            k_copies.append(k.clone())
            v_copies.append(v.clone())
    cur = [0]

    def kv():
        """The current K/V copy."""
        return k_copies[cur[0]], v_copies[cur[0]]

    def rotate():
        cur[0] = (cur[0] + 1) % n_copies
    lens = torch.from_numpy(x.seq_lens).to(dev)
    B, Hq, Hkv, T, d = w.batch, w.num_q_heads, w.num_kv_heads, w.q_len, w.head_dim
    max_ctx = w.max_ctx()
    desc = Bn.make_desc(q, k, bt, max_ctx)
    ws_v = torch.empty(Bn.verify_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    rows = w.collect_rows if args.collect == "two" else tuple(range(T))
    # a head subset (online scoring on chosen heads): n heads spread evenly
    heads = None
    if 0 < args.score_heads < Hq:
        heads = tuple(i * Hq // args.score_heads for i in range(args.score_heads))
    n_heads = Hq if heads is None else len(heads)
    KV = Bn.LOGITS_KVGROUP_SUM if args.logits == "kvgroup_sum" else Bn.LOGITS_PER_HEAD
    lshape = (B, Hkv, max_ctx) if KV == Bn.LOGITS_KVGROUP_SUM else (B, len(rows), n_heads, max_ctx)
    logits = torch.empty(lshape, dtype=torch.float32, device=dev)
    out = torch.empty((B, Hq, T, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    scores = torch.empty((B, max_ctx), dtype=torch.float32, device=dev)
    # block selection: ceil(k / 16) whole 16-position blocks
    BLK = 16
    k_blocks = -(-w.budget // BLK)
    stride = k_blocks * BLK if args.select == "blocks" else w.budget
    idx = torch.empty((B, stride), dtype=torch.int32, device=dev)
    n_idx = torch.empty((B,), dtype=torch.int32, device=dev)
    # block mode: the kept blocks' ids (the gathers expand them themselves)
    blocks = args.select == "blocks"
    blk_ids = torch.empty((B, k_blocks), dtype=torch.int32, device=dev)
    n_ids = torch.empty((B,), dtype=torch.int32, device=dev)
    ws_s = torch.zeros(Bn.sparse_workspace_bytes(desc, stride), dtype=torch.uint8, device=dev)
    out_s = torch.empty_like(out)
    lse_s = torch.empty_like(lse)
    # draft steps: step s attends with one fresh query per head over the
    # selected positions plus the s positions drafted since (lengths L + s)
    n_draft = w.draft_steps
    q_draft = [d_bf16(x.q_draft[s]) for s in range(n_draft)]
    lens_draft = [(lens + s).contiguous() for s in range(1, n_draft + 1)]
    if n_draft:
        desc_d = Bn.make_desc(q_draft[0], k, bt, max_ctx)
        ws_d = torch.zeros(Bn.sparse_workspace_bytes(desc_d, stride + n_draft), dtype=torch.uint8,
                           device=dev)
        out_d = torch.empty((B, Hq, 1, d), dtype=torch.bfloat16, device=dev)
        lse_d = torch.empty((B, Hq, 1), dtype=torch.float32, device=dev)

    def draft_steps(k, v):
        # step s attends the kept positions and the s + 1 drafted since (the
        # trailing positions of its length), in one launch
        for s in range(n_draft):
            if blocks:
                Bn.sparse_attention_blocks(q_draft[s], k, v, lens_draft[s], blk_ids, n_ids, BLK,
                                           block_table=bt, max_ctx=max_ctx, tail=s + 1, out=out_d,
                                           lse=lse_d, workspace=ws_d)
            else:
                Bn.sparse_attention(q_draft[s], k, v, lens_draft[s], idx, n_idx, block_table=bt,
                                    max_ctx=max_ctx, tail=s + 1, out=out_d, lse=lse_d, workspace=ws_d)

    draft_sc = torch.from_numpy(W.draft_scores(w)).to(dev)
    # rows of several 32768-position rounds: selection spread over one workgroup per round
    n_ws_sel = Bn.select_workspace_bytes(B, max_ctx)
    ws_sel = torch.empty(n_ws_sel, dtype=torch.uint8, device=dev) if n_ws_sel else None

    # plain selection on rows of up to 65536 positions: finish (combine +
    # aggregate) and selection in one launch.  Longer rows keep the separate
    # launches: one workgroup per 32768-position round selects them faster
    # than the one selecting workgroup of the fused launch (128K x b8: 41 us
    # against 52 us)
    fused = args.select == "plain" and max_ctx <= 65536 and args.finish_select == "fused"
    ws_fs = torch.zeros(Bn.finish_select_workspace_bytes(B, max_ctx), dtype=torch.uint8, device=dev) \
        if fused else None

    def finish_select():
        Bn.verify_finish_select(desc, lens, ws_v, out, lse, KV, logits, scores, w.budget, w.n_sink,
                                w.window, idx, n_idx, ws_fs)

    def select():
        if args.select == "hybrid":
            Bn.select_topk_hybrid(scores, draft_sc, lens, w.budget, w.draft_m, w.n_sink, w.window,
                                  idx=idx, n_idx=n_idx, workspace=ws_sel)
        elif blocks:
            Bn.select_block_ids(scores, lens, k_blocks, BLK, w.n_sink, w.window, ids=blk_ids,
                                n_ids=n_ids)
        else:
            Bn.select_topk(scores, lens, w.budget, w.n_sink, w.window, idx=idx, n_idx=n_idx,
                           workspace=ws_sel)

    def layer_step(ql, k, v):
        Bn.verify_partials(desc, ql, k, v, lens, bt, rows, KV, logits, ws_v, heads=heads)
        if fused:
            finish_select()
        else:
            # split combine + score aggregation in one launch, then the selection
            Bn.verify_finish(desc, lens, ws_v, out, lse, KV, logits, scores)
            select()
        if w.sparse_verify:
            sparse_pass(ql, k, v)
        draft_steps(k, v)

    def sparse_pass(ql, k, v):
        if blocks:
            Bn.sparse_attention_blocks(ql, k, v, lens, blk_ids, n_ids, BLK, block_table=bt,
                                       max_ctx=max_ctx, out=out_s, lse=lse_s, workspace=ws_s)
        else:
            Bn.sparse_attention(ql, k, v, lens, idx, n_idx, block_table=bt, max_ctx=max_ctx,
                                out=out_s, lse=lse_s, workspace=ws_s)

    def step():
        if n_layers > 1:
            # every layer in turn, each on its own cache
            for layer in range(n_layers):
                layer_step(q_layers[layer], k_copies[layer], v_copies[layer])
            return
        rotate()
        layer_step(q, *kv())

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    graphs = None
    if args.graph:
        # one step captured as a HIP graph per K/V copy (no memsets are
        # recorded: every kernel writes its outputs); replays run the same
        # kernels
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        for _ in range(n_copies):
            g_ = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                with torch.cuda.graph(g_, stream=cap):
                    step()
            graphs.append(g_)
        torch.cuda.current_stream().wait_stream(cap)
        for i in range(args.warmup):
            graphs[i % n_copies].replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, launched back to back.  No event
    # is recorded inside it: an event record drains the queue (about 6 us of
    # idle GPU), which would slow the very steps being timed.
    K = args.steps
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {K} steps")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e_start.record()
    if graphs is None:
        for _ in range(K):
            step()
    else:
        for i in range(K):
            graphs[i % n_copies].replay()
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_ms = e_start.elapsed_time(e_end)
    log(f"[bench] {K} steps: wall {wall * 1e3:.2f} ms, gpu {gpu_ms:.2f} ms")

    # ---- stage breakdown and logit-emit overhead (outside the timed region):
    # each stage launched K times back to back between one pair of events, so
    # the figure is its pipelined per-launch time (no queue drain per launch)
    def per_launch_us(fn, n=None):
        n = K if n is None else n
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            rotate()  # the next K/V copy (the launches below read it through kv())
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    # the verify kernel's launch duration for the roofline: K launches of the
    # timed configuration back to back on the launch stream
    verify_us = per_launch_us(
        lambda: Bn.verify_partials(desc, q, *kv(), lens, bt, rows, KV, logits, ws_v, heads=heads))
    log(f"[bench] verify kernel {verify_us:.1f} us per launch")
    # the finish and the selection as separate launches (the step's form when
    # they are not fused)
    finish_us = per_launch_us(lambda: Bn.verify_finish(desc, lens, ws_v, out, lse, KV, logits, scores))
    select_us = per_launch_us(select)
    stages = {"verify_partials": verify_us}
    if fused:
        stages["finish_select"] = per_launch_us(finish_select)
    else:
        stages["combine_aggregate"] = finish_us
        stages["select"] = select_us
    if w.sparse_verify:
        stages["sparse"] = per_launch_us(lambda: sparse_pass(q, *kv()))
    if n_draft:
        stages["draft_steps"] = per_launch_us(lambda: draft_steps(*kv()))
    # Logit-collection overhead: the collecting kernel (the step's rows, and
    # every verify row: the score summed over all T rows, same layout) against
    # the same kernel with collection off, in alternating rounds, medians over
    # the rounds.  One back-to-back sample of each drifts by a few per cent
    # over a run: as much as the overhead itself at the short ragged workload.
    all_rows = tuple(range(T))
    logits_all = logits
    if KV == Bn.LOGITS_PER_HEAD and len(rows) != T:
        logits_all = torch.empty((B, T, n_heads, max_ctx), dtype=torch.float32, device=dev)
    ovh_fns = {
        "none": lambda: Bn.verify_partials(desc, q, *kv(), lens, bt, rows, Bn.LOGITS_NONE, None, ws_v),
        "rows": lambda: Bn.verify_partials(desc, q, *kv(), lens, bt, rows, KV, logits, ws_v,
                                           heads=heads),
        "all": lambda: Bn.verify_partials(desc, q, *kv(), lens, bt, all_rows, KV, logits_all, ws_v,
                                          heads=heads),
    }
    ovh_samples = {key: [] for key in ovh_fns}
    for _ in range(OVERHEAD_ROUNDS):
        for key, fn in ovh_fns.items():
            ovh_samples[key].append(per_launch_us(fn, max(4, K // 2)))
    ovh = {key: statistics.median(v_) for key, v_ in ovh_samples.items()}
    verify_none_us, verify_all_us = ovh["none"], ovh["all"]
    del logits_all
    # hybrid selection (draft signal first) on the same scores, for comparison
    select_hybrid_us = per_launch_us(
        lambda: Bn.select_topk_hybrid(scores, draft_sc, lens, w.budget, w.draft_m, w.n_sink,
                                      w.window, idx=idx, n_idx=n_idx, workspace=ws_sel))
    # block selection on the same scores, and the sparse pass over its lists
    idx_b = torch.empty((B, k_blocks * BLK), dtype=torch.int32, device=dev)
    n_b = torch.empty((B,), dtype=torch.int32, device=dev)
    select_blocks_us = per_launch_us(
        lambda: Bn.select_blocks(scores, lens, k_blocks, BLK, w.n_sink, w.window, idx=idx_b, n_idx=n_b))
    # ... and as block ids, with the gather over the block lists
    ids_b = torch.empty((B, k_blocks), dtype=torch.int32, device=dev)
    nid_b = torch.empty((B,), dtype=torch.int32, device=dev)
    select_block_ids_us = per_launch_us(
        lambda: Bn.select_block_ids(scores, lens, k_blocks, BLK, w.n_sink, w.window, ids=ids_b,
                                    n_ids=nid_b))
    sparse_blocks_us = sparse_block_ids_us = None
    if w.sparse_verify:
        ws_b = torch.zeros(Bn.sparse_workspace_bytes(desc, k_blocks * BLK), dtype=torch.uint8, device=dev)
        sparse_blocks_us = per_launch_us(
            lambda: Bn.sparse_attention(q, *kv(), lens, idx_b, n_b, block_table=bt, max_ctx=max_ctx,
                                        out=out_s, lse=lse_s, workspace=ws_b))
        sparse_block_ids_us = per_launch_us(
            lambda: Bn.sparse_attention_blocks(q, *kv(), lens, ids_b, nid_b, BLK, block_table=bt,
                                               max_ctx=max_ctx, out=out_s, lse=lse_s, workspace=ws_b))

    ab = alg_bytes(w, x.seq_lens, args.logits, len(rows), n_heads,
                   k_blocks * BLK if args.select == "blocks" else None)
    iters = K * n_layers / wall  # iterations per second per layer
    achieved = ab["verify_kernel"] / (verify_us * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": iters,
        "unit": "iters/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "ctx": w.ctx if w.ctx else list(w.ctx_range),
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "gamma": w.gamma,
                   "budget": w.budget, "n_sink": w.n_sink, "window": w.window,
                   "draft_steps": n_draft, "sparse_verify": w.sparse_verify,
                   "paged": w.paged, "logits": args.logits, "collect_rows": list(rows),
                   "score_heads": None if heads is None else list(heads),
                   "select": args.select, "draft_m": w.draft_m if args.select == "hybrid" else None,
                   "k_blocks": k_blocks if args.select == "blocks" else None,
                   "finish_select_fused": fused,
                   "kv_copies": n_copies if n_layers == 1 else 1, "layers_per_step": n_layers},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": counter_traffic(name),
                     "kernel": "attn_partials_kernel (verify)",
                     "alg_bytes_per_launch": ab["verify_kernel"], "avg_launch_us": verify_us},
        "iteration_alg_bytes": ab["iteration"],
        "iteration_hbm_frac": ab["iteration"] * iters / (HBM_PEAK_GBS * 1e9),
        "gpu_ms_per_step": gpu_ms / K,
        "stages_us": stages,
        "verify_partials_no_logits_us": verify_none_us,
        "verify_partials_collect_us": ovh["rows"],
        "logit_emit_overhead": ovh["rows"] / verify_none_us - 1.0,
        "verify_partials_all_rows_us": verify_all_us,
        "logit_emit_overhead_all_rows": verify_all_us / verify_none_us - 1.0,
        "logit_overhead_method": f"medians of {OVERHEAD_ROUNDS} alternating rounds of "
                                 f"{max(4, K // 2)} launches per kernel form",
        "combine_aggregate_us": finish_us,
        "select_us": select_us,
        "select_hybrid_us": select_hybrid_us,
        "select_blocks_us": select_blocks_us,
        "sparse_over_blocks_us": sparse_blocks_us,
        "select_block_ids_us": select_block_ids_us,
        "sparse_over_block_ids_us": sparse_block_ids_us,
    }
    if w.sparse_verify and stages.get("sparse"):
        sb = ab["sparse_kernel_kv"]
        result["sparse_roofline"] = {"achieved": sb / (stages["sparse"] * 1e-6) / 1e9,
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "alg_bytes_per_launch": sb,
                                     "avg_launch_us": stages["sparse"],
                                     "note": "whole sparse call (one kernel when it fits one split)"}
        result["sparse_roofline"]["frac"] = result["sparse_roofline"]["achieved"] / HBM_PEAK_GBS
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        # the GPU's plain selection of this layer, from its own fp32 scores
        Bn.verify_attention(q, k_copies[0], v_copies[0], lens, block_table=bt, max_ctx=max_ctx,
                            collect_rows=rows, heads=heads, layout=args.logits, logits=logits,
                            out=out, lse=lse)
        Bn.aggregate_scores(logits, lens, Hq, Hkv, layout=args.logits, scores=scores)
        Bn.select_topk(scores, lens, w.budget, w.n_sink, w.window, idx=idx, n_idx=n_idx,
                       workspace=ws_sel)
        torch.cuda.synchronize()
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds, rows, heads,
                                              gpu_idx=(idx.cpu().numpy(), n_idx.cpu().numpy()))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
