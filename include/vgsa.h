/*
 * vgsa.h -- C ABI of the verification-guided sparse attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * One decode iteration of long-context self-speculative decoding, per layer:
 *
 *   1. vgsa_verify_attention  full attention of the T = gamma + 1 verify rows
 *      (gamma draft tokens + the bonus token) over the whole KV cache, writing
 *      the pre-softmax logits of the collected rows only: normally two, the
 *      first draft token and the bonus token (any subset of the T rows can be
 *      collected, all of them included).
 *        Vegas (gist.science 2602.07223), section 2 "core mechanism", step 1
 *        (the verify pass computes the logits of every KV entry);
 *        "B. Collect-2-Query" (collect the first draft and the bonus token);
 *        section 3 "implementation" (logits before softmax normalisation are
 *        written to HBM).
 *   2. vgsa_aggregate_scores  one importance score per KV position: the sum of
 *      those logits over the collected rows and all query heads.
 *        Vegas, "A. aggregated attention-logit selection" (the summand of the
 *        argmax over subsets of size k).
 *   3. vgsa_select_topk  the k positions kept for the next step: a few
 *      attention-sink prefix positions and a recent window are always kept,
 *      the rest of the budget goes to the highest scores.
 *        Vegas "A." (argmax of the summed logits; it is separable, so it is a
 *        top-k of per-position sums); Dustin (gist.science 2606.24957),
 *        "1. hybrid attention aggregation" (sinks and local window protected,
 *        remaining budget by score).  vgsa_select_topk_hybrid fills that
 *        budget from two signals, the top m by a draft-lookahead score first.
 *   4. vgsa_sparse_attention  attention over only the selected positions, an
 *      index list used as a page-size-1 page table.
 *        Vegas section 2 step 3 (drafting with the selected entries) and
 *        section 3 (page size 1, selected token indices as page indices);
 *        Dustin "3. verification workflow" (verify on the compressed cache).
 *
 * Conventions
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or keeps a pointer after returning.
 *   - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream).  Nothing synchronises with the host.
 *   - Arguments are checked on the host before anything is launched; a failed
 *     check returns VGSA_ERR_INVALID_ARG / VGSA_ERR_UNSUPPORTED /
 *     VGSA_ERR_WORKSPACE and launches nothing.  A failed launch returns
 *     VGSA_ERR_HIP.  Faults during execution surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - Device-side values (seq_lens, n_idx, idx, block_table) are preconditions:
 *     q_len <= seq_lens[b] <= max_ctx; idx[b][0:n_idx[b]] ascending, distinct
 *     and < seq_lens[b]; n_idx[b] <= idx_stride; block ids < num_blocks.  The
 *     kernels clamp them into range so a violation gives wrong numbers, never
 *     an out-of-bounds access.
 *   - Alignment: q, k_cache, v_cache and out are read or written as 16-byte
 *     vectors and must be 16-byte aligned; a workspace must be 256-byte
 *     aligned (hipMalloc and caching-allocator blocks are).  Checked on the
 *     host: VGSA_ERR_INVALID_ARG, or VGSA_ERR_WORKSPACE for the workspace.
 *     Other pointers need only their element's natural alignment.
 *   - Row-major layouts.  GQA: q-head h reads kv-head h / (Hq / Hkv).
 *   - No global mutable state; calls are reentrant.  Calls that share a
 *     workspace must be ordered on one stream.
 *   - Causality: seq_lens[b] = L counts every cached position including the
 *     T query tokens' own K/V.  Query row t sits at absolute position L-T+t and
 *     sees positions j <= L-T+t.  The same rule applies to the absolute
 *     positions of an index list.
 */
#ifndef VGSA_H
#define VGSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vgsa_status {
  VGSA_OK = 0,
  VGSA_ERR_INVALID_ARG = 1, /* a scalar, shape or pointer is invalid         */
  VGSA_ERR_UNSUPPORTED = 2, /* valid, but outside what the kernels implement */
  VGSA_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned    */
  VGSA_ERR_HIP = 4,         /* a HIP launch failed                           */
  VGSA_ERR_TOO_LARGE = 5    /* needs more than the library's static scratch
                               (vgsa_verify_attention_noalloc only)          */
} vgsa_status;

/* Layout of the collected pre-softmax logits written by the verify pass.
 * R = number of collected rows (2 for Collect-2-Query), H = number of
 * collected q-heads (Hq unless a head subset is given). */
typedef enum vgsa_logit_layout {
  VGSA_LOGITS_NONE = 0,        /* no logits are written                           */
  VGSA_LOGITS_PER_HEAD = 1,    /* fp32 [B][R][H][max_ctx]; [b][c][i][j] is the
                                  c-th collected row (ascending row index) of the
                                  i-th collected head (ascending head index)      */
  VGSA_LOGITS_KVGROUP_SUM = 2  /* fp32 [B][Hkv][max_ctx]: sum over the collected
                                  rows and the collected q-heads of kv-head g
                                  (same total as PER_HEAD summed, R*G times fewer
                                  bytes); 0 for a kv-head with no collected head */
} vgsa_logit_layout;

/* Head mask that collects every q-head (any number of heads). */
#define VGSA_ALL_HEADS (~(uint64_t)0)

/* Shape of one attention call.  The KV cache is either contiguous,
 * K/V [B][Hkv][max_ctx][head_dim] bf16, or a paged pool of 16-position blocks,
 * K/V [num_blocks][Hkv][16][head_dim] bf16 addressed through
 * block_table[B][max_blocks_per_seq] (int32 block ids).  Cache rows are
 * addressed with 32-bit byte offsets: max_ctx * head_dim (contiguous) and
 * num_blocks * Hkv * 16 * head_dim (paged) must stay below 2^31, else
 * VGSA_ERR_UNSUPPORTED. */
typedef struct vgsa_attn_desc {
  int32_t batch;              /* B >= 0                                          */
  int32_t num_q_heads;        /* Hq >= 1, a multiple of num_kv_heads             */
  int32_t num_kv_heads;       /* Hkv >= 1                                        */
  int32_t head_dim;           /* 64 or 128                                       */
  int32_t q_len;              /* T query rows per sequence, 1..16;
                                 (Hq/Hkv) * T <= 64                              */
  int32_t max_ctx;            /* logical positions per sequence (row capacity)   */
  int32_t block_size;         /* 0: contiguous cache; 16: paged pool             */
  int32_t max_blocks_per_seq; /* paged: block_table row stride, with
                                 max_ctx <= 16 * max_blocks_per_seq              */
  int32_t num_blocks;         /* paged: blocks in the pool                       */
  float softmax_scale;        /* <= 0 selects 1/sqrt(head_dim)                   */
} vgsa_attn_desc;

/* Human-readable name of a status code (static string). */
const char* vgsa_status_string(vgsa_status status);

/* Library version string (static). */
const char* vgsa_version(void);

/* ------------------------------------------------------------------------ */
/* Split plan.  Attention over a span of positions (max_ctx for verify,
 * idx_stride for sparse) is split into num_splits chunks of `chunk`
 * positions, one workgroup per (chunk, kv-head, sequence); the partial
 * results are merged by an exact log-sum-exp combine.  Returns
 * VGSA_ERR_INVALID_ARG on a bad desc or span. */
vgsa_status vgsa_split_plan(const vgsa_attn_desc* desc, int32_t span, int32_t* num_splits,
                            int32_t* chunk);

/* Workspace bytes needed by vgsa_verify_attention / vgsa_verify_partials for
 * this desc (partial outputs of every split).  0 on an invalid desc. */
size_t vgsa_verify_workspace_bytes(const vgsa_attn_desc* desc);

/* Workspace bytes needed by vgsa_sparse_attention / vgsa_sparse_partials
 * (idx_stride: the list capacity, plus the tail of vgsa_sparse_attention).
 * vgsa_sparse_attention keeps per-(sequence, kv-head) counters in the first
 * ceil(B * Hkv * 4 / 256) * 256 bytes of its workspace, at the same place
 * whatever the span, so one workspace sized for the largest span serves
 * every smaller one: they must be zero when the workspace is first used
 * (allocate it zero-filled, and zero it again before using it with a larger
 * B * Hkv), and every call leaves them zero.  Other calls
 * (vgsa_sparse_partials, the verify calls) write a header at the start of
 * their workspace and must not be given this buffer. */
size_t vgsa_sparse_workspace_bytes(const vgsa_attn_desc* desc, int32_t idx_stride);

/* ------------------------------------------------------------------------ */
/* 1. Verify pass: full attention of the T rows, with the Collect-2-Query
 *    logit epilogue.
 *    (Vegas, section 2 step 1; "B. Collect-2-Query"; section 3.)
 *
 * q            bf16 [B][Hq][T][d]
 * k_cache,
 * v_cache      bf16, contiguous or paged (see vgsa_attn_desc)
 * block_table  int32 [B][max_blocks_per_seq]; NULL iff block_size == 0
 * seq_lens     int32 [B]; L_b includes the T verify tokens
 * collect_mask the rows whose logits are written: bit t for query row t, at
 *              least one bit, none at or above T.  Collect-2-Query: the first
 *              draft token's row 0 and the bonus row gamma, (1 | 1 << gamma).
 *              All rows, (1 << T) - 1, is the full sum of Vegas "A." (every
 *              draft token, accepted or not).  Ignored when layout ==
 *              VGSA_LOGITS_NONE.
 * head_mask    the q-heads whose logits are collected: VGSA_ALL_HEADS, or bit
 *              h for q-head h (at least one bit, none at or above Hq; needs
 *              Hq <= 64, else VGSA_ERR_UNSUPPORTED).  A subset scores on the
 *              chosen heads only (Dustin, "2. efficient estimation via
 *              semantic retrieval heads", online part); attention itself
 *              still runs on every head.  Ignored when layout == NONE.
 * logits       fp32 in `layout`; NULL iff layout == NONE.  Written for
 *              positions j < L_b only: scale * q.k for visible positions,
 *              -inf where the row may not see j.  Entries j >= L_b untouched.
 * out          bf16 [B][Hq][T][d]: softmax(scale * q K^T) V
 * lse          fp32 [B][Hq][T] natural-log sum-exp of the scaled logits, or NULL
 * workspace    >= vgsa_verify_workspace_bytes(desc) bytes of device memory;
 *              contents on entry do not matter.
 */
vgsa_status vgsa_verify_attention(const vgsa_attn_desc* desc, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, uint32_t collect_mask,
                                  uint64_t head_mask, vgsa_logit_layout layout, float* logits,
                                  void* out, float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* 1 (no allocation).  For callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid it.
 * The same call as vgsa_verify_attention, same arguments (the caller still
 * passes q, the caches, logits, out and lse) and bit-identical results, but
 * without a workspace: the split partials go to a static device array of
 * vgsa_noalloc_scratch_bytes() bytes (64 MiB) that the library holds on each
 * GPU it runs on until the process ends.  The call allocates nothing and
 * frees nothing.
 *   - VGSA_ERR_TOO_LARGE, with nothing launched, when the desc needs more
 *     than that (vgsa_verify_workspace_bytes(desc) > the scratch size).
 *   - Every call on one GPU shares that GPU's array: calls that overlap on
 *     one GPU (other streams, other host threads) race and give wrong
 *     results.  Order them on one stream.  The array keeps the last call's
 *     contents; nothing in it needs to start at zero (each call writes every
 *     byte it reads).
 *   - The array's device address is looked up on the first call made on each
 *     device (that call must run with the device current).
 */
size_t vgsa_noalloc_scratch_bytes(void);
vgsa_status vgsa_verify_attention_noalloc(const vgsa_attn_desc* desc, const void* q,
                                          const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          uint32_t collect_mask, uint64_t head_mask,
                                          vgsa_logit_layout layout, float* logits, void* out,
                                          float* lse, void* stream);

/* 2. Aggregate collected logits into one score per position.
 *    (Vegas, "A. aggregated attention-logit selection": the sum over draft
 *    rows t and heads h of l_ti^(h).)
 * logits   fp32 in `layout` (PER_HEAD or KVGROUP_SUM) as written by step 1
 * num_rows PER_HEAD: logit rows per sequence, R * H (collected rows times
 *          collected heads), 1..16*Hq; ignored for KVGROUP_SUM
 * accumulate  0: scores[b][j] = the sum; nonzero: scores[b][j] += the sum
 *          (scores summed over several layers' calls, e.g. the layers whose
 *          heads are scored)
 * scores   fp32 [B][max_ctx]; for j < L_b the sum, in a fixed order, over
 *          the logit rows (or over kv-groups).  Entries j >= L_b untouched.
 */
vgsa_status vgsa_aggregate_scores(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t max_ctx, vgsa_logit_layout layout, int32_t num_rows,
                                  int32_t accumulate, const float* logits,
                                  const int32_t* seq_lens, float* scores, void* stream);

/* 3. Select the positions kept for the next step.
 *    (Vegas "A." argmax over |T| = k; Dustin "1." protected sinks and window.)
 * scores    fp32 [B][max_ctx]
 * k         budget >= 1, including sinks and window; n_sink + window <= k
 * n_sink    leading positions always kept
 * window    trailing positions always kept
 * idx       int32 [B][idx_stride], idx_stride >= k.  Row b receives, in
 *           ascending order, F = [0, min(n_sink, L)) U [max(0, L-window), L)
 *           plus the k - |F| other positions of highest score (lower position
 *           first among equal scores; -0.0 equals +0.0); every position when
 *           k >= L.
 * n_idx     int32 [B]: min(k, L_b)
 */
vgsa_status vgsa_select_topk(int32_t batch, int32_t max_ctx, const float* scores,
                             const int32_t* seq_lens, int32_t k, int32_t n_sink, int32_t window,
                             int32_t* idx, int32_t idx_stride, int32_t* n_idx, void* stream);

/* 3 (with a workspace).  The same selection as vgsa_select_topk, same
 * arguments and results; a max_ctx of 49153 .. 262144 positions spreads each
 * row over one workgroup per round of 32768 (three launches on `stream`)
 * instead of one workgroup per row.
 * workspace  >= vgsa_select_workspace_bytes(batch, max_ctx) bytes of device
 *            memory, 256-byte aligned; it holds per-round histograms,
 *            bitmaps and candidate lists between the launches, needs no
 *            initial contents, and calls that share it must not overlap.
 *            When that size is 0 (max_ctx <= 49152 or > 262144) workspace may
 *            be NULL and the call is vgsa_select_topk.
 * Errors: as vgsa_select_topk; VGSA_ERR_WORKSPACE for a missing, small or
 * misaligned workspace.
 */
size_t vgsa_select_workspace_bytes(int32_t batch, int32_t max_ctx);
vgsa_status vgsa_select_topk_ws(int32_t batch, int32_t max_ctx, const float* scores,
                                const int32_t* seq_lens, int32_t k, int32_t n_sink,
                                int32_t window, int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                                void* workspace, size_t workspace_bytes, void* stream);

/* 3'. Hybrid selection from two signals.
 *    (Dustin, "1. hybrid attention aggregation": target-historical attention
 *    from the previous forward pass and draft-lookahead attention from the
 *    draft; after the protected sinks and window the budget is filled
 *    hierarchically, the top m by the draft signal first, the remainder by
 *    the target signal.)
 * target_scores  fp32 [B][max_ctx], e.g. as written by step 2
 * draft_scores   fp32 [B][max_ctx], the draft-lookahead score per position
 *                (the library does not compute it: it comes from the draft)
 * m              draft-chosen positions, >= 0; clamped to r = k - |F|
 * k, n_sink, window, idx, idx_stride, n_idx  as vgsa_select_topk.  Row b
 *           receives, ascending, F plus the min(m, r) positions of F's
 *           complement with the highest draft scores plus the r - min(m, r)
 *           positions of highest target score among the rest (ties: lower
 *           position first); every position when k >= L.
 * Rows are limited to max_ctx <= 262144 (VGSA_ERR_UNSUPPORTED beyond).
 */
vgsa_status vgsa_select_topk_hybrid(int32_t batch, int32_t max_ctx, const float* target_scores,
                                    const float* draft_scores, const int32_t* seq_lens, int32_t k,
                                    int32_t m, int32_t n_sink, int32_t window, int32_t* idx,
                                    int32_t idx_stride, int32_t* n_idx, void* stream);

/* 3' (with a workspace).  The same selection as vgsa_select_topk_hybrid,
 * same arguments and results; for a max_ctx of 49153 .. 262144 positions
 * each stage spreads a row over one workgroup per round of 32768 (six
 * launches on `stream`).  workspace as for vgsa_select_topk_ws (same size,
 * vgsa_select_workspace_bytes); when that size is 0 the call is
 * vgsa_select_topk_hybrid.
 */
vgsa_status vgsa_select_topk_hybrid_ws(int32_t batch, int32_t max_ctx, const float* target_scores,
                                       const float* draft_scores, const int32_t* seq_lens,
                                       int32_t k, int32_t m, int32_t n_sink, int32_t window,
                                       int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* 3''. Block-granular selection (structured block sparsity).
 *    (The euno.news summary of arXiv 2512.21911, "3. sparse verification
 *    engine": top keys kept in structured blocks; Quest's page-level
 *    selection in Dustin's comparison.  Under Vegas "A."'s summed-logit
 *    objective the best whole blocks are those of largest block sum.)
 * scores    fp32 [B][max_ctx]
 * k_blocks  blocks kept, >= 1
 * block     positions per block, 1..1024 (16 matches a paged cache's pages)
 * n_sink, window  the blocks holding positions [0, n_sink) and
 *           [L - window, L) are always kept; ceil(n_sink / block) +
 *           ceil(window / block) + 1 (the last term only when window > 0)
 *           must not exceed k_blocks
 * idx       int32 [B][idx_stride], idx_stride >= k_blocks * block.  Row b
 *           receives, ascending, every position below L of the kept blocks:
 *           the forced ones plus the others of largest block sum (the sum of
 *           the members' scores in float32, position order; lower block first
 *           among equal sums); every position when the blocks of L number at
 *           most k_blocks.
 * n_idx     int32 [B]: positions written
 * block_sums  nullable fp32 [B][ceil(max_ctx / block)], caller-owned device
 *           memory: when given, row b receives the block sums the ranking
 *           compared (float32, members summed in position order) for blocks
 *           [0, ceil(L / block)); later entries are left untouched.  It lets a
 *           caller check the sums against an exact sum and rank them itself.
 * Rows are limited to ceil(max_ctx / block) <= 8704 blocks
 * (VGSA_ERR_UNSUPPORTED beyond).
 */
vgsa_status vgsa_select_blocks(int32_t batch, int32_t max_ctx, const float* scores,
                               const int32_t* seq_lens, int32_t k_blocks, int32_t block,
                               int32_t n_sink, int32_t window, int32_t* idx, int32_t idx_stride,
                               int32_t* n_idx, float* block_sums, void* stream);

/* 3'' (block ids).  The same selection as vgsa_select_blocks, written as
 * the kept blocks' ids instead of their positions, for the block-list gather
 * (vgsa_sparse_attention_blocks).
 * block_ids  int32 [B][ids_stride], ids_stride >= k_blocks.  Row b receives
 *          the kept blocks ascending (block i covers positions
 *          [i * block, (i + 1) * block)); every block of [0, L) when they
 *          number at most k_blocks.
 * n_ids    int32 [B]: blocks written
 * Other arguments, limits and errors as vgsa_select_blocks.
 */
vgsa_status vgsa_select_block_ids(int32_t batch, int32_t max_ctx, const float* scores,
                                  const int32_t* seq_lens, int32_t k_blocks, int32_t block,
                                  int32_t n_sink, int32_t window, int32_t* block_ids,
                                  int32_t ids_stride, int32_t* n_ids, float* block_sums,
                                  void* stream);

/* 4. Sparse attention over an index list (page size 1).
 *    (Vegas section 2 step 3 and section 3; Dustin "3.")
 * desc->q_len is T' (1 for a draft step, gamma + 1 for a sparse verify).
 * idx, n_idx, idx_stride  as written by vgsa_select_topk (a caller may append
 *          positions, e.g. freshly drafted tokens, keeping the row ascending)
 * tail     >= 0: the last min(tail, L'_b) positions below L'_b are attended
 *          too, after the listed ones (the tokens drafted since the selection,
 *          without appending them to the lists); listed positions must lie
 *          below L'_b - tail.  0: the list alone.
 * seq_lens L'_b for the causal rule: row t sees listed j <= L'_b - T' + t.
 *          A row that sees no listed position gets out = 0, lse = -inf.
 * workspace  >= vgsa_sparse_workspace_bytes(desc, idx_stride + tail) bytes,
 *          its counter part zero on first use (see there).  One launch: a
 *          long list is split over several workgroups per (sequence,
 *          kv-head), and the last of them to finish merges their partial
 *          results.  Calls that share a workspace must not overlap.
 * Other arguments as in vgsa_verify_attention.
 */
vgsa_status vgsa_sparse_attention(const vgsa_attn_desc* desc, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, const int32_t* idx,
                                  const int32_t* n_idx, int32_t idx_stride, int32_t tail,
                                  void* out, float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* 4 (block lists).  Sparse attention over whole blocks of positions
 *    (structured block sparsity: the euno.news summary of arXiv 2512.21911,
 *    "3. sparse verification engine"; with block = 16 on a paged cache each
 *    listed block is one page, Vegas section 3).  The same attention as
 *    vgsa_sparse_attention over the position list that the blocks expand
 *    to, without that list being written out.
 * block_ids, n_ids, ids_stride  int32 [B][ids_stride] ascending distinct
 *          block ids as written by vgsa_select_block_ids, n_ids[b] of them
 *          (0 .. ids_stride); block i stands for positions [i * block,
 *          (i + 1) * block) clipped to [0, L'_b - tail): only the last
 *          listed block may reach past L'_b - tail, and ids must be below
 *          ceil((L'_b - tail) / block).
 * block    positions per block, 1 .. 1024
 * tail     as in vgsa_sparse_attention (the positions L'_b - tail .. L'_b - 1
 *          follow the blocks' positions)
 * workspace  >= vgsa_sparse_workspace_bytes(desc, ids_stride * block + tail)
 *          bytes, its counter part zero on first use (as for
 *          vgsa_sparse_attention, which it may share).
 * Other arguments and errors as vgsa_sparse_attention; VGSA_ERR_INVALID_ARG
 * for a block outside 1 .. 1024.
 */
vgsa_status vgsa_sparse_attention_blocks(const vgsa_attn_desc* desc, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         const int32_t* block_ids, const int32_t* n_ids,
                                         int32_t ids_stride, int32_t block, int32_t tail, void* out,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* Draft steps: append consecutive positions to index lists.
 *    (Vegas section 2 step 3: each drafting step attends over the selected
 *    entries and the tokens drafted since the selection.)
 * For each b, positions base[b] + first, ..., base[b] + first + count - 1 are
 * written at idx[b][n_idx[b]], ... and n_idx[b] grows by count; entries that
 * would land at or past idx_stride are dropped (n_idx[b] stops at
 * idx_stride).  The row stays ascending when the new positions lie past every
 * listed one, as drafted tokens past the selection's lengths do.
 * base      int32 [B], e.g. the lengths the lists were selected at
 * idx       int32 [B][idx_stride]; n_idx int32 [B]: both updated in place
 * count 0 or batch 0: nothing is launched. */
vgsa_status vgsa_append_positions(int32_t batch, const int32_t* base, int32_t first, int32_t count,
                                  int32_t* idx, int32_t idx_stride, int32_t* n_idx, void* stream);

/* ------------------------------------------------------------------------ */
/* Two-phase form of steps 1 and 4, for callers that time or schedule the
 * phases separately.  vgsa_verify_attention == vgsa_verify_partials followed
 * by vgsa_combine_partials(span = max_ctx, lengths = seq_lens);
 * vgsa_sparse_attention == vgsa_sparse_partials followed by
 * vgsa_combine_partials(span = idx_stride, lengths = n_idx).
 * The partials live in the workspace between the two calls. */
vgsa_status vgsa_verify_partials(const vgsa_attn_desc* desc, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, uint32_t collect_mask,
                                 uint64_t head_mask, vgsa_logit_layout layout, float* logits,
                                 void* workspace, size_t workspace_bytes, void* stream);

vgsa_status vgsa_sparse_partials(const vgsa_attn_desc* desc, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* idx,
                                 const int32_t* n_idx, int32_t idx_stride, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Merge the split partials (exact log-sum-exp combine) into out / lse.
 * lengths: seq_lens (verify) or n_idx (sparse): chunks at or past a
 * sequence's length hold nothing and are skipped. */
vgsa_status vgsa_combine_partials(const vgsa_attn_desc* desc, int32_t span,
                                  const int32_t* lengths, const void* workspace,
                                  size_t workspace_bytes, void* out, float* lse, void* stream);

/* Steps 1 (second phase) and 2 in one launch: merge the verify partials into
 * out / lse exactly as vgsa_combine_partials(span = max_ctx, lengths =
 * seq_lens) and, when scores is non-NULL, aggregate the collected logits into
 * scores exactly as vgsa_aggregate_scores (same per-position summation order,
 * so the values are identical).  Both only read what vgsa_verify_partials
 * wrote, so one kernel does both.
 * (Vegas §2 step 1 and "A. aggregated attention-logit selection".)
 * layout   the layout logits were written in (PER_HEAD or KVGROUP_SUM);
 *          ignored when scores is NULL
 * num_rows PER_HEAD: logit rows per sequence (R * H), 1..q_len*Hq
 * accumulate  as in vgsa_aggregate_scores
 * scores   fp32 [B][max_ctx] or NULL */
vgsa_status vgsa_verify_finish(const vgsa_attn_desc* desc, const int32_t* seq_lens,
                               const void* workspace, size_t workspace_bytes, void* out, float* lse,
                               vgsa_logit_layout layout, int32_t num_rows, int32_t accumulate,
                               const float* logits, float* scores, void* stream);

/* Steps 1 (second phase), 2 and 3 in one launch: vgsa_verify_finish with
 * scores, then vgsa_select_topk on the scores it wrote, with the same results
 * as those two calls (identical out, lse, scores, idx and n_idx).
 *    (Vegas §2 steps 1-2, "A. aggregated attention-logit selection";
 *    Dustin "1." protected sinks and window.)
 * The workgroups that sum a sequence's scores also count the leading 12 bits
 * of their order-preserving keys into a histogram of that sequence and list
 * their candidates (the keys at or above their own threshold bin); the last
 * of them to finish selects the sequence's positions in the same launch from
 * that histogram and those lists.  No workgroup waits on another.  One
 * workgroup selects each sequence, so rows of more than two 32768-position
 * rounds select faster with the two calls (vgsa_select_topk_ws spreads a
 * row over one workgroup per round).
 * desc .. scores  as vgsa_verify_finish; scores must not be NULL
 * k, n_sink, window, idx, idx_stride, n_idx  as vgsa_select_topk
 * select_workspace  >= vgsa_finish_select_workspace_bytes(batch, max_ctx)
 *          bytes of device memory, 256-byte aligned: per-sequence histograms
 *          and counters, then the candidate lists (scratch, 8 bytes per
 *          position).  It must be zero before its first use (e.g. a
 *          zero-filled allocation); every call leaves it ready for the next
 *          (the histograms and counters zero again).  Calls that share it
 *          must not overlap.
 * Errors: as vgsa_verify_finish and vgsa_select_topk; VGSA_ERR_UNSUPPORTED
 * for max_ctx > 262144 (make the two calls instead); VGSA_ERR_WORKSPACE for a
 * missing, small or misaligned select_workspace.
 */
/* Bytes of select_workspace for batch sequences of capacity max_ctx; 0 for
 * batch outside 1..65535 or max_ctx outside 1..262144. */
size_t vgsa_finish_select_workspace_bytes(int32_t batch, int32_t max_ctx);
vgsa_status vgsa_verify_finish_select(const vgsa_attn_desc* desc, const int32_t* seq_lens,
                                      const void* workspace, size_t workspace_bytes, void* out,
                                      float* lse, vgsa_logit_layout layout, int32_t num_rows,
                                      int32_t accumulate, const float* logits, float* scores,
                                      int32_t k, int32_t n_sink, int32_t window, int32_t* idx,
                                      int32_t idx_stride, int32_t* n_idx, void* select_workspace,
                                      size_t select_workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VGSA_H */
