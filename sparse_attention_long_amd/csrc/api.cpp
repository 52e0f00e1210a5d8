// C ABI of the library: argument validation on the host, split planning and
// kernel launches.  Validation is pure host code and runs before any HIP call,
// so a rejected call touches neither the device nor the stream.
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace vgsa {

size_t partial_bytes(const vgsa_attn_desc& d, const SplitPlan& p);
size_t sparse_sync_bytes(const vgsa_attn_desc& d);

namespace {

constexpr int64_t kMaxGridYZ = 65535;
// Largest block of a block list (positions per entry), as in block selection.
constexpr int32_t kMaxIdBlock = 1024;
constexpr int64_t kMaxOffset = 0x7FFFFFFFLL;  // elements: byte offsets stay within 32 bits
constexpr uintptr_t kWorkspaceAlign = 256;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

vgsa_status check_desc(const vgsa_attn_desc* d) {
  if (d == nullptr) return VGSA_ERR_INVALID_ARG;
  if (d->batch < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1) return VGSA_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return VGSA_ERR_INVALID_ARG;
  if (d->head_dim < 1 || d->q_len < 1 || d->max_ctx < 1) return VGSA_ERR_INVALID_ARG;
  if (!isfinite(d->softmax_scale)) return VGSA_ERR_INVALID_ARG;
  if (d->block_size < 0) return VGSA_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return VGSA_ERR_UNSUPPORTED;
  if (d->q_len > 16) return VGSA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)(d->num_q_heads / d->num_kv_heads) * d->q_len;
  if (rows > kMaxRows) return VGSA_ERR_UNSUPPORTED;
  if (d->batch > kMaxGridYZ || d->num_kv_heads > kMaxGridYZ) return VGSA_ERR_UNSUPPORTED;
  if (d->block_size == 16) {
    if (d->max_blocks_per_seq < 1 || d->num_blocks < 1) return VGSA_ERR_INVALID_ARG;
    if ((int64_t)d->max_ctx > (int64_t)16 * d->max_blocks_per_seq) return VGSA_ERR_INVALID_ARG;
    // element offsets inside the pool are 32-bit
    if ((int64_t)d->num_blocks * d->num_kv_heads * 16 * d->head_dim > kMaxOffset)
      return VGSA_ERR_UNSUPPORTED;
  } else if (d->block_size != 0) {
    return VGSA_ERR_UNSUPPORTED;
  }
  // element offsets inside one (sequence, kv-head) row are 32-bit
  if ((int64_t)d->max_ctx * d->head_dim > kMaxOffset) return VGSA_ERR_UNSUPPORTED;
  return VGSA_OK;
}

float effective_scale(const vgsa_attn_desc& d) {
  return d.softmax_scale > 0.f ? d.softmax_scale : 1.0f / sqrtf((float)d.head_dim);
}

struct Carve {
  int32_t* header;
  float* part_o;
  float* part_ml;
};

Carve carve(const vgsa_attn_desc& d, const SplitPlan& p, void* ws) {
  const size_t o_bytes = (size_t)d.batch * d.num_q_heads * d.q_len * p.part_splits * d.head_dim * 4;
  const size_t o_aligned = (o_bytes + 255) / 256 * 256;
  Carve c;
  c.header = static_cast<int32_t*>(ws);
  c.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + kHeaderBytes);
  c.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + kHeaderBytes + o_aligned);
  return c;
}

vgsa_status hip_status(hipError_t e) { return e == hipSuccess ? VGSA_OK : VGSA_ERR_HIP; }

AttnArgs base_args(const vgsa_attn_desc& d, const SplitPlan& p, const void* q, const void* k,
                   const void* v, const int32_t* block_table, const int32_t* seq_lens,
                   void* workspace) {
  AttnArgs a{};
  a.row_split = 1;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.batch = d.batch;
  a.hq = d.num_q_heads;
  a.hkv = d.num_kv_heads;
  a.group = d.num_q_heads / d.num_kv_heads;
  a.q_len = d.q_len;
  a.head_dim = d.head_dim;
  a.max_ctx = d.max_ctx;
  a.paged = d.block_size == 16 ? 1 : 0;
  a.max_blocks = d.max_blocks_per_seq;
  a.num_blocks = d.num_blocks;
  a.num_splits = p.num_splits;
  a.chunk = p.chunk;
  a.waves = p.waves;
  a.scale = effective_scale(d);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  const Carve c = carve(d, p, workspace);
  a.part_o = c.part_o;
  a.part_ml = c.part_ml;
  a.header = c.header;
  a.part_splits = p.part_splits;
  a.balance = 0;
  a.layout = VGSA_LOGITS_NONE;
  a.row_mask = 0u;
  a.n_rows = 0;
  a.head_mask = kAllHeads;
  a.n_heads = d.num_q_heads;
  a.out = nullptr;
  a.lse = nullptr;
  a.direct = 0;
  a.id_block = 1;
  return a;
}

bool aligned(const void* p, uintptr_t bytes) {
  return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0;
}

// The partials are read and written as 16-byte vectors.
vgsa_status check_workspace(const void* ws, size_t have, size_t need) {
  if (ws == nullptr || have < need || !aligned(ws, kWorkspaceAlign)) return VGSA_ERR_WORKSPACE;
  return VGSA_OK;
}

vgsa_status check_attn_pointers(const vgsa_attn_desc& d, const void* q, const void* k,
                                const void* v, const int32_t* block_table,
                                const int32_t* seq_lens) {
  if (q == nullptr || k == nullptr || v == nullptr || seq_lens == nullptr)
    return VGSA_ERR_INVALID_ARG;
  // q, K and V rows are loaded as 16-byte vectors
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return VGSA_ERR_INVALID_ARG;
  if ((d.block_size == 16) != (block_table != nullptr)) return VGSA_ERR_INVALID_ARG;
  return VGSA_OK;
}

}  // namespace

SplitPlan make_plan(const vgsa_attn_desc& d, int32_t span) {
  if (span < 1) span = 1;  // callers validate; keep the plan total anyway
  const int waves = attention_waves(d);
  const bool wide = waves == kWavesWide;
  const int64_t min_chunk = wide ? kMinChunkWide : kMinChunk;
  const int64_t plan_chunk = wide ? kPlanChunkWide : kPlanChunk;
  const int64_t max_chunk = wide ? kMaxChunkWide : kMaxChunk;
  const int64_t target = wide ? kTargetWorkgroupsWide : kTargetWorkgroups;
  const int64_t bh = (int64_t)(d.batch > 0 ? d.batch : 1) * d.num_kv_heads;
  const int64_t max_splits =
      span <= kDirectSpan ? 1 : (ceil_div(span, min_chunk) > 0 ? ceil_div(span, min_chunk) : 1);
  int64_t s = ceil_div(target, bh);
  if (s < 1) s = 1;
  if (s > max_splits) s = max_splits;
  int64_t chunk = ceil_div(ceil_div(span, s), min_chunk) * min_chunk;
  if (chunk > plan_chunk) {
    chunk = plan_chunk;
    // A last split of a sliver would add a workgroup to every (sequence,
    // kv-head), and one more split changes which workgroups share a CU and
    // an XCD (17 splits measured 10 % slower than 16 at 128K x b8): the
    // sliver is spread over the other splits instead (chunk <= max_chunk).
    const int64_t n = ceil_div(span, plan_chunk);
    if (n > 1 && span - (n - 1) * plan_chunk <= max_chunk - plan_chunk)
      chunk = ceil_div(ceil_div(span, n - 1), min_chunk) * min_chunk;
  }
  s = ceil_div(span, chunk);
  SplitPlan p;
  p.num_splits = (int32_t)s;
  p.chunk = (int32_t)chunk;
  p.part_splits = (s > 1 && d.batch > 1 && d.batch <= kMaxBalanceBatch)
                      ? (int32_t)(kBalanceSplits * s) : (int32_t)s;
  p.waves = waves;
  return p;
}

size_t partial_bytes(const vgsa_attn_desc& d, const SplitPlan& p) {
  const size_t rows = (size_t)d.batch * d.num_q_heads * d.q_len * p.part_splits;
  const size_t o_bytes = rows * d.head_dim * 4;
  return kHeaderBytes + (o_bytes + 255) / 256 * 256 + rows * 2 * 4;
}

// The one-call sparse workspace: the fused merge's arrival counters (one
// int32 per (sequence, kv-head)) at its start, then the partials.  The
// counters' place does not depend on the span, so one zero-filled workspace
// serves calls whose split plans differ (e.g. draft steps of growing tails).
size_t sparse_sync_bytes(const vgsa_attn_desc& d) {
  return ((size_t)d.batch * d.num_kv_heads * 4 + 255) / 256 * 256;
}

}  // namespace vgsa

using namespace vgsa;

extern "C" {

const char* vgsa_status_string(vgsa_status status) {
  switch (status) {
    case VGSA_OK: return "ok";
    case VGSA_ERR_INVALID_ARG: return "invalid argument";
    case VGSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case VGSA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case VGSA_ERR_HIP: return "HIP launch failed";
    case VGSA_ERR_TOO_LARGE: return "request exceeds the library's static scratch";
  }
  return "unknown status";
}

const char* vgsa_version(void) { return "vgsa 0.1.0 gfx950"; }

vgsa_status vgsa_split_plan(const vgsa_attn_desc* desc, int32_t span, int32_t* num_splits,
                            int32_t* chunk) {
  const vgsa_status st = check_desc(desc);
  if (st != VGSA_OK) return st;
  if (span < 1 || num_splits == nullptr || chunk == nullptr) return VGSA_ERR_INVALID_ARG;
  const SplitPlan p = make_plan(*desc, span);
  *num_splits = p.num_splits;
  *chunk = p.chunk;
  return VGSA_OK;
}

size_t vgsa_verify_workspace_bytes(const vgsa_attn_desc* desc) {
  if (check_desc(desc) != VGSA_OK) return 0;
  return partial_bytes(*desc, make_plan(*desc, desc->max_ctx));
}

size_t vgsa_sparse_workspace_bytes(const vgsa_attn_desc* desc, int32_t idx_stride) {
  if (check_desc(desc) != VGSA_OK || idx_stride < 1) return 0;
  return sparse_sync_bytes(*desc) +
         partial_bytes(*desc, make_plan(*desc, idx_stride));
}

}  // extern "C"

namespace {

// Verify launch: partials into the workspace, or (out != null, one split)
// the final output directly.
vgsa_status verify_launch(const vgsa_attn_desc* desc, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                          uint32_t collect_mask, uint64_t head_mask, vgsa_logit_layout layout,
                          float* logits, void* workspace, size_t workspace_bytes, void* out,
                          float* lse, void* stream) {
  vgsa_status st = check_desc(desc);
  if (st != VGSA_OK) return st;
  const vgsa_attn_desc& d = *desc;
  st = check_attn_pointers(d, q, k_cache, v_cache, block_table, seq_lens);
  if (st != VGSA_OK) return st;
  if (layout != VGSA_LOGITS_NONE && layout != VGSA_LOGITS_PER_HEAD &&
      layout != VGSA_LOGITS_KVGROUP_SUM)
    return VGSA_ERR_INVALID_ARG;
  if (layout != VGSA_LOGITS_NONE) {
    if (logits == nullptr) return VGSA_ERR_INVALID_ARG;
    if (collect_mask == 0u || (collect_mask >> d.q_len) != 0u) return VGSA_ERR_INVALID_ARG;
    if (head_mask != kAllHeads) {
      // a head subset names heads by bit: at most 64 heads, at least one named
      if (d.num_q_heads > 64) return VGSA_ERR_UNSUPPORTED;
      if (head_mask == 0ull) return VGSA_ERR_INVALID_ARG;
      if (d.num_q_heads < 64 && (head_mask >> d.num_q_heads) != 0ull) return VGSA_ERR_INVALID_ARG;
    }
  }
  const SplitPlan p = make_plan(d, d.max_ctx);
  st = check_workspace(workspace, workspace_bytes, partial_bytes(d, p));
  if (st != VGSA_OK) return st;
  if (d.batch == 0) return VGSA_OK;
  AttnArgs a = base_args(d, p, q, k_cache, v_cache, block_table, seq_lens, workspace);
  a.layout = layout;
  a.logits = layout == VGSA_LOGITS_NONE ? nullptr : logits;
  a.row_mask = layout == VGSA_LOGITS_NONE ? 0u : collect_mask;
  a.n_rows = __builtin_popcount(a.row_mask);
  a.head_mask = layout == VGSA_LOGITS_NONE ? kAllHeads : head_mask;
  a.n_heads = a.head_mask == kAllHeads ? d.num_q_heads : __builtin_popcountll(a.head_mask);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.direct = out != nullptr ? 1 : 0;
  a.balance = (!a.direct && p.part_splits > p.num_splits) ? 1 : 0;
  return hip_status(launch_attention_partials(a, false, static_cast<hipStream_t>(stream)));
}

vgsa_status sparse_launch(const vgsa_attn_desc* desc, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                          const int32_t* idx, const int32_t* n_idx, int32_t idx_stride,
                          int32_t tail, void* workspace, size_t workspace_bytes, void* out,
                          float* lse, bool fused, void* stream, int32_t id_block = 1) {
  vgsa_status st = check_desc(desc);
  if (st != VGSA_OK) return st;
  const vgsa_attn_desc& d = *desc;
  st = check_attn_pointers(d, q, k_cache, v_cache, block_table, seq_lens);
  if (st != VGSA_OK) return st;
  if (idx == nullptr || n_idx == nullptr || idx_stride < 1 || tail < 0) return VGSA_ERR_INVALID_ARG;
  if ((int64_t)idx_stride * id_block + tail > 0x7fffffff) return VGSA_ERR_UNSUPPORTED;
  // entries: up to idx_stride listed (times the block size for block lists),
  // then the trailing positions
  const int32_t span = idx_stride * id_block + tail;
  // one split for lists up to kDirectSpan (the output is written directly);
  // longer lists split, and with `fused` the splits merge in the same launch
  const SplitPlan p = make_plan(d, span);
  // fused: the counters first, the partials after them; the fused merge
  // addresses the partials with 32-bit byte offsets
  if (fused && p.num_splits > 1 && partial_bytes(d, p) > (size_t)0x7FFFFFFF)
    return VGSA_ERR_UNSUPPORTED;
  const size_t sync_bytes = fused ? sparse_sync_bytes(d) : 0;
  st = check_workspace(workspace, workspace_bytes, sync_bytes + partial_bytes(d, p));
  if (st != VGSA_OK) return st;
  if (d.batch == 0) return VGSA_OK;
  AttnArgs a = base_args(d, p, q, k_cache, v_cache, block_table, seq_lens,
                         static_cast<char*>(workspace) + sync_bytes);
  a.idx = idx;
  a.n_idx = n_idx;
  a.idx_stride = idx_stride;
  a.tail = tail;
  a.id_block = id_block;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  // one call: a single split writes the output itself, several merge in the launch
  a.direct = (out != nullptr && p.num_splits == 1) ? 1 : 0;
  // a single split of more than one 16-row block: two workgroups share the
  // rows (all 256 CUs work, each workgroup runs fewer MFMA blocks and merges
  // fewer rows; the pair's gathers cost one HBM read)
  a.row_split = (a.direct && p.waves == kWavesWide && a.group * a.q_len > 16) ? 2 : 1;
  if (fused && p.num_splits > 1) {
    a.fuse = 1;
    a.sync = static_cast<int32_t*>(workspace);
  }
  return hip_status(launch_attention_partials(a, true, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

vgsa_status vgsa_verify_partials(const vgsa_attn_desc* desc, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, uint32_t collect_mask,
                                 uint64_t head_mask, vgsa_logit_layout layout, float* logits,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return verify_launch(desc, q, k_cache, v_cache, block_table, seq_lens, collect_mask, head_mask,
                       layout,
                       logits, workspace, workspace_bytes, nullptr, nullptr,
                       stream);
}

vgsa_status vgsa_sparse_partials(const vgsa_attn_desc* desc, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* idx,
                                 const int32_t* n_idx, int32_t idx_stride, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return sparse_launch(desc, q, k_cache, v_cache, block_table, seq_lens, idx, n_idx, idx_stride,
                       0, workspace, workspace_bytes, nullptr, nullptr, false, stream);
}

vgsa_status vgsa_combine_partials(const vgsa_attn_desc* desc, int32_t span,
                                  const int32_t* lengths, const void* workspace,
                                  size_t workspace_bytes, void* out, float* lse, void* stream) {
  vgsa_status st = check_desc(desc);
  if (st != VGSA_OK) return st;
  const vgsa_attn_desc& d = *desc;
  if (span < 1 || lengths == nullptr || out == nullptr || !aligned(out, 16))
    return VGSA_ERR_INVALID_ARG;
  const SplitPlan p = make_plan(d, span);
  st = check_workspace(workspace, workspace_bytes, partial_bytes(d, p));
  if (st != VGSA_OK) return st;
  const int64_t rows = (int64_t)d.batch * d.num_q_heads * d.q_len;
  if (rows > 0x7fffffff) return VGSA_ERR_UNSUPPORTED;
  if (rows == 0) return VGSA_OK;
  const Carve c = carve(d, p, const_cast<void*>(workspace));
  CombineArgs a{};
  a.part_o = c.part_o;
  a.part_ml = c.part_ml;
  a.lengths = lengths;
  a.rows = (int32_t)rows;
  a.rows_per_seq = d.num_q_heads * d.q_len;
  a.head_dim = d.head_dim;
  a.num_splits = p.num_splits;
  a.chunk = p.chunk;
  a.span = span;
  a.part_splits = p.part_splits;
  a.header = c.header;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  return hip_status(launch_combine(a, static_cast<hipStream_t>(stream)));
}

vgsa_status vgsa_verify_attention(const vgsa_attn_desc* desc, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, uint32_t collect_mask,
                                  uint64_t head_mask, vgsa_logit_layout layout, float* logits,
                                  void* out, float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  vgsa_status st = check_desc(desc);
  if (st != VGSA_OK) return st;
  if (out == nullptr || !aligned(out, 16)) return VGSA_ERR_INVALID_ARG;
  const SplitPlan p = make_plan(*desc, desc->max_ctx);
  if (p.num_splits == 1) {
    // one split: the partials kernel finishes the softmax and writes out / lse
    return verify_launch(desc, q, k_cache, v_cache, block_table, seq_lens, collect_mask, head_mask,
                         layout, logits, workspace, workspace_bytes, out, lse, stream);
  }
  st = verify_launch(desc, q, k_cache, v_cache, block_table, seq_lens, collect_mask, head_mask,
                     layout, logits, workspace, workspace_bytes, nullptr, nullptr, stream);
  if (st != VGSA_OK) return st;
  return vgsa_combine_partials(desc, desc->max_ctx, seq_lens, workspace, workspace_bytes, out,
                               lse, stream);
}

vgsa_status vgsa_sparse_attention(const vgsa_attn_desc* desc, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, const int32_t* idx,
                                  const int32_t* n_idx, int32_t idx_stride, int32_t tail, void* out,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  vgsa_status st = check_desc(desc);
  if (st != VGSA_OK) return st;
  if (out == nullptr || !aligned(out, 16) || idx_stride < 1) return VGSA_ERR_INVALID_ARG;
  // one launch: the splits of a (sequence, kv-head) merge in the same kernel
  return sparse_launch(desc, q, k_cache, v_cache, block_table, seq_lens, idx, n_idx, idx_stride,
                       tail, workspace, workspace_bytes, out, lse, true, stream);
}

vgsa_status vgsa_sparse_attention_blocks(const vgsa_attn_desc* desc, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         const int32_t* block_ids, const int32_t* n_ids,
                                         int32_t ids_stride, int32_t block, int32_t tail, void* out,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  vgsa_status st = check_desc(desc);
  if (st != VGSA_OK) return st;
  if (out == nullptr || !aligned(out, 16) || ids_stride < 1 || block < 1 || block > kMaxIdBlock)
    return VGSA_ERR_INVALID_ARG;
  return sparse_launch(desc, q, k_cache, v_cache, block_table, seq_lens, block_ids, n_ids,
                       ids_stride, tail, workspace, workspace_bytes, out, lse, true, stream, block);
}

}  // extern "C"

namespace {

// Validation and launch arguments of the finish step (combine + aggregate).
vgsa_status finish_args(const vgsa_attn_desc* desc, const int32_t* seq_lens,
                        const void* workspace, size_t workspace_bytes, void* out, float* lse,
                        vgsa_logit_layout layout, int32_t num_rows, int32_t accumulate,
                        const float* logits, float* scores, CombineArgs& ca, AggregateArgs& ag) {
  vgsa_status st = check_desc(desc);
  if (st != VGSA_OK) return st;
  const vgsa_attn_desc& d = *desc;
  if (seq_lens == nullptr || out == nullptr || !aligned(out, 16)) return VGSA_ERR_INVALID_ARG;
  if (scores != nullptr) {
    if (layout != VGSA_LOGITS_PER_HEAD && layout != VGSA_LOGITS_KVGROUP_SUM)
      return VGSA_ERR_INVALID_ARG;
    if (logits == nullptr) return VGSA_ERR_INVALID_ARG;
    if (layout == VGSA_LOGITS_PER_HEAD &&
        (num_rows < 1 || num_rows > (int64_t)d.q_len * d.num_q_heads))
      return VGSA_ERR_INVALID_ARG;
  }
  const SplitPlan p = make_plan(d, d.max_ctx);
  st = check_workspace(workspace, workspace_bytes, partial_bytes(d, p));
  if (st != VGSA_OK) return st;
  const int64_t rows = (int64_t)d.batch * d.num_q_heads * d.q_len;
  if (rows > 0x7fffffff) return VGSA_ERR_UNSUPPORTED;
  const Carve c = carve(d, p, const_cast<void*>(workspace));
  ca = CombineArgs{};
  ca.part_o = c.part_o;
  ca.part_ml = c.part_ml;
  ca.lengths = seq_lens;
  ca.rows = (int32_t)rows;
  ca.rows_per_seq = d.num_q_heads * d.q_len;
  ca.head_dim = d.head_dim;
  ca.num_splits = p.num_splits;
  ca.chunk = p.chunk;
  ca.span = d.max_ctx;
  ca.part_splits = p.part_splits;
  ca.header = c.header;
  ca.out = static_cast<uint16_t*>(out);
  ca.lse = lse;
  ag = AggregateArgs{d.batch,  d.num_q_heads,         d.num_kv_heads, d.max_ctx, (int32_t)layout,
                     num_rows, accumulate ? 1 : 0, logits,          seq_lens,  scores};
  return VGSA_OK;
}

}  // namespace

extern "C" {

vgsa_status vgsa_verify_finish(const vgsa_attn_desc* desc, const int32_t* seq_lens,
                               const void* workspace, size_t workspace_bytes, void* out, float* lse,
                               vgsa_logit_layout layout, int32_t num_rows, int32_t accumulate,
                               const float* logits, float* scores, void* stream) {
  CombineArgs ca;
  AggregateArgs ag;
  const vgsa_status st = finish_args(desc, seq_lens, workspace, workspace_bytes, out, lse, layout,
                                     num_rows, accumulate, logits, scores, ca, ag);
  if (st != VGSA_OK) return st;
  if (ca.rows == 0) return VGSA_OK;
  return hip_status(launch_combine_aggregate(ca, ag, static_cast<hipStream_t>(stream)));
}

size_t vgsa_finish_select_workspace_bytes(int32_t batch, int32_t max_ctx) {
  if (batch < 1 || batch > kMaxGridYZ || max_ctx < 1 || max_ctx > kFinishSelectMaxCtx) return 0;
  return finish_select_workspace_bytes(batch, max_ctx);
}

vgsa_status vgsa_verify_finish_select(const vgsa_attn_desc* desc, const int32_t* seq_lens,
                                      const void* workspace, size_t workspace_bytes, void* out,
                                      float* lse, vgsa_logit_layout layout, int32_t num_rows,
                                      int32_t accumulate, const float* logits, float* scores,
                                      int32_t k, int32_t n_sink, int32_t window, int32_t* idx,
                                      int32_t idx_stride, int32_t* n_idx, void* select_workspace,
                                      size_t select_workspace_bytes, void* stream) {
  if (scores == nullptr) return VGSA_ERR_INVALID_ARG;
  if (k < 1 || n_sink < 0 || window < 0 || (int64_t)n_sink + window > k) return VGSA_ERR_INVALID_ARG;
  if (idx_stride < k || idx == nullptr || n_idx == nullptr) return VGSA_ERR_INVALID_ARG;
  CombineArgs ca;
  AggregateArgs ag;
  vgsa_status st = finish_args(desc, seq_lens, workspace, workspace_bytes, out, lse, layout,
                               num_rows, accumulate, logits, scores, ca, ag);
  if (st != VGSA_OK) return st;
  if (desc->max_ctx > kFinishSelectMaxCtx || desc->batch > kMaxGridYZ) return VGSA_ERR_UNSUPPORTED;
  if ((int64_t)desc->batch * idx_stride > 0x7fffffff) return VGSA_ERR_UNSUPPORTED;
  if (ca.rows == 0) return VGSA_OK;
  st = check_workspace(select_workspace, select_workspace_bytes,
                       finish_select_workspace_bytes(desc->batch, desc->max_ctx));
  if (st != VGSA_OK) return st;
  return hip_status(launch_finish_select(ca, ag, k, n_sink, window, idx, idx_stride, n_idx,
                                         select_workspace, static_cast<hipStream_t>(stream)));
}

vgsa_status vgsa_aggregate_scores(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t max_ctx, vgsa_logit_layout layout, int32_t num_rows,
                                  int32_t accumulate, const float* logits,
                                  const int32_t* seq_lens, float* scores, void* stream) {
  if (batch < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_ctx < 1) return VGSA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return VGSA_ERR_INVALID_ARG;
  if (layout != VGSA_LOGITS_PER_HEAD && layout != VGSA_LOGITS_KVGROUP_SUM)
    return VGSA_ERR_INVALID_ARG;
  if (layout == VGSA_LOGITS_PER_HEAD && (num_rows < 1 || num_rows > (int64_t)16 * num_q_heads))
    return VGSA_ERR_INVALID_ARG;
  if (logits == nullptr || seq_lens == nullptr || scores == nullptr) return VGSA_ERR_INVALID_ARG;
  if (batch > kMaxGridYZ) return VGSA_ERR_UNSUPPORTED;
  if (batch == 0) return VGSA_OK;
  return hip_status(launch_aggregate(batch, num_q_heads, num_kv_heads, max_ctx, layout, num_rows,
                                     accumulate ? 1 : 0, logits, seq_lens, scores,
                                     static_cast<hipStream_t>(stream)));
}

vgsa_status vgsa_select_topk(int32_t batch, int32_t max_ctx, const float* scores,
                             const int32_t* seq_lens, int32_t k, int32_t n_sink, int32_t window,
                             int32_t* idx, int32_t idx_stride, int32_t* n_idx, void* stream) {
  if (batch < 0 || max_ctx < 1 || k < 1 || n_sink < 0 || window < 0) return VGSA_ERR_INVALID_ARG;
  if ((int64_t)n_sink + window > k) return VGSA_ERR_INVALID_ARG;
  if (idx_stride < k) return VGSA_ERR_INVALID_ARG;
  if (scores == nullptr || seq_lens == nullptr || idx == nullptr || n_idx == nullptr)
    return VGSA_ERR_INVALID_ARG;
  if (batch == 0) return VGSA_OK;
  return hip_status(launch_select_topk(batch, max_ctx, scores, nullptr, seq_lens, k, 0, n_sink,
                                       window, idx, idx_stride, n_idx,
                                       static_cast<hipStream_t>(stream)));
}

size_t vgsa_select_workspace_bytes(int32_t batch, int32_t max_ctx) {
  if (batch < 1 || max_ctx < 1 || batch > kMaxGridYZ) return 0;
  return select_workspace_bytes(batch, max_ctx);
}

vgsa_status vgsa_select_topk_ws(int32_t batch, int32_t max_ctx, const float* scores,
                                const int32_t* seq_lens, int32_t k, int32_t n_sink,
                                int32_t window, int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const size_t need = vgsa_select_workspace_bytes(batch, max_ctx);
  if (need == 0)
    return vgsa_select_topk(batch, max_ctx, scores, seq_lens, k, n_sink, window, idx, idx_stride,
                            n_idx, stream);
  if (max_ctx < 1 || k < 1 || n_sink < 0 || window < 0) return VGSA_ERR_INVALID_ARG;
  if ((int64_t)n_sink + window > k) return VGSA_ERR_INVALID_ARG;
  if (idx_stride < k) return VGSA_ERR_INVALID_ARG;
  if (scores == nullptr || seq_lens == nullptr || idx == nullptr || n_idx == nullptr)
    return VGSA_ERR_INVALID_ARG;
  const vgsa_status st = check_workspace(workspace, workspace_bytes, need);
  if (st != VGSA_OK) return st;
  return hip_status(launch_select_topk_split(batch, max_ctx, scores, nullptr, seq_lens, k, 0,
                                             n_sink, window, idx, idx_stride, n_idx, workspace,
                                             static_cast<hipStream_t>(stream)));
}

vgsa_status vgsa_select_topk_hybrid_ws(int32_t batch, int32_t max_ctx, const float* target_scores,
                                       const float* draft_scores, const int32_t* seq_lens,
                                       int32_t k, int32_t m, int32_t n_sink, int32_t window,
                                       int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  const size_t need = vgsa_select_workspace_bytes(batch, max_ctx);
  if (need == 0)
    return vgsa_select_topk_hybrid(batch, max_ctx, target_scores, draft_scores, seq_lens, k, m,
                                   n_sink, window, idx, idx_stride, n_idx, stream);
  if (max_ctx < 1 || k < 1 || m < 0 || n_sink < 0 || window < 0) return VGSA_ERR_INVALID_ARG;
  if ((int64_t)n_sink + window > k) return VGSA_ERR_INVALID_ARG;
  if (idx_stride < k) return VGSA_ERR_INVALID_ARG;
  if (target_scores == nullptr || draft_scores == nullptr || seq_lens == nullptr ||
      idx == nullptr || n_idx == nullptr)
    return VGSA_ERR_INVALID_ARG;
  const vgsa_status st = check_workspace(workspace, workspace_bytes, need);
  if (st != VGSA_OK) return st;
  return hip_status(launch_select_topk_split(batch, max_ctx, target_scores, draft_scores,
                                             seq_lens, k, m, n_sink, window, idx, idx_stride,
                                             n_idx, workspace, static_cast<hipStream_t>(stream)));
}

vgsa_status vgsa_select_topk_hybrid(int32_t batch, int32_t max_ctx, const float* target_scores,
                                    const float* draft_scores, const int32_t* seq_lens, int32_t k,
                                    int32_t m, int32_t n_sink, int32_t window, int32_t* idx,
                                    int32_t idx_stride, int32_t* n_idx, void* stream) {
  if (batch < 0 || max_ctx < 1 || k < 1 || m < 0 || n_sink < 0 || window < 0)
    return VGSA_ERR_INVALID_ARG;
  if ((int64_t)n_sink + window > k) return VGSA_ERR_INVALID_ARG;
  if (idx_stride < k) return VGSA_ERR_INVALID_ARG;
  if (target_scores == nullptr || draft_scores == nullptr || seq_lens == nullptr ||
      idx == nullptr || n_idx == nullptr)
    return VGSA_ERR_INVALID_ARG;
  if (max_ctx > kMaxHybridRow) return VGSA_ERR_UNSUPPORTED;
  if (batch == 0) return VGSA_OK;
  return hip_status(launch_select_topk(batch, max_ctx, target_scores, draft_scores, seq_lens, k,
                                       m, n_sink, window, idx, idx_stride, n_idx,
                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

vgsa_status select_blocks_call(int32_t batch, int32_t max_ctx, const float* scores,
                               const int32_t* seq_lens, int32_t k_blocks, int32_t block,
                               int32_t n_sink, int32_t window, int32_t* out, int32_t out_stride,
                               int32_t* n_out, float* block_sums, bool ids, void* stream) {
  if (batch < 0 || max_ctx < 1 || k_blocks < 1 || block < 1 || block > kMaxIdBlock || n_sink < 0 ||
      window < 0)
    return VGSA_ERR_INVALID_ARG;
  // the sink blocks and (at most ceil(window / block) + 1) window blocks fit the budget
  const int64_t forced = ((int64_t)n_sink + block - 1) / block +
                         (window > 0 ? ((int64_t)window + block - 1) / block + 1 : 0);
  if (forced > k_blocks) return VGSA_ERR_INVALID_ARG;
  if ((int64_t)out_stride < (int64_t)k_blocks * (ids ? 1 : block)) return VGSA_ERR_INVALID_ARG;
  if (scores == nullptr || seq_lens == nullptr || out == nullptr || n_out == nullptr)
    return VGSA_ERR_INVALID_ARG;
  if (((int64_t)max_ctx + block - 1) / block > kMaxSelBlocks) return VGSA_ERR_UNSUPPORTED;
  if (batch == 0) return VGSA_OK;
  return hip_status(launch_select_blocks(batch, max_ctx, scores, seq_lens, k_blocks, block, n_sink,
                                         window, out, out_stride, n_out, block_sums, ids,
                                         static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

vgsa_status vgsa_select_blocks(int32_t batch, int32_t max_ctx, const float* scores,
                               const int32_t* seq_lens, int32_t k_blocks, int32_t block,
                               int32_t n_sink, int32_t window, int32_t* idx, int32_t idx_stride,
                               int32_t* n_idx, float* block_sums, void* stream) {
  return select_blocks_call(batch, max_ctx, scores, seq_lens, k_blocks, block, n_sink, window, idx,
                            idx_stride, n_idx, block_sums, false, stream);
}

vgsa_status vgsa_select_block_ids(int32_t batch, int32_t max_ctx, const float* scores,
                                  const int32_t* seq_lens, int32_t k_blocks, int32_t block,
                                  int32_t n_sink, int32_t window, int32_t* block_ids,
                                  int32_t ids_stride, int32_t* n_ids, float* block_sums,
                                  void* stream) {
  return select_blocks_call(batch, max_ctx, scores, seq_lens, k_blocks, block, n_sink, window,
                            block_ids, ids_stride, n_ids, block_sums, true, stream);
}

vgsa_status vgsa_append_positions(int32_t batch, const int32_t* base, int32_t first, int32_t count,
                                  int32_t* idx, int32_t idx_stride, int32_t* n_idx, void* stream) {
  if (batch < 0 || first < 0 || count < 0 || idx_stride < 1) return VGSA_ERR_INVALID_ARG;
  if (batch == 0 || count == 0) return VGSA_OK;
  if (base == nullptr || idx == nullptr || n_idx == nullptr) return VGSA_ERR_INVALID_ARG;
  if (batch > 0x7fffffff / idx_stride) return VGSA_ERR_UNSUPPORTED;
  return hip_status(launch_append_positions(batch, base, first, count, idx, idx_stride, n_idx,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
