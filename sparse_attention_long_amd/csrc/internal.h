// Internal declarations shared by the HIP sources of the library (not part
// of the C ABI).  Host-side launchers take already-validated arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "vgsa.h"

namespace vgsa {

// Positions one wavefront processes per step.
constexpr int kTile = 32;
// Launch layouts of the attention kernels.  Wide: one workgroup of 8
// wavefronts per CU (two per SIMD), every workgroup the same age on its CU.
// Two 4-wavefront workgroups sharing a CU ran at different speeds: the SIMD
// arbiter favours the older wavefronts, so the workgroup dispatched second
// looped 7-8 % longer and set the verify kernel's end.  Narrow: 4
// wavefronts, for d = 128 with four 16-row blocks, whose registers allow one
// wavefront per SIMD.
constexpr int kWaves = 4;
constexpr int kWavesWide = 8;
// Smallest chunk a workgroup is given (one step of every wavefront).
constexpr int kMinChunk = kTile * kWaves;
constexpr int kMinChunkWide = kTile * kWavesWide;
// Workgroups aimed for per attention launch: one round on 256 CUs (wide: one
// per CU; narrow: two per CU), so each workgroup slot pays its start-up and
// merge once.
constexpr int kTargetWorkgroups = 512;
constexpr int kTargetWorkgroupsWide = 256;
// Spans up to this many positions get one split: a single workgroup per
// (sequence, kv-head) finishes the softmax itself and writes the output
// directly (no partials, no combine launch).
constexpr int kDirectSpan = 1024;
// Chunk of one split, as planned.  A workgroup keeps the kv-group logits of
// its chunk in LDS (fp32) and writes them out after its loop (narrow paged
// launches hold kLogitBuf positions and flush whenever the buffer is full).
// Narrow: 8192 positions (longer chunks measured slower at 128K x b8: one
// round of 512 workgroups then spans 4 GB of K/V at once).  Wide: 16384, the
// same bytes per CU.
constexpr int kPlanChunk = 8192;
constexpr int kPlanChunkWide = 16384;
// Largest chunk: the plan widens its chunks up to this size instead of adding
// a split for a last sliver (a capacity a few positions past a multiple of
// the planned chunk, e.g. headroom for drafted tokens): up to kPlanChunk / 8
// positions (narrow) or one step of every wavefront (wide, whose LDS logit
// buffer holds exactly this many positions).
constexpr int kMaxChunk = kPlanChunk + kPlanChunk / 8;
constexpr int kMaxChunkWide = kPlanChunkWide + kMinChunkWide;
constexpr int kLogitBuf = 4096;     // narrow paged caches (the block-id table shares the space)
constexpr int kLogitBufMax = 8192;  // narrow contiguous caches: a whole planned chunk
// Largest (Hq/Hkv) * T handled by one workgroup: four 16-row MFMA blocks.
constexpr int kMaxRows = 64;

struct SplitPlan {
  int32_t num_splits;
  int32_t chunk;
  int32_t part_splits;  // row stride of the partial arrays: num_splits, or
                        // kBalanceSplits * num_splits when items may shrink
  int32_t waves;        // kWavesWide, or kWaves for d = 128 with four row blocks
};

// Wavefronts per attention workgroup for this shape (wide unless d = 128 with
// more than three 16-row blocks).
inline int attention_waves(const vgsa_attn_desc& d) {
  const int64_t rows = (int64_t)(d.num_q_heads / d.num_kv_heads) * d.q_len;
  return (d.head_dim == 128 && rows > 48) ? kWaves : kWavesWide;
}

// Ragged batches: a verify launch over several sequences (at most
// kMaxBalanceBatch) shrinks its items so that the non-empty ones fill the
// grid (see attn_partials_kernel); an item is never shorter than
// chunk / kBalanceSplits, so the partials hold kBalanceSplits times the splits.
constexpr int kBalanceSplits = 4;
constexpr int kMaxBalanceBatch = 256;

// Split plan of an attention launch over `span` positions (the capacity for
// verify, the list capacity plus tail for sparse) for this shape.
SplitPlan make_plan(const vgsa_attn_desc& d, int32_t span);

// Partial results of one attention launch, carved out of the workspace:
//   header  int32 [64]               [0]: the item length the launch used
//   part_o  fp32 [B][Hq][T][P][d]    un-normalised sum of p * v of the item
//   part_ml fp32 [B][Hq][T][P][2]    (running max m in log2 units, sum l)
// with P = part_splits.
constexpr size_t kHeaderBytes = 256;
size_t partial_bytes(const vgsa_attn_desc& d, const SplitPlan& p);

// Head mask value that collects every q-head (any head count).
constexpr uint64_t kAllHeads = ~0ull;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* idx;    // sparse only
  const int32_t* n_idx;  // sparse only
  int32_t idx_stride;
  int32_t tail;          // sparse: the last `tail` positions below the length follow the list
  int32_t id_block;      // sparse: positions per list entry (1: positions; B > 1: block ids,
                         // entry i covering positions B*i .. B*i + B - 1)
  float* logits;         // verify only, may be null
  int32_t layout;
  uint32_t row_mask;  // collected rows: bit t set for query row t
  int32_t n_rows;     // popcount(row_mask): collected rows per sequence
  uint64_t head_mask; // collected q-heads: bit h for head h, or kAllHeads
  int32_t n_heads;    // collected q-heads (PER_HEAD head rows per collected row)
  float* part_o;
  float* part_ml;
  int32_t* header;   // the launch records its item length in header[0]
  int32_t part_splits;
  int32_t balance;   // shrink items to the lengths (verify, several sequences)
  uint16_t* out;     // direct mode (one split) or fused merge: final bf16 output ...
  float* lse;        // ... and lse (may be null)
  int32_t direct;
  // Fused merge (sparse, several splits): the last workgroup of a (sequence,
  // kv-head) to finish merges the splits' partials into out / lse.  sync[b *
  // hkv + g] counts the finished workgroups; zero before the launch, and the
  // merging workgroup sets it back to zero.
  int32_t* sync;
  int32_t fuse;
  int32_t batch, hq, hkv, group, q_len, head_dim;
  int32_t max_ctx, paged, max_blocks, num_blocks;
  int32_t num_splits, chunk;
  int32_t waves;     // wavefronts per workgroup (the plan's layout)
  // Sparse, one split: the G*T query rows of a (sequence, kv-head) are shared
  // by this many workgroups (1 or 2), each gathering every listed K/V row.
  // The two run on one XCD (linear ids x + 8*(2j) and x + 8*(2j + 1)), so the
  // second read of a row is served by that XCD's L2.
  int32_t row_split;
  float scale;       // natural-log softmax scale
  float scale_log2;  // scale * log2(e)
};

hipError_t launch_attention_partials(const AttnArgs& a, bool sparse, hipStream_t stream);

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  const int32_t* lengths;
  int32_t rows;  // B * Hq * T
  int32_t rows_per_seq;  // Hq * T
  int32_t head_dim;
  int32_t num_splits, chunk, span;
  int32_t part_splits;    // row stride of the partials
  const int32_t* header;  // header[0]: the item length the partials were made with
  uint16_t* out;
  float* lse;
  int32_t tail;           // entries after lengths[b] (sparse trailing positions)
};

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

struct AggregateArgs {
  int32_t batch, hq, hkv, max_ctx, layout;
  int32_t n_rows;      // PER_HEAD: logit rows per sequence (rows x heads collected)
  int32_t accumulate;  // add the sum to scores instead of overwriting them
  const float* logits;
  const int32_t* seq_lens;
  float* scores;
};

// Combine and (when ag.scores != null) aggregate in one launch.
hipError_t launch_combine_aggregate(const CombineArgs& c, const AggregateArgs& ag,
                                    hipStream_t stream);

hipError_t launch_aggregate(int32_t batch, int32_t hq, int32_t hkv, int32_t max_ctx, int32_t layout,
                            int32_t n_rows, int32_t accumulate,
                            const float* logits, const int32_t* seq_lens, float* scores,
                            hipStream_t stream);

hipError_t launch_append_positions(int32_t batch, const int32_t* base, int32_t first, int32_t count,
                                   int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                                   hipStream_t stream);
// draft_scores non-null: hybrid selection (m positions by draft_scores
// first); rows longer than the one-workgroup kernel's limit are then refused.
hipError_t launch_select_topk(int32_t batch, int32_t max_ctx, const float* scores,
                              const float* draft_scores, const int32_t* seq_lens, int32_t k,
                              int32_t m, int32_t n_sink, int32_t window, int32_t* idx,
                              int32_t idx_stride, int32_t* n_idx, hipStream_t stream);
// Rows of 2 .. 8 rounds of 32768 positions with a workspace: one workgroup
// per round in three launches (select_workspace_bytes is 0 for other rows).
size_t select_workspace_bytes(int32_t batch, int32_t max_ctx);
// draft_scores non-null: hybrid selection (m positions by draft_scores first).
hipError_t launch_select_topk_split(int32_t batch, int32_t max_ctx, const float* scores,
                                    const float* draft_scores, const int32_t* seq_lens, int32_t k,
                                    int32_t m, int32_t n_sink, int32_t window, int32_t* idx,
                                    int32_t idx_stride, int32_t* n_idx, void* workspace,
                                    hipStream_t stream);
// Longest row (positions) the hybrid selection takes.
constexpr int kMaxHybridRow = 8 * 32768;
// Block-granular selection: blocks per row (their sums live in LDS).
constexpr int kMaxSelBlocks = 8704;
// Combine + aggregate + select in one launch (rows of max_ctx <= 262144; the
// workspace holds per-row key histograms and arrival counts, zero between
// calls).
constexpr int kFinishSelectMaxCtx = 262144;
size_t finish_select_workspace_bytes(int32_t batch, int32_t max_ctx);
hipError_t launch_finish_select(const CombineArgs& c, const AggregateArgs& ag, int32_t k,
                                int32_t n_sink, int32_t window, int32_t* idx, int32_t idx_stride,
                                int32_t* n_idx, void* workspace, hipStream_t stream);
hipError_t launch_select_blocks(int32_t batch, int32_t max_ctx, const float* scores,
                                const int32_t* seq_lens, int32_t k_blocks, int32_t block,
                                int32_t n_sink, int32_t window, int32_t* idx, int32_t idx_stride,
                                int32_t* n_idx, float* block_sums, bool ids, hipStream_t stream);

}  // namespace vgsa
