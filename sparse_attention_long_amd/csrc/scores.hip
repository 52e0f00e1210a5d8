// Score aggregation: one importance score per cached position.
//
// Vegas (gist.science 2602.07223), "A. aggregated attention-logit selection":
// the selected set maximises the sum over the draft/bonus rows and all query
// heads of the logits of its members, so each position's contribution is the
// sum of its collected logits.  The collected rows are the first draft token
// and the bonus token ("B. Collect-2-Query").
//
// One thread per (sequence, position); the sum runs in a fixed order (row,
// then head; or kv-group ascending), so results are deterministic.  The
// kernel is a coalesced streaming read, bound by HBM bandwidth.
#include "internal.h"
#include "merge_ops.h"

namespace vgsa {
namespace {

constexpr int kBlock = kMergeBlock;

__global__ __launch_bounds__(kBlock) void aggregate_kernel(AggregateArgs a) {
  aggregate_position(a, blockIdx.y, blockIdx.x * kBlock + threadIdx.x);
}

// Combine (the first n_combine workgroups) and aggregate (the rest, kBlock
// positions each, sequences in order) in one launch.
template <int D>
__global__ __launch_bounds__(kBlock) void combine_aggregate_kernel(CombineArgs c, AggregateArgs ag,
                                                                   int32_t n_combine,
                                                                   int32_t pos_blocks) {
  if ((int)blockIdx.x < n_combine) {
    combine_block<D>(c, blockIdx.x);
    return;
  }
  const int q = blockIdx.x - n_combine;
  aggregate_position(ag, q / pos_blocks, (q % pos_blocks) * kBlock + threadIdx.x);
}

// One workgroup per sequence: list entries n .. n + count - 1 (those below
// idx_stride) receive base + first + i; then the count grows.
__global__ __launch_bounds__(kBlock) void append_positions_kernel(const int32_t* base, int32_t first,
                                                                  int32_t count, int32_t* idx,
                                                                  int32_t idx_stride,
                                                                  int32_t* n_idx) {
  const int b = blockIdx.x;
  const int n = min(max(n_idx[b], 0), idx_stride);
  const int p0 = base[b] + first;
  for (int i = threadIdx.x; i < count && n + i < idx_stride; i += kBlock)
    idx[(size_t)b * idx_stride + n + i] = p0 + i;
  __syncthreads();  // every thread has read n_idx[b]
  if (threadIdx.x == 0) n_idx[b] = (int32_t)min((int64_t)n + count, (int64_t)idx_stride);
}

}  // namespace

hipError_t launch_append_positions(int32_t batch, const int32_t* base, int32_t first, int32_t count,
                                   int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(append_positions_kernel, dim3(batch), dim3(kBlock), 0, stream, base, first,
                     count, idx, idx_stride, n_idx);
  return hipGetLastError();
}

hipError_t launch_aggregate(int32_t batch, int32_t hq, int32_t hkv, int32_t max_ctx, int32_t layout,
                            int32_t n_rows, int32_t accumulate, const float* logits,
                            const int32_t* seq_lens,
                            float* scores, hipStream_t stream) {
  AggregateArgs a{batch, hq, hkv, max_ctx, layout, n_rows, accumulate, logits, seq_lens, scores};
  const dim3 grid((max_ctx + kBlock - 1) / kBlock, batch);
  hipLaunchKernelGGL(aggregate_kernel, grid, dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine_aggregate(const CombineArgs& c, const AggregateArgs& ag,
                                    hipStream_t stream) {
  const int n_combine = c.head_dim == 64 ? combine_blocks<64>(c.rows) : combine_blocks<128>(c.rows);
  const int pos_blocks = ag.scores ? (ag.max_ctx + kBlock - 1) / kBlock : 0;
  const int64_t total = (int64_t)n_combine + (int64_t)pos_blocks * (ag.scores ? ag.batch : 0);
  if (total <= 0) return hipSuccess;
  if (c.head_dim == 64) {
    hipLaunchKernelGGL(combine_aggregate_kernel<64>, dim3((unsigned)total), dim3(kBlock), 0, stream,
                       c, ag, n_combine, pos_blocks);
  } else {
    hipLaunchKernelGGL(combine_aggregate_kernel<128>, dim3((unsigned)total), dim3(kBlock), 0,
                       stream, c, ag, n_combine, pos_blocks);
  }
  return hipGetLastError();
}

}  // namespace vgsa
