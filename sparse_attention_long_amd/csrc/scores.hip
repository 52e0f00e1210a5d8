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

namespace vgsa {
namespace {

constexpr int kBlock = 256;

__global__ __launch_bounds__(kBlock) void aggregate_kernel(int32_t hq, int32_t hkv, int32_t max_ctx,
                                                           int32_t layout, const float* logits,
                                                           const int32_t* seq_lens, float* scores) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * kBlock + threadIdx.x;
  const int L = min(max(seq_lens[b], 0), max_ctx);
  if (j >= L) return;
  float s = 0.f;
  if (layout == VGSA_LOGITS_KVGROUP_SUM) {
    const float* p = logits + (size_t)b * hkv * max_ctx + j;
    for (int g = 0; g < hkv; ++g) s += p[(size_t)g * max_ctx];
  } else {
    const float* p = logits + (size_t)b * 2 * hq * max_ctx + j;
    for (int r = 0; r < 2 * hq; ++r) s += p[(size_t)r * max_ctx];
  }
  scores[(size_t)b * max_ctx + j] = s;
}

}  // namespace

hipError_t launch_aggregate(int32_t batch, int32_t hq, int32_t hkv, int32_t max_ctx, int32_t layout,
                            const float* logits, const int32_t* seq_lens, float* scores,
                            hipStream_t stream) {
  const dim3 grid((max_ctx + kBlock - 1) / kBlock, batch);
  hipLaunchKernelGGL(aggregate_kernel, grid, dim3(kBlock), 0, stream, hq, hkv, max_ctx, layout,
                     logits, seq_lens, scores);
  return hipGetLastError();
}

}  // namespace vgsa
