// Top-k selection of the positions kept for the next step.
//
// Vegas (gist.science 2602.07223), "A. aggregated attention-logit selection":
// the kept set T, |T| = k, maximises the summed logits of its members; the
// objective is a sum of per-position scores, so T is a top-k of the scores.
// Dustin (gist.science 2606.24957), "1. hybrid attention aggregation": a few
// attention-sink prefix positions and a window of recent positions are kept
// first and the remaining budget is filled by score.
//
// One workgroup of 1024 threads per sequence:
//   1. F = [0, s_end) U [w_start, L) is forced; r = k - |F| positions are
//      picked from the middle range M = [s_end, w_start).
//   2. Radix select over order-preserving 32-bit keys (digits of 12, 12 and 8
//      bits, histograms in LDS) finds the key `thr` of the r-th largest score
//      in M and how many keys equal to `thr` are needed.
//   3. An ordered compaction (block-wide scans) writes F, every key above thr,
//      and the lowest-positioned keys equal to thr, in ascending position
//      order.  Everything is integer arithmetic, so the result is exact and
//      deterministic.
#include "internal.h"

namespace vgsa {
namespace {

constexpr int kThreadsTk = 1024;
constexpr int kWavesTk = kThreadsTk / 64;
constexpr int kBins = 4096;

// Larger score -> larger key; -0.0 and +0.0 share one key.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the workgroup; `total` receives the sum.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWavesTk; ++w) {
    const uint32_t c = s_wave[w];
    base += (w < wave) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

__global__ __launch_bounds__(kThreadsTk) void select_topk_kernel(
    int32_t max_ctx, const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    int32_t k, int32_t n_sink, int32_t window, int32_t* __restrict__ idx, int32_t idx_stride,
    int32_t* __restrict__ n_idx) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t s_wave[kWavesTk];
  __shared__ uint32_t s_prefix, s_want;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = min(max(seq_lens[b], 0), max_ctx);
  int32_t* out = idx + (size_t)b * idx_stride;
  const float* sc = scores + (size_t)b * max_ctx;

  if (L <= k) {
    for (int j = tid; j < L; j += kThreadsTk) out[j] = j;
    if (tid == 0) n_idx[b] = L;
    return;
  }
  const int s_end = min(n_sink, L);
  const int w_start = max(s_end, L - window);
  const int r = k - (s_end + (L - w_start));  // >= 0: n_sink + window <= k is checked on the host

  uint32_t prefix = 0u, want = (uint32_t)r;
  if (r > 0) {
    // digits: bits [31:20], [19:8], [7:0]
    const int shifts[3] = {20, 8, 0};
    const int widths[3] = {12, 12, 8};
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = shifts[pass];
      const uint32_t nb = 1u << widths[pass];
      const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shifts[pass - 1]));
      for (int i = tid; i < kBins; i += kThreadsTk) hist[i] = 0u;
      __syncthreads();
      for (int j = s_end + tid; j < w_start; j += kThreadsTk) {
        const uint32_t key = order_key(sc[j]);
        if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1u)], 1u);
      }
      __syncthreads();
      // Thread t owns the 4 bins nb-1-4t .. nb-4-4t (descending); the
      // exclusive scan gives how many keys lie above its highest bin.
      uint32_t c[4] = {0u, 0u, 0u, 0u};
      const int top = (int)nb - 1 - 4 * tid;
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = (top - q >= 0) ? hist[top - q] : 0u;
      uint32_t tot;
      uint32_t above = block_exclusive_scan(c[0] + c[1] + c[2] + c[3], s_wave, tot);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (top - q >= 0 && above < want && want <= above + c[q]) {
          s_prefix = prefix | ((uint32_t)(top - q) << shift);
          s_want = want - above;
        }
        above += c[q];
      }
      __syncthreads();
      prefix = s_prefix;
      want = s_want;
      __syncthreads();
    }
  }
  const uint32_t thr = prefix;     // key of the r-th largest score in M
  const uint32_t need_eq = want;   // keys equal to thr that are kept (lowest positions first)

  // Ordered compaction over contiguous runs, one run per thread.
  const int run = (L + kThreadsTk - 1) / kThreadsTk;
  const int j0 = min(tid * run, L), j1 = min(j0 + run, L);
  uint32_t ceq = 0u;
  if (r > 0) {
    for (int j = max(j0, s_end); j < min(j1, w_start); ++j) ceq += order_key(sc[j]) == thr;
  }
  uint32_t tot;
  const uint32_t eq_base = block_exclusive_scan(ceq, s_wave, tot);

  auto keep = [&](int j, uint32_t& e) -> bool {
    if (j < s_end || j >= w_start) return true;
    if (r == 0) return false;
    const uint32_t key = order_key(sc[j]);
    if (key > thr) return true;
    if (key == thr) return e++ < need_eq;
    return false;
  };
  uint32_t e = eq_base, csel = 0u;
  for (int j = j0; j < j1; ++j) csel += keep(j, e);
  const uint32_t out_base = block_exclusive_scan(csel, s_wave, tot);
  e = eq_base;
  uint32_t o = out_base;
  for (int j = j0; j < j1; ++j)
    if (keep(j, e) && o < (uint32_t)idx_stride) out[o++] = j;
  if (tid == 0) n_idx[b] = (int32_t)tot;
}

}  // namespace

hipError_t launch_select_topk(int32_t batch, int32_t max_ctx, const float* scores,
                              const int32_t* seq_lens, int32_t k, int32_t n_sink, int32_t window,
                              int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                              hipStream_t stream) {
  hipLaunchKernelGGL(select_topk_kernel, dim3(batch), dim3(kThreadsTk), 0, stream, max_ctx, scores,
                     seq_lens, k, n_sink, window, idx, idx_stride, n_idx);
  return hipGetLastError();
}

}  // namespace vgsa
