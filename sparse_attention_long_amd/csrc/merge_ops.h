// Device-side pieces shared by the combine, aggregate and fused kernels.
#pragma once

#include "internal.h"

namespace vgsa {

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP moves: row
// shifts by 1, 2, 4, 8 (zero fill) scan each 16-lane row, then the last lane
// of row 0 / row 2 is added to row 1 / row 3 and the last lane of row 1 to
// rows 2 and 3; lane 63 holds the total.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return (uint32_t)v;
}
// Sum of x over the 64 lanes, the same value in every lane.
__device__ __forceinline__ uint32_t wave_total(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(x), 63);
}

// Threads of a combine / aggregate workgroup.
constexpr int kMergeBlock = 256;

// 16- and 8-byte accesses at device scope for partial results exchanged
// inside one launch: the SC1 cache-policy bit makes a store write through, and
// a load read past, the issuing XCD's L2, so another XCD sees the data without
// a cache-wide write-back.  Buffer instructions take a wave-uniform base (the
// partial array) and a 32-bit byte offset (the host keeps these arrays below
// 2 GiB); the resource word is the gfx9 raw-buffer one.
constexpr int kCpolSc1 = 16;
constexpr int kRawBufferWord3 = 0x00020000;
typedef uint32_t u32x4m __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2m __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t device_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7fffffff, kRawBufferWord3);
}
__device__ __forceinline__ void store4_device(float* base, uint32_t byte_off, float4 v) {
  const u32x4m u = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(u, device_rsrc(base), byte_off, 0, kCpolSc1);
}
__device__ __forceinline__ void store2_device(float* base, uint32_t byte_off, float2 v) {
  const u32x2m u = {__float_as_uint(v.x), __float_as_uint(v.y)};
  __builtin_amdgcn_raw_buffer_store_b64(u, device_rsrc(base), byte_off, 0, kCpolSc1);
}
__device__ __forceinline__ float4 load4_device(const float* base, uint32_t byte_off) {
  const u32x4m u = __builtin_amdgcn_raw_buffer_load_b128(device_rsrc(base), byte_off, 0, kCpolSc1);
  return make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]),
                     __uint_as_float(u[3]));
}
__device__ __forceinline__ float2 load2_device(const float* base, uint32_t byte_off) {
  const u32x2m u = __builtin_amdgcn_raw_buffer_load_b64(device_rsrc(base), byte_off, 0, kCpolSc1);
  return make_float2(__uint_as_float(u[0]), __uint_as_float(u[1]));
}
__device__ __forceinline__ float load1_device(const float* base, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(device_rsrc(base), byte_off, 0, kCpolSc1));
}
__device__ __forceinline__ void store1_device(float* base, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), device_rsrc(base), byte_off, 0, kCpolSc1);
}

// Splits (or logit rows) whose loads are issued together before any is used:
// the merge is a chain of dependent HBM round trips otherwise.
constexpr int kMergeBatch = 8;

// Exact merge of the split partials of four output elements (row of
// [B][Hq][T], columns 4t..4t+3): m = max_s m_s, l = sum_s l_s 2^(m_s - m),
// o = sum_s o_s 2^(m_s - m) / l, lse = ln 2 * (m + log2 l).  The m_s are in
// log2 units.  Splits at or past the sequence's length hold nothing; a split
// the row sees nothing of has m_s = -inf and is skipped.  Splits are merged
// kMergeBatch at a time, each batch rescaled to its running maximum, in split
// order (with at most kMergeBatch splits this is the plain two-pass sum).
// `chunk`: the item length the partials were made with.  COHERENT: the
// partials were written in the same launch by other workgroups (possibly on
// another XCD, whose L2 this one's does not see): read them with device-scope
// loads, which bypass stale cache lines.
// `entries` >= 0: the number of entries the partials cover (given by a caller
// that has it); otherwise min(lengths[b], span) + tail.
template <int D, bool COHERENT = false>
__device__ __forceinline__ void combine_quad(const CombineArgs& a, int row, int t, int chunk,
                                             int entries = -1) {
  constexpr float kNegInf = -__builtin_huge_valf();
  constexpr int Q = D / 4;
  const int b = row / a.rows_per_seq;
  const int len = entries >= 0 ? entries : min(max(a.lengths[b], 0), a.span) + a.tail;
  const int nvalid = min((len + chunk - 1) / chunk, a.part_splits);
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + (size_t)row * a.part_splits;
  const float4* po = reinterpret_cast<const float4*>(a.part_o) + (size_t)row * a.part_splits * Q + t;
  float M = kNegInf, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nvalid; s0 += kMergeBatch) {
    float2 m[kMergeBatch];
    float4 o[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (s0 + i < nvalid) {
        if (COHERENT) {
          const size_t ps = (size_t)row * a.part_splits + s0 + i;  // partial row of split s0 + i
          m[i] = load2_device(a.part_ml, (uint32_t)(ps * 8));
          o[i] = load4_device(a.part_o, (uint32_t)((ps * Q + t) * 16));
        } else {
          m[i] = ml[s0 + i];
          o[i] = po[(size_t)(s0 + i) * Q];
        }
      } else {
        m[i] = make_float2(kNegInf, 0.f);
        o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float mc = M;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) mc = fmaxf(mc, m[i].x);
    if (mc == kNegInf) continue;
    const float r = __builtin_amdgcn_exp2f(M - mc);  // 0 while nothing was merged
    l *= r;
    acc.x *= r; acc.y *= r; acc.z *= r; acc.w *= r;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (m[i].x == kNegInf) continue;  // also skips unused slots of the batch
      const float w = __builtin_amdgcn_exp2f(m[i].x - mc);
      l += w * m[i].y;
      acc.x += w * o[i].x; acc.y += w * o[i].y; acc.z += w * o[i].z; acc.w += w * o[i].w;
    }
    M = mc;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)(acc.x * inv)) |
                      (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.y * inv)) << 16;
  const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)(acc.z * inv)) |
                      (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.w * inv)) << 16;
  reinterpret_cast<uint2*>(a.out)[(size_t)row * Q + t] = make_uint2(lo, hi);
  if (a.lse != nullptr && t == 0)
    a.lse[row] = l > 0.f ? (M + __log2f(l)) * 0.69314718055994530942f : kNegInf;
}

// One workgroup of kMergeBlock threads combines kMergeBlock / (D / 4) rows.
template <int D>
__device__ __forceinline__ void combine_block(const CombineArgs& a, int block) {
  constexpr int Q = D / 4;
  const int row = block * (kMergeBlock / Q) + threadIdx.x / Q;
  // the item length the partials were made with (clamped: the header only
  // ever narrows the plan's chunk)
  const int chunk = min(max(a.header[0], kTile), a.chunk);
  if (row < a.rows) combine_quad<D>(a, row, threadIdx.x % Q, chunk);
}

template <int D>
constexpr int combine_blocks(int rows) {
  return (rows + kMergeBlock / (D / 4) - 1) / (kMergeBlock / (D / 4));
}

// Score of position j < L of sequence b (returned, not stored): the
// collected logits summed in a fixed order (kv-groups ascending, or rows then
// heads ascending), then added to the score already there when accumulating
// (e.g. over layers).
// U positions j0 + u * stride at once (those at or past L give 0), their
// loads issued together.
template <int U>
__device__ __forceinline__ void aggregate_values(const AggregateArgs& a, int b, int j0, int stride,
                                                 int L, float (&res)[U]) {
  const int n = a.layout == VGSA_LOGITS_KVGROUP_SUM ? a.hkv : a.n_rows;
  const float* p = a.logits + (size_t)b * n * a.max_ctx;
  float s[U];
#pragma unroll
  for (int u = 0; u < U; ++u) s[u] = 0.f;
  for (int r0 = 0; r0 < n; r0 += kMergeBatch) {
    float v[U][kMergeBatch];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const int j = j0 + u * stride;
        v[u][i] = (r0 + i < n && j < L) ? p[(size_t)(r0 + i) * a.max_ctx + j] : 0.f;
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i)
        if (r0 + i < n) s[u] += v[u][i];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = j0 + u * stride;
    res[u] = (a.accumulate && j < L) ? a.scores[(size_t)b * a.max_ctx + j] + s[u] : s[u];
  }
}

__device__ __forceinline__ float aggregate_value(const AggregateArgs& a, int b, int j) {
  float v[1];
  aggregate_values<1>(a, b, j, 0, j + 1, v);
  return v[0];
}

__device__ __forceinline__ void aggregate_position(const AggregateArgs& a, int b, int j) {
  const int L = min(max(a.seq_lens[b], 0), a.max_ctx);
  if (j >= L) return;
  a.scores[(size_t)b * a.max_ctx + j] = aggregate_value(a, b, j);
}

}  // namespace vgsa
