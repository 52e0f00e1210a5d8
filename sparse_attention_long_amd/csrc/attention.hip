// Split-KV attention for the verify pass and for the index-gather sparse pass,
// plus the log-sum-exp combine of the splits.
//
// What is computed (Vegas, gist.science 2602.07223):
//   * section 2 "core mechanism", step 1: the verify rows attend with full
//     attention over every cached position;
//   * "B. Collect-2-Query" and section 3 "implementation": the logits of two
//     rows (first draft token, bonus token) are written to HBM before softmax
//     normalisation -- here straight from the MFMA accumulators, before any
//     rescaling, so nothing extra is held on chip;
//   * section 2 step 3 and section 3: the sparse pass attends only over listed
//     positions, the list acting as a page-size-1 page table.
//
// Layout of the work: one workgroup per (split, kv-head, sequence); its four
// wavefronts take 32-position tiles of the split in turn.  All G*T query rows
// that share the kv-head live in one wavefront as 16-row MFMA blocks, so every
// K/V byte is read from HBM once.  Per tile a wavefront:
//   1. loads 32 K rows and 32 V rows with 16-byte loads (prefetched one tile
//      ahead in registers),
//   2. computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (positions are the
//      M side, query rows the N side),
//   3. writes the collected logits (per head, or summed over the kv-group),
//   4. runs an online softmax in log2 units per query row,
//   5. accumulates O^T += V^T P^T with the same MFMA; P comes straight from
//      the S^T accumulators, V^T is read from a per-wavefront LDS tile.
// The four wavefronts are merged through LDS at the end and the workgroup
// writes its un-normalised partial (o, m, l) for the combine kernel.
#include "internal.h"

namespace vgsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ bf16x8 load16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
__device__ __forceinline__ size_t kv_row(const AttnArgs& a, int b, int g, int pos) {
  if (a.paged) {
    int blk = a.block_table[(size_t)b * a.max_blocks + (pos >> 4)];
    blk = min(max(blk, 0), a.num_blocks - 1);
    return (((size_t)blk * a.hkv + g) * 16 + (pos & 15)) * D;
  }
  return (((size_t)b * a.hkv + g) * a.max_ctx + pos) * D;
}

// D: head dim (64/128); QB: 16-row query blocks (G*T <= 16*QB); SPARSE: index list.
template <int D, int QB, bool SPARSE>
__global__ __launch_bounds__(kThreads) void attn_partials_kernel(AttnArgs a) {
  constexpr int KS = D / 32;       // MFMA steps over the head dimension
  constexpr int DB = D / 16;       // 16-wide blocks of the head dimension
  constexpr int VS = D + 4;        // padded LDS row, in elements (breaks bank aliasing)
  // V tiles of the four wavefronts; reused at the end as the fp32 merge
  // buffer [64][D + 4] (both are 256 * (D + 4) bytes).
  __shared__ __align__(16) uint16_t sbuf[kWaves * kTile * VS];
  __shared__ float s_m[kWaves][kMaxRows];
  __shared__ float s_l[kWaves][kMaxRows];
  __shared__ int s_idx[kWaves][kTile];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, kg = lane >> 4;

  const int L = min(max(a.seq_lens[b], 0), a.max_ctx);
  const int count = SPARSE ? min(max(a.n_idx[b], 0), a.idx_stride) : L;
  const int start = split * a.chunk;
  if (start >= count) return;  // whole workgroup: nothing in this split
  const int end = min(start + a.chunk, count);
  const int G = a.group, T = a.q_len, rows = G * T;

  // Query fragments: B operand of S^T = K Q^T; lane column c16 of block qb is
  // query row m = qb*16 + c16 = (head-in-group, t).
  bf16x8 qf[QB][KS];
  int lim[QB], rowc[QB], head[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int m = qb * 16 + c16;
    const bool ok = m < rows;
    const int hh = ok ? m / T : 0, t = ok ? m % T : 0;
    head[qb] = g * G + hh;
    lim[qb] = ok ? L - T + t : 0x7fffffff;  // row t sees positions <= L - T + t
    rowc[qb] = (!SPARSE && ok) ? (t == a.row0 ? 0 : (t == a.row1 ? 1 : -1)) : -1;
    const uint16_t* qp = a.q + (((size_t)b * a.hq + head[qb]) * T + t) * D + kg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ok) {
        qf[qb][ks] = load16(qp + ks * 32);
      } else {
        qf[qb][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      }
    }
  }

  f32x4 oacc[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
  }

  uint16_t* vt = sbuf + wave * kTile * VS;
  int* sidx = s_idx[wave];
  const int step = kWaves * kTile;

  // Row offsets of the two 16-position blocks this lane loads for tile ts.
  auto rows_of = [&](int ts, size_t roff[2]) {
    if (SPARSE) {
      if (lane < kTile) {
        const int li = ts + lane;
        const int p = li < end ? a.idx[(size_t)b * a.idx_stride + li] : 0;
        sidx[lane] = min(max(p, 0), max(L - 1, 0));
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const int li = min(ts + pb * 16 + c16, end - 1);
      const int pos = SPARSE ? sidx[pb * 16 + c16] : li;
      roff[pb] = kv_row<D>(a, b, g, pos);
    }
  };

  bf16x8 kf[2][KS], vv[2][KS];
  int ts = start + wave * kTile;
  if (ts < end) {
    size_t roff[2];
    rows_of(ts, roff);
#pragma unroll
    for (int pb = 0; pb < 2; ++pb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kf[pb][ks] = load16(a.k + roff[pb] + ks * 32 + kg * 8);
        vv[pb][ks] = load16(a.v + roff[pb] + ks * 32 + kg * 8);
      }
  }

  for (; ts < end; ts += step) {
    // Absolute positions of the 8 S^T entries this lane holds.
    int apos[2][4];
    bool inr[2][4];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int li = ts + pb * 16 + 4 * kg + r;
        inr[pb][r] = li < end;
        apos[pb][r] = SPARSE ? sidx[pb * 16 + 4 * kg + r] : li;
      }

    // V tile -> LDS in natural [position][d] layout (two 8-byte stores per 16 B).
#pragma unroll
    for (int pb = 0; pb < 2; ++pb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 w = __builtin_bit_cast(u32x4, vv[pb][ks]);
        u32x2* dst = reinterpret_cast<u32x2*>(vt + (pb * 16 + c16) * VS + ks * 32 + kg * 8);
        dst[0] = u32x2{w[0], w[1]};
        dst[1] = u32x2{w[2], w[3]};
      }

    // S^T = K Q^T: entry (position pb*16 + 4*kg + r, query row qb*16 + c16).
    f32x4 sacc[2][QB];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[pb][ks], qf[qb][ks], acc, 0, 0, 0);
        sacc[pb][qb] = acc;
      }

    // Prefetch the next tile's K/V rows while this one is consumed.
    const int tn = ts + step;
    if (tn < end) {
      size_t roff[2];
      rows_of(tn, roff);
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          kf[pb][ks] = load16(a.k + roff[pb] + ks * 32 + kg * 8);
          vv[pb][ks] = load16(a.v + roff[pb] + ks * 32 + kg * 8);
        }
    }

    // Collect-2-Query epilogue: pre-softmax logits of rows row0 / row1.
    if (!SPARSE && a.layout != VGSA_LOGITS_NONE) {
      if (a.layout == VGSA_LOGITS_PER_HEAD) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (rowc[qb] < 0) continue;
          float* lp = a.logits + (((size_t)b * 2 + rowc[qb]) * a.hq + head[qb]) * a.max_ctx;
#pragma unroll
          for (int pb = 0; pb < 2; ++pb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (inr[pb][r])
                lp[apos[pb][r]] = apos[pb][r] <= lim[qb] ? sacc[pb][qb][r] * a.scale : kNegInf;
        }
      } else {
        float* lp = a.logits + ((size_t)b * a.hkv + g) * a.max_ctx;
#pragma unroll
        for (int pb = 0; pb < 2; ++pb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              if (rowc[qb] >= 0)
                acc += apos[pb][r] <= lim[qb] ? sacc[pb][qb][r] * a.scale : kNegInf;
            // sum over the 16 query-row lanes of this position (butterfly:
            // every lane ends with the same value)
            acc += __shfl_xor(acc, 1);
            acc += __shfl_xor(acc, 2);
            acc += __shfl_xor(acc, 4);
            acc += __shfl_xor(acc, 8);
            if (c16 == 0 && inr[pb][r]) lp[apos[pb][r]] = acc;
          }
      }
    }

    // Online softmax (log2 units) and the P fragments (B operand of O^T = V^T P^T).
    bf16x8 pf[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float x[2][4];
      float mx = kNegInf;
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool vis = inr[pb][r] && apos[pb][r] <= lim[qb];
          x[pb][r] = vis ? sacc[pb][qb][r] * a.scale_log2 : kNegInf;
          mx = fmaxf(mx, x[pb][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[qb], mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[qb] - m_use);
      float psum = 0.f;
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = fast_exp2(x[pb][r] - m_use);
          pf[qb][pb * 4 + r] = (__bf16)pv;
          psum += pv;
        }
      l_run[qb] = l_run[qb] * alpha + psum;
      m_run[qb] = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
    }

    // O^T += V^T P^T.  A operand: row d = db*16 + c16, k slots 0..3 are
    // positions 4*kg + j, slots 4..7 are positions 16 + 4*kg + j (the same
    // positions the P fragment holds).
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x8 vf;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int pos = (j < 4) ? 4 * kg + j : 16 + 4 * kg + (j - 4);
        vf[j] = __builtin_bit_cast(__bf16, vt[pos * VS + db * 16 + c16]);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb], oacc[db][qb], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  // Row sums: combine the four 16-lane groups.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l_run[qb] += __shfl_xor(l_run[qb], 16);
    l_run[qb] += __shfl_xor(l_run[qb], 32);
  }
  if (kg == 0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      s_m[wave][qb * 16 + c16] = m_run[qb];
      s_l[wave][qb * 16 + c16] = l_run[qb];
    }
  }
  __syncthreads();

  // Merge the four wavefronts into obuf (relative to the workgroup max).
  float* obuf = reinterpret_cast<float*>(sbuf);
  float scl[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qb * 16 + c16;
    float M = s_m[0][row];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][row]);
    scl[qb] = m_run[qb] == kNegInf ? 0.f : fast_exp2(m_run[qb] - M);
  }
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          f32x4* dst = reinterpret_cast<f32x4*>(obuf + (qb * 16 + c16) * VS + db * 16 + 4 * kg);
          const f32x4 add = oacc[db][qb] * scl[qb];
          *dst = (w == 0) ? add : (*dst + add);
        }
    }
    __syncthreads();
  }

  const int S = a.num_splits;
  for (int e = threadIdx.x; e < rows * D; e += kThreads) {
    const int m = e / D, d = e % D;
    const int h = g * G + m / T, t = m % T;
    const size_t prow = (((size_t)b * a.hq + h) * T + t) * S + split;
    a.part_o[prow * D + d] = obuf[m * VS + d];
  }
  if ((int)threadIdx.x < rows) {
    const int m = threadIdx.x;
    const int h = g * G + m / T, t = m % T;
    const size_t prow = (((size_t)b * a.hq + h) * T + t) * S + split;
    float M = s_m[0][m];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][m]);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (s_m[w][m] != kNegInf) l += s_l[w][m] * fast_exp2(s_m[w][m] - M);
    a.part_ml[prow * 2 + 0] = M;
    a.part_ml[prow * 2 + 1] = l;
  }
}

// One block of D threads per (sequence, head, row): exact merge of the splits.
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(CombineArgs a) {
  const int row = blockIdx.x;
  const int b = row / a.rows_per_seq;
  const int d = threadIdx.x;
  const int len = min(max(a.lengths[b], 0), a.span);
  const int nvalid = min((len + a.chunk - 1) / a.chunk, a.num_splits);
  const float* ml = a.part_ml + (size_t)row * a.num_splits * 2;
  const float* po = a.part_o + (size_t)row * a.num_splits * D;
  float M = kNegInf;
  for (int s = 0; s < nvalid; ++s) M = fmaxf(M, ml[2 * s]);
  float l = 0.f, acc = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < nvalid; ++s) {
      const float ms = ml[2 * s];
      if (ms == kNegInf) continue;
      const float w = fast_exp2(ms - M);
      l += w * ml[2 * s + 1];
      acc += w * po[(size_t)s * D + d];
    }
  }
  const float o = l > 0.f ? acc / l : 0.f;
  a.out[(size_t)row * D + d] = __builtin_bit_cast(uint16_t, (__bf16)o);
  if (a.lse != nullptr && d == 0) a.lse[row] = l > 0.f ? (M + __log2f(l)) * kLn2 : kNegInf;
}

template <int D, bool SPARSE>
hipError_t launch_d(const AttnArgs& a, dim3 grid, hipStream_t s) {
  const int rows = a.group * a.q_len;
  if (rows <= 16) {
    hipLaunchKernelGGL((attn_partials_kernel<D, 1, SPARSE>), grid, dim3(kThreads), 0, s, a);
  } else if (rows <= 32) {
    hipLaunchKernelGGL((attn_partials_kernel<D, 2, SPARSE>), grid, dim3(kThreads), 0, s, a);
  } else if (rows <= 48) {
    hipLaunchKernelGGL((attn_partials_kernel<D, 3, SPARSE>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_partials_kernel<D, 4, SPARSE>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_partials(const AttnArgs& a, bool sparse, hipStream_t s) {
  const dim3 grid(a.num_splits, a.hkv, a.batch);
  if (a.head_dim == 64) return sparse ? launch_d<64, true>(a, grid, s) : launch_d<64, false>(a, grid, s);
  return sparse ? launch_d<128, true>(a, grid, s) : launch_d<128, false>(a, grid, s);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.head_dim == 64) {
    hipLaunchKernelGGL(combine_kernel<64>, dim3(a.rows), dim3(64), 0, s, a);
  } else {
    hipLaunchKernelGGL(combine_kernel<128>, dim3(a.rows), dim3(128), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace vgsa
