// Top-k selection of the positions kept for the next step.
//
// Vegas (gist.science 2602.07223), "A. aggregated attention-logit selection":
// the kept set T, |T| = k, maximises the summed logits of its members; the
// objective is a sum of per-position scores, so T is a top-k of the scores.
// Dustin (gist.science 2606.24957), "1. hybrid attention aggregation": a few
// attention-sink prefix positions and a window of recent positions are kept
// first and the remaining budget is filled by score.
//
// One workgroup of 1024 threads per sequence.  Rows of up to 262144 positions
// take select_topk_kernel (radix pass over coalesced keys, the threshold bin
// ranked directly, output from a position bitmap).  With a workspace, a
// capacity of 49153 .. 262144 positions takes the per-round kernels instead
// (select_round_hist_kernel, select_round_mark_kernel, select_final_kernel:
// one workgroup per round of 32768 positions and sequence).  Longer rows take
// select_topk_large_kernel, described here:
//   * F = [0, s_end) U [w_start, L) is forced; r = k - |F| positions are
//     picked from the middle range M = [s_end, w_start).
//   * Scores become order-preserving 32-bit keys (larger score, larger key;
//     -0.0 == +0.0).  Positions outside M get key 0, below every real key.
//   * Thread t owns the contiguous run [t*run, (t+1)*run) of positions, so
//     runs are in position order and one block-wide scan orders any subset.
//   * Pass 1: a 4096-bin histogram of the top 12 key bits (LDS atomics)
//     locates the bin holding the r-th largest key.
//   * Fast path: the keys at or above that bin (typically a few hundred to a
//     few thousand) are compacted, in position order, into an LDS list; the
//     remaining 20 key bits are resolved by two more histogram passes over
//     the list only, and the output is written from the list:
//     [0, s_end) ++ selected list entries ++ [w_start, L), ascending.
//   * If the list would overflow (massive ties in one bin) the same passes
//     run over all keys instead.
// All decisions are integer comparisons, so the result is exact and
// deterministic: keys above the threshold key, then the lowest positions
// among keys equal to it.
#include "internal.h"
#include "merge_ops.h"

namespace vgsa {
namespace {

constexpr int kThreadsTk = 1024;
constexpr int kWavesTk = kThreadsTk / 64;
constexpr int kBins = 4096;
constexpr int kRunMax = 16;      // keys a thread holds in registers at once
constexpr int kCandMax = 4096;   // LDS candidate list capacity
constexpr int kCandPerThread = kCandMax / kThreadsTk;

// Larger score -> larger key; -0.0 and +0.0 share one key; every real key >= 1
// (only a NaN pattern would map to 0), so 0 marks positions outside M.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return key > 1u ? key : 1u;
}

// Sum of x over lanes 0..15 (DPP row scan; lane 15 holds the total), the
// same value in every lane.
__device__ __forceinline__ uint32_t row0_sum(uint32_t x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  return (uint32_t)__builtin_amdgcn_readlane(v, 15);
}

// Exclusive prefix sum of v over the workgroup (.x) and the sum (.y).  Lane w
// of every wave reads wave w's total, so the waves before this one and all
// waves are two 16-lane sums rather than a loop over the totals.  Results
// come back by value: a call the compiler keeps out of line then needs no
// stack slots.
__device__ uint2 block_scan(uint32_t v, uint32_t* s_wave) {
  static_assert(kWavesTk == 16, "one DPP row of wave totals");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  const uint32_t c = lane < kWavesTk ? s_wave[lane] : 0u;
  const uint32_t tot = row0_sum(c);
  const uint32_t base = row0_sum(lane < wave ? c : 0u);
  __syncthreads();
  return make_uint2(base + x - v, tot);
}

__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t& total) {
  const uint2 r = block_scan(v, s_wave);
  total = r.y;
  return r.x;
}

struct Row {
  const float* sc;
  int L, s_end, w_start, run, j0;
  bool vec;  // 16-byte aligned runs: float4 loads
};

// Keys of positions [j0 + base, j0 + base + n) of this thread's run, n <= kRunMax;
// positions outside M (or past L) get key 0.
__device__ __forceinline__ void load_keys(const Row& c, int base, uint32_t (&key)[kRunMax], int& n) {
  n = min(kRunMax, c.run - base);
  const int j = c.j0 + base;
  if (c.vec) {
#pragma unroll
    for (int i = 0; i < kRunMax; i += 4) {
      if (i < n) {
        if (j + i + 3 < c.L) {
          const float4 v = *reinterpret_cast<const float4*>(c.sc + j + i);
          key[i] = order_key(v.x);
          key[i + 1] = order_key(v.y);
          key[i + 2] = order_key(v.z);
          key[i + 3] = order_key(v.w);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) key[i + e] = (j + i + e < c.L) ? order_key(c.sc[j + i + e]) : 0u;
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kRunMax; ++i)
      if (i < n) key[i] = (j + i < c.L) ? order_key(c.sc[j + i]) : 0u;
  }
#pragma unroll
  for (int i = 0; i < kRunMax; ++i) {
    const int p = j + i;
    if (i >= n || p < c.s_end || p >= c.w_start) key[i] = 0u;
  }
}

// Finds, among the counted keys, the digit of the `want`-th largest, the rank
// left inside that digit, and (in s_out[2]) how many keys the digit's bin
// holds.  hist holds nb bins; all threads call.  Returns (prefix, want) by
// value (an out-of-line call then needs no stack slots).
__device__ uint2 find_digit_v(const uint32_t* hist, uint32_t nb, int shift, uint32_t prefix,
                              uint32_t want, uint32_t* s_wave, uint32_t* s_out) {
  const int tid = threadIdx.x;
  uint32_t cnt[4];
  const int top = (int)nb - 1 - 4 * tid;  // thread t owns bins top .. top-3 (descending)
#pragma unroll
  for (int q = 0; q < 4; ++q) cnt[q] = (top - q >= 0) ? hist[top - q] : 0u;
  uint32_t above = block_scan(cnt[0] + cnt[1] + cnt[2] + cnt[3], s_wave).x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (top - q >= 0 && above < want && want <= above + cnt[q]) {
      s_out[0] = prefix | ((uint32_t)(top - q) << shift);
      s_out[1] = want - above;
      s_out[2] = cnt[q];
    }
    above += cnt[q];
  }
  __syncthreads();
  const uint2 r = make_uint2(s_out[0], s_out[1]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t nb, int shift,
                                           uint32_t& prefix, uint32_t& want, uint32_t* s_wave,
                                           uint32_t* s_out) {
  const uint2 r = find_digit_v(hist, nb, shift, prefix, want, s_wave, s_out);
  prefix = r.x;
  want = r.y;
}

__global__ __launch_bounds__(kThreadsTk) void select_topk_large_kernel(
    int32_t max_ctx, const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    int32_t k, int32_t n_sink, int32_t window, int32_t* __restrict__ idx, int32_t idx_stride,
    int32_t* __restrict__ n_idx) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t s_wave[kWavesTk];
  __shared__ uint32_t s_out[4];
  __shared__ uint32_t cand_key[kCandMax];
  __shared__ int32_t cand_pos[kCandMax];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = min(max(seq_lens[b], 0), max_ctx);
  int32_t* out = idx + (size_t)b * idx_stride;

  if (L <= k) {
    for (int j = tid; j < L; j += kThreadsTk) out[j] = j;
    if (tid == 0) n_idx[b] = L;
    return;
  }
  Row c;
  c.sc = scores + (size_t)b * max_ctx;
  c.L = L;
  c.s_end = min(n_sink, L);
  c.w_start = max(c.s_end, L - window);
  c.run = (L + kThreadsTk - 1) / kThreadsTk;
  c.j0 = tid * c.run;
  c.vec = (c.run % 4 == 0) && (max_ctx % 4 == 0);
  const int r = k - (c.s_end + (L - c.w_start));  // >= 0: n_sink + window <= k is checked on the host
  const int tail = L - c.w_start;

  // Forced positions: [0, s_end) first, [w_start, L) last.
  for (int i = tid; i < c.s_end; i += kThreadsTk) out[i] = i;
  for (int i = tid; i < tail; i += kThreadsTk) out[c.s_end + r + i] = c.w_start + i;
  if (tid == 0) n_idx[b] = k;
  if (r == 0) return;

  const bool resident = c.run <= kRunMax;
  uint32_t key[kRunMax];
  int n = 0;
  if (resident) load_keys(c, 0, key, n);

  // Pass 1 over all keys: top 12 bits.
  for (int i = tid; i < kBins; i += kThreadsTk) hist[i] = 0u;
  __syncthreads();
  for (int base = 0; base < c.run; base += kRunMax) {
    if (!resident) load_keys(c, base, key, n);
#pragma unroll
    for (int i = 0; i < kRunMax; ++i)
      if (key[i] != 0u && i < n) atomicAdd(&hist[key[i] >> 20], 1u);
  }
  __syncthreads();
  uint32_t prefix = 0u, want = (uint32_t)r;
  find_digit(hist, kBins, 20, prefix, want, s_wave, s_out);
  const uint32_t cand_lo = prefix;  // keys >= cand_lo: the threshold bin and above

  // Count candidates; compact them into the LDS list if they fit.
  uint32_t ccount = 0u;
  for (int base = 0; base < c.run; base += kRunMax) {
    if (!resident) load_keys(c, base, key, n);
#pragma unroll
    for (int i = 0; i < kRunMax; ++i) ccount += (i < n && key[i] >= cand_lo) ? 1u : 0u;
  }
  uint32_t ctotal;
  const uint32_t cbase = block_exclusive_scan(ccount, s_wave, ctotal);

  // passes 2 and 3: 12 then 8 key bits (selects, not arrays indexed at run
  // time, which would live in scratch memory)
  const auto pass_shift = [](int pass) { return pass == 0 ? 8 : 0; };
  const auto pass_mask = [](int pass) { return pass == 0 ? 0xFFF00000u : 0xFFFFFF00u; };
  const auto pass_bins = [](int pass) { return pass == 0 ? 4096u : 256u; };
  if (ctotal <= (uint32_t)kCandMax) {
    // ---------------- fast path: resolve and emit from the candidate list
    uint32_t o = cbase;
    for (int base = 0; base < c.run; base += kRunMax) {
      if (!resident) load_keys(c, base, key, n);
#pragma unroll
      for (int i = 0; i < kRunMax; ++i)
        if (i < n && key[i] >= cand_lo) {
          cand_key[o] = key[i];
          cand_pos[o] = c.j0 + base + i;
          ++o;
        }
    }
    // passes 2 and 3 over the candidates of the threshold bin
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      for (int i = tid; i < kBins; i += kThreadsTk) hist[i] = 0u;
      __syncthreads();
      for (int q = tid; q < (int)ctotal; q += kThreadsTk) {
        const uint32_t kk = cand_key[q];
        if ((kk & pass_mask(pass)) == prefix) atomicAdd(&hist[(kk >> pass_shift(pass)) & (pass_bins(pass) - 1u)], 1u);
      }
      __syncthreads();
      find_digit(hist, pass_bins(pass), pass_shift(pass), prefix, want, s_wave, s_out);
    }
    const uint32_t thr = prefix, need_eq = want;
    // ordered emit: thread t owns list entries [4t, 4t+4)
    uint32_t kk[kCandPerThread];
    uint32_t ceq = 0u;
#pragma unroll
    for (int q = 0; q < kCandPerThread; ++q) {
      const int e = tid * kCandPerThread + q;
      kk[q] = e < (int)ctotal ? cand_key[e] : 0u;
      ceq += kk[q] == thr ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t eq = block_exclusive_scan(ceq, s_wave, tot);
    uint32_t csel = 0u;
    bool keep[kCandPerThread];
#pragma unroll
    for (int q = 0; q < kCandPerThread; ++q) {
      keep[q] = kk[q] > thr || (kk[q] == thr && eq++ < need_eq);
      csel += keep[q] ? 1u : 0u;
    }
    uint32_t so = block_exclusive_scan(csel, s_wave, tot) + (uint32_t)c.s_end;
#pragma unroll
    for (int q = 0; q < kCandPerThread; ++q)
      if (keep[q] && so < (uint32_t)idx_stride) out[so++] = cand_pos[tid * kCandPerThread + q];
    return;
  }

  // ---------------- general path: passes 2 and 3 and the emit over all keys
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = tid; i < kBins; i += kThreadsTk) hist[i] = 0u;
    __syncthreads();
    for (int base = 0; base < c.run; base += kRunMax) {
      if (!resident) load_keys(c, base, key, n);
#pragma unroll
      for (int i = 0; i < kRunMax; ++i)
        if (i < n && key[i] != 0u && (key[i] & pass_mask(pass)) == prefix)
          atomicAdd(&hist[(key[i] >> pass_shift(pass)) & (pass_bins(pass) - 1u)], 1u);
    }
    __syncthreads();
    find_digit(hist, pass_bins(pass), pass_shift(pass), prefix, want, s_wave, s_out);
  }
  const uint32_t thr = prefix, need_eq = want;
  uint32_t ceq = 0u;
  for (int base = 0; base < c.run; base += kRunMax) {
    if (!resident) load_keys(c, base, key, n);
#pragma unroll
    for (int i = 0; i < kRunMax; ++i) ceq += (i < n && key[i] == thr) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t eq_base = block_exclusive_scan(ceq, s_wave, tot);
  uint32_t e = eq_base, csel = 0u;
  for (int base = 0; base < c.run; base += kRunMax) {
    if (!resident) load_keys(c, base, key, n);
#pragma unroll
    for (int i = 0; i < kRunMax; ++i)
      if (i < n) csel += (key[i] > thr || (key[i] == thr && e++ < need_eq)) ? 1u : 0u;
  }
  uint32_t o = block_exclusive_scan(csel, s_wave, tot) + (uint32_t)c.s_end;
  e = eq_base;
  for (int base = 0; base < c.run; base += kRunMax) {
    if (!resident) load_keys(c, base, key, n);
#pragma unroll
    for (int i = 0; i < kRunMax; ++i)
      if (i < n && (key[i] > thr || (key[i] == thr && e++ < need_eq)) && o < (uint32_t)idx_stride)
        out[o++] = c.j0 + base + i;
  }
}

// ---------------------------------------------------------------------------
// Rows of up to R * 32768 positions (R <= 8 rounds).
//   * Round r of the keys: thread t holds positions r*32768 + 4096c + 4t + e
//     (c < 8, e < 4), so every load instruction reads 1 KB of contiguous
//     scores (16-byte loads when rows are 16-byte aligned, 4-byte loads
//     otherwise).  With one round the keys stay in registers for the whole
//     kernel; otherwise each pass reloads them (from L2 after the first).
//   * Radix passes (12, 12, then 8 bits; usually the first suffices) find the
//     bin of the r-th largest key, stopping as soon as that bin holds at most
//     kBinCapOne keys (one round: another pass over registers costs about
//     2 us) or kBinCapMany keys (reloaded rounds: a pass reloads the row,
//     about 17 us at 131072 positions).  Ranking n members directly costs
//     O(n^2) comparisons: about 75 us for 2000 members.
//   * Keys above the bin are marked in an LDS bitmap of the positions; the
//     bin's members go to an LDS list, are ranked directly (larger key, then
//     lower position) and the best `want` are marked too.  If the bin is
//     bigger than the cap after the last pass, its keys are all equal and the
//     lowest positions win: they are marked from a second bitmap.
//   * The output is written from the bitmap: thread t owns bitmap words
//     R*t .. R*t + R - 1 (positions 32Rt .. 32R(t+1) - 1), one block scan
//     orders the threads.
constexpr int kSmallChunks = 8;                          // 4096-position chunks per round
constexpr int kRoundLen = kSmallChunks * 4 * kThreadsTk;  // positions per round (32768)
constexpr int kMaxRounds = 8;
constexpr int kBinCapOne = 252;    // bin members ranked directly: one round
constexpr int kBinCapMany = 764;   // ... reloaded rounds
constexpr int kBinCap = kBinCapMany;

// LDS of the one-workgroup selection, for rows of up to RM rounds.
template <int RM>
struct SelectLdsT {
  uint32_t hist[kBins];
  uint32_t s_wave[kWavesTk];
  uint32_t s_out[4];
  __align__(16) uint32_t taken[RM * kThreadsTk];   // positions selected (above the bin, or ranked in)
  __align__(16) uint32_t in_bin[RM * kThreadsTk];  // bin members, when they are all equal
  // bin members as (key << 32 | ~position): larger means ranked first
  __align__(16) uint64_t bin_rank_key[kBinCap + 4];
  uint32_t rank[kBinCap];  // members ranked before each one
  uint32_t count;
};
using SelectLds = SelectLdsT<kMaxRounds>;

// The threshold bin: sh.bin_rank_key[0, nbin) holds its members (not
// exact), or sh.in_bin marks them (exact: their keys are all equal).  The
// best `want` of them join sh.taken: larger key, then lower position.
// Starts with a workgroup barrier (after the members were written) and ends
// with one.
template <class Lds>
__device__ void resolve_bin(Lds& sh, uint32_t nbin, uint32_t want, bool exact, int R) {
  const int tid = threadIdx.x;
  nbin = __builtin_amdgcn_readfirstlane(nbin);  // the same in every lane (read from LDS)
  want = __builtin_amdgcn_readfirstlane(want);
  if (!exact) {
    if (tid < 4) sh.bin_rank_key[nbin + tid] = 0u;  // padding to a multiple of 4; ranks last
    for (int q = tid; q < (int)nbin; q += kThreadsTk) sh.rank[q] = 0u;
  }
  __syncthreads();
  if (!exact) {
    // rank = members with a larger key, or an equal key at a lower position.
    // Members go 64 to a wave (lane = member), and the waves left over split
    // the list to compare against into shares: every lane of a wave reads the
    // same entries, and the partial counts meet in sh.rank.
    const int lane = tid & 63, wave = tid >> 6;
    const int n4 = (int)(nbin + 3u) / 4;
    const int blocks = (int)(nbin + 63u) / 64;  // <= kWavesTk: nbin <= kBinCap
    const int shares = max(1, kWavesTk / blocks);
    const int mb = wave / shares, sh_i = wave % shares;
    if (mb < blocks) {
      const int q = mb * 64 + lane;
      const uint64_t cq = q < (int)nbin ? sh.bin_rank_key[q] : ~0ull;
      const int f1 = (sh_i + 1) * n4 / shares;
      uint32_t cnt = 0u;
#pragma unroll 4
      for (int f = sh_i * n4 / shares; f < f1; ++f) {
        const uint64_t* c4 = sh.bin_rank_key + 4 * f;
        cnt += (c4[0] > cq ? 1u : 0u) + (c4[1] > cq ? 1u : 0u) + (c4[2] > cq ? 1u : 0u) +
               (c4[3] > cq ? 1u : 0u);
      }
      if (q < (int)nbin && cnt != 0u) atomicAdd(&sh.rank[q], cnt);
    }
    __syncthreads();
    for (int q = tid; q < (int)nbin; q += kThreadsTk)
      if (sh.rank[q] < want) {
        const int pq = (int)~(uint32_t)sh.bin_rank_key[q];
        atomicOr(&sh.taken[pq >> 5], 1u << (pq & 31));
      }
  } else {
    // the first `want` bin members in position order join the taken set;
    // thread t owns words R*t .. R*t + R - 1
    uint32_t n_in = 0u, tot;
    for (int j = 0; j < R; ++j) n_in += (uint32_t)__builtin_popcount(sh.in_bin[R * tid + j]);
    uint32_t q = block_exclusive_scan(n_in, sh.s_wave, tot);
    for (int j = 0; j < R; ++j) {
      uint32_t w = sh.taken[R * tid + j];
      for (uint32_t bits = sh.in_bin[R * tid + j]; bits != 0u && q < want; ++q) {
        w |= bits & (~bits + 1u);  // lowest remaining member
        bits &= bits - 1u;
      }
      sh.taken[R * tid + j] = w;
      sh.in_bin[R * tid + j] = 0u;
    }
  }
  __syncthreads();
}

// Lanes 0..7 of the result: the 32-bit halves of four 64-bit wave-uniform
// masks, b[j / 2] >> 32 (j % 2) in lane j (other lanes 0).  v_writelane
// takes the scalar operand directly, one instruction per lane (a register
// move; the asm touches no memory).
__device__ __forceinline__ uint32_t words8(const uint64_t (&b)[4]) {
  uint32_t w = 0u;
#define VGSA_WL(J, X) asm("v_writelane_b32 %0, %1, " #J : "+v"(w) : "s"(X))
  VGSA_WL(0, (uint32_t)b[0]);
  VGSA_WL(1, (uint32_t)(b[0] >> 32));
  VGSA_WL(2, (uint32_t)b[1]);
  VGSA_WL(3, (uint32_t)(b[1] >> 32));
  VGSA_WL(4, (uint32_t)b[2]);
  VGSA_WL(5, (uint32_t)(b[2] >> 32));
  VGSA_WL(6, (uint32_t)b[3]);
  VGSA_WL(7, (uint32_t)(b[3] >> 32));
#undef VGSA_WL
  return w;
}

// One selection stage: marks in sh.taken the `want_stage` middle positions
// [s_end, w_start) of highest score in row `sc` (lower position first among
// equal keys).  FROM_LDS: `sc` is an LDS array (else global memory, read as a
// buffer bounded by the row, whose loads past the row return 0).  EXCL:
// positions already marked are no candidates; a thread only marks positions
// whose keys it has already read, so the marks it reads are the earlier
// stage's.  COHERENT: the scores were written in this launch by other
// workgroups (possibly on another XCD): they are read with device-scope
// loads.  PREHIST: ghist holds the first pass's histogram (top 12 key bits of
// the stage's candidates, kBins counts, written in this launch: read with
// device-scope loads, together with the first round's keys).
// Slot (c, e) of a thread holds position rd * kRoundLen + c * 4 * kThreadsTk +
// 256 * wave + 64 * e + lane: one slot of a wave is 64 consecutive positions,
// two whole bitmap words, which a ballot over the slot gives at once.
// Starts and ends with a workgroup barrier.
template <bool FROM_LDS, bool EXCL, bool COHERENT = false, bool PREHIST = false, class Lds>
__device__ __forceinline__ void select_stage(Lds& sh, const float* __restrict__ sc,
                                             int max_ctx, int R, int s_end, int w_start,
                                             uint32_t want_stage,
                                             const uint32_t* __restrict__ ghist = nullptr) {
  static_assert(!(PREHIST && EXCL), "a precomputed histogram has no exclusions");
  static_assert(!(FROM_LDS && COHERENT), "device-scope loads read global memory");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool reload = R > 1;
  // (unused when FROM_LDS)
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sc), 0, max_ctx * 4, kRawBufferWord3);
  // Keys of round `rd`; 0 outside M = [s_end, w_start) (and for excluded
  // positions).  A wave whose 256 positions of a chunk all lie in M (and no
  // exclusions) skips the per-position tests.
  uint32_t key[kSmallChunks][4];
  auto load_round = [&](int rd) {
    float v[kSmallChunks][4];
    const int p_lane = rd * kRoundLen + 256 * wave + lane;
#pragma unroll
    for (int c = 0; c < kSmallChunks; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = p_lane + c * 4 * kThreadsTk + 64 * e;
        if constexpr (FROM_LDS)
          v[c][e] = sc[min(p, max_ctx - 1)];
        else
          v[c][e] = __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)p * 4u, 0, COHERENT ? kCpolSc1 : 0));
      }
#pragma unroll
    for (int c = 0; c < kSmallChunks; ++c) {
      const int b0 = rd * kRoundLen + c * 4 * kThreadsTk + 256 * wave;  // wave-uniform
      if (!EXCL && b0 >= s_end && b0 + 256 <= w_start) {
#pragma unroll
        for (int e = 0; e < 4; ++e) key[c][e] = order_key(v[c][e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = b0 + 64 * e + lane;
          bool in = p >= s_end && p < w_start;
          if (EXCL) in = in && ((sh.taken[p >> 5] >> (p & 31)) & 1u) == 0u;
          key[c][e] = in ? order_key(v[c][e]) : 0u;
        }
      }
    }
  };
  bool have0 = false;  // key[] holds round 0
  if (PREHIST) {
    uint32_t h[kBins / kThreadsTk];
#pragma unroll
    for (int q = 0; q < kBins / kThreadsTk; ++q)
      h[q] = __float_as_uint(
          load1_device(reinterpret_cast<const float*>(ghist), (uint32_t)(tid + q * kThreadsTk) * 4u));
    load_round(0);
    have0 = true;
#pragma unroll
    for (int q = 0; q < kBins / kThreadsTk; ++q) sh.hist[tid + q * kThreadsTk] = h[q];
    if (tid == 0) sh.count = 0u;
    __syncthreads();
  } else {
    if (tid == 0) sh.count = 0u;
    __syncthreads();  // earlier marks complete
    if (!reload) {
      load_round(0);
      have0 = true;
    }
  }

  // Radix passes: after each, keys whose masked value exceeds `prefix` are
  // taken and `want` more come from the bin (masked value == prefix).  Real
  // keys are >= 1 and the bin holds one at least, so with hi = prefix | ~mask
  // and lo = max(prefix, 1) a key is above the bin iff key > hi and in it iff
  // key - lo <= hi - lo (unsigned; key 0 is neither).
  uint32_t prefix = 0u, mask = 0u, want = want_stage, nbin = 0u;
  int level = 0;
#pragma unroll 1
  for (; level < 3; ++level) {
    const int shift = level == 0 ? 20 : (level == 1 ? 8 : 0);
    const uint32_t nb = level == 2 ? 256u : (uint32_t)kBins;
    if (!PREHIST || level > 0) {
      const uint32_t lo = prefix > 1u ? prefix : 1u, span = (prefix | ~mask) - lo;
      for (int i = tid; i < (int)nb; i += kThreadsTk) sh.hist[i] = 0u;
      __syncthreads();
#pragma unroll 1
      for (int rd = 0; rd < R; ++rd) {
        if (reload && !(rd == 0 && have0)) load_round(rd);
#pragma unroll
        for (int c = 0; c < kSmallChunks; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (key[c][e] - lo <= span) atomicAdd(&sh.hist[(key[c][e] >> shift) & (nb - 1u)], 1u);
      }
      if (reload) have0 = false;  // key[] ends on the last round
      __syncthreads();
    }
    find_digit(sh.hist, nb, shift, prefix, want, sh.s_wave, sh.s_out);
    nbin = sh.s_out[2];
    mask |= (nb - 1u) << shift;
    if (nbin <= (uint32_t)(reload ? kBinCapMany : kBinCapOne)) break;
  }
  const bool exact = level == 3;  // the bin's keys are all equal: lowest positions first
  const uint32_t hi = prefix | ~mask, lo = prefix > 1u ? prefix : 1u;

  // Mark keys above the bin; collect (or mark) the bin's members.  A chunk's
  // four slots are eight bitmap words that only this wave writes: their
  // ballots go into lanes 0..7 (lane 2e + h holds half h of slot e) and
  // those lanes OR them in with one LDS instruction.  Ranked bin members
  // (few) take list slots with one LDS atomic per chunk that has any.
  const int wlane = lane < 8 ? lane : 7;
  const auto mark = [&](auto exact_c) {
    constexpr bool EXACT = decltype(exact_c)::value;
#pragma unroll 1
    for (int rd = 0; rd < R; ++rd) {
      if (reload && !(rd == 0 && have0)) load_round(rd);
#pragma unroll
      for (int c = 0; c < kSmallChunks; ++c) {
        const int b0 = rd * kRoundLen + c * 4 * kThreadsTk + 256 * wave;  // wave-uniform
        uint64_t up[4], in[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          up[e] = __ballot(key[c][e] > hi);
          in[e] = __ballot(key[c][e] >= lo) & ~up[e];  // lo <= key <= hi
        }
        if (lane < 8) atomicOr(&sh.taken[(b0 >> 5) + wlane], words8(up));
        if constexpr (EXACT) {
          if (lane < 8) atomicOr(&sh.in_bin[(b0 >> 5) + wlane], words8(in));
        } else if ((in[0] | in[1] | in[2] | in[3]) != 0u) {
          const uint32_t n =
              (uint32_t)(__popcll(in[0]) + __popcll(in[1]) + __popcll(in[2]) + __popcll(in[3]));
          uint32_t slot = 0u;
          if (lane == 0) slot = atomicAdd(&sh.count, n);  // total < nbin <= kBinCap
          slot = __builtin_amdgcn_readfirstlane(slot);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if ((in[e] >> lane) & 1u) {
              const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                  (uint32_t)(in[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)in[e], 0u));
              sh.bin_rank_key[slot + below] =
                  ((uint64_t)key[c][e] << 32) | (uint32_t)~(uint32_t)(b0 + 64 * e + lane);
            }
            slot += (uint32_t)__popcll(in[e]);
          }
        }
      }
    }
  };
  if (exact)
    mark(std::true_type{});
  else
    mark(std::false_type{});
  resolve_bin(sh, nbin, want, exact, R);
}

// Ordered emit: [0, s_end) ++ the positions marked in sh.taken ++ [w_start, L)
// (r of them marked).  Thread t owns words R*t .. R*t + R - 1.
template <class Lds>
__device__ void emit_taken(Lds& sh, int R, int s_end, int w_start, int L, int r,
                           int32_t* __restrict__ out, int32_t idx_stride) {
  const int tid = threadIdx.x;
  const uint32_t* my = sh.taken + R * tid;
  uint32_t n_sel = 0u, tot;
  for (int j = 0; j < R; ++j) n_sel += (uint32_t)__builtin_popcount(my[j]);
  uint32_t o = block_exclusive_scan(n_sel, sh.s_wave, tot) + (uint32_t)s_end;
  for (int j = 0; j < R; ++j)
    for (uint32_t bits = my[j]; bits != 0u; bits &= bits - 1u)
      if (o < (uint32_t)idx_stride) out[o++] = 32 * (R * tid + j) + __builtin_ctz(bits);
  for (int i = tid; i < s_end; i += kThreadsTk) out[i] = i;
  for (int i = tid; i < L - w_start; i += kThreadsTk) out[s_end + r + i] = w_start + i;
}

// HYBRID: two stages (Dustin, "1. hybrid attention aggregation"): the first
// picks min(m, r) free positions by `first` (the draft-lookahead scores), the
// second the other r - min(m, r) by `scores` (the target-historical scores)
// among the positions the first stage left free.  Without HYBRID only the
// second stage runs, picking all r by `scores`.
template <bool HYBRID>
__global__ __launch_bounds__(kThreadsTk) void select_topk_kernel(
    int32_t max_ctx, const float* __restrict__ scores, const float* __restrict__ first,
    const int32_t* __restrict__ seq_lens, int32_t k, int32_t m, int32_t n_sink, int32_t window,
    int32_t* __restrict__ idx, int32_t idx_stride, int32_t* __restrict__ n_idx) {
  __shared__ SelectLds sh;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int L = min(max(seq_lens[b], 0), max_ctx);
  int32_t* out = idx + (size_t)b * idx_stride;
  if (L <= k) {
    for (int j = tid; j < L; j += kThreadsTk) out[j] = j;
    if (tid == 0) n_idx[b] = L;
    return;
  }
  const int s_end = min(n_sink, L), w_start = max(s_end, L - window);
  const int r = k - (s_end + (L - w_start));  // >= 0: n_sink + window <= k is checked on the host
  const int tail = L - w_start;
  if (r == 0) {
    for (int i = tid; i < s_end; i += kThreadsTk) out[i] = i;
    for (int i = tid; i < tail; i += kThreadsTk) out[s_end + i] = w_start + i;
    if (tid == 0) n_idx[b] = k;
    return;
  }
  // Rounds this row needs (the launcher guarantees max_ctx <= kMaxRounds
  // rounds); with one round the keys stay in registers within a stage.
  const int R = (L + kRoundLen - 1) / kRoundLen;
  for (int i = tid; i < R * kThreadsTk; i += kThreadsTk) {
    sh.taken[i] = 0u;
    sh.in_bin[i] = 0u;
  }
  const int m_first = HYBRID ? min(max(m, 0), r) : 0;
  if (HYBRID && m_first > 0)
    select_stage<false, false>(sh, first + (size_t)b * max_ctx, max_ctx, R, s_end, w_start,
                             (uint32_t)m_first);
  if (r > m_first)
    select_stage<false, HYBRID>(sh, scores + (size_t)b * max_ctx, max_ctx, R, s_end, w_start,
                              (uint32_t)(r - m_first));

  emit_taken(sh, R, s_end, w_start, L, r, out, idx_stride);
  if (tid == 0) n_idx[b] = k;
}

// ---------------------------------------------------------------------------
// Block-granular selection (structured block sparsity): whole blocks of
// `block` positions are kept.  The score of a block is the sum of its
// members' scores (float32, position order); the blocks holding the sinks and
// the recent window are kept first and the rest of the k_blocks go to the
// largest block sums, lower block first among equals.  The block sums of the
// row go to LDS, one selection stage runs over them (keys in registers: a
// row has at most kMaxSelBlocks blocks), and the kept blocks are written out
// expanded to their positions, ascending, so the list feeds the sparse
// attention call as it is.  With bsum_out the fp32 block sums the ranking
// compared are also written out ([B][ceil(max_ctx / block)], blocks below
// ceil(L / block)), so a caller can check them and rank them itself.
// IDS: the kept blocks' ids are written instead (ascending, n_idx[b] of
// them), for a gather over block lists.
template <bool VEC, bool IDS>
__global__ __launch_bounds__(kThreadsTk) void select_blocks_kernel(
    int32_t max_ctx, const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    int32_t k_blocks, int32_t block, int32_t n_sink, int32_t window, int32_t* __restrict__ idx,
    int32_t idx_stride, int32_t* __restrict__ n_idx, float* __restrict__ bsum_out) {
  __shared__ SelectLds sh;
  __shared__ __align__(16) float s_bsum[kMaxSelBlocks];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int L = min(max(seq_lens[b], 0), max_ctx);
  const int nb = (L + block - 1) / block;
  int32_t* out = idx + (size_t)b * idx_stride;
  const bool keep_all = nb <= k_blocks;
  // forced blocks: [0, s_end) hold the sinks, [w_start, nb) the window
  const int s_end = min((n_sink + block - 1) / block, nb);
  const int w_start = window > 0 ? max(s_end, max(0, L - window) / block) : nb;
  const int r = keep_all ? 0 : k_blocks - (s_end + (nb - w_start));  // >= 0: checked on the host
  const int head_pos = min(L, s_end * block), tail0 = w_start * block;
  const int tail_pos = w_start < nb ? L - tail0 : 0;

  if (r > 0 || bsum_out != nullptr) {
    // block sums (members below L only), float32 in position order
    const float* sc = scores + (size_t)b * max_ctx;
    if (VEC && block == 16) {
      // the loads of four blocks go out together (one round trip per four
      // blocks instead of one per block); blocks wholly below L only
      const int nfull = L / 16;
      for (int i0 = tid; i0 < nb; i0 += 4 * kThreadsTk) {
        float4 x[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * kThreadsTk;
          if (i < nfull)
#pragma unroll
            for (int q = 0; q < 4; ++q) x[u][q] = *reinterpret_cast<const float4*>(sc + i * 16 + 4 * q);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * kThreadsTk;
          if (i < nb) {
            float sum = 0.f;
            if (i < nfull) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                sum += x[u][q].x; sum += x[u][q].y; sum += x[u][q].z; sum += x[u][q].w;
              }
            } else {
              for (int j = i * 16; j < L; ++j) sum += sc[j];
            }
            s_bsum[i] = sum;
          }
        }
      }
    } else {
      for (int i = tid; i < nb; i += kThreadsTk) {
        const int j0 = i * block, j1 = min(L, j0 + block);
        float sum = 0.f;
        if (VEC && j1 - j0 == block) {
          for (int j = j0; j < j1; j += 4) {
            const float4 x = *reinterpret_cast<const float4*>(sc + j);
            sum += x.x; sum += x.y; sum += x.z; sum += x.w;
          }
        } else {
          for (int j = j0; j < j1; ++j) sum += sc[j];
        }
        s_bsum[i] = sum;
      }
    }
    if (bsum_out != nullptr) {
      // each thread reads back only the sums it wrote itself
      const int nbs = (max_ctx + block - 1) / block;
      for (int i = tid; i < nb; i += kThreadsTk) bsum_out[(size_t)b * nbs + i] = s_bsum[i];
    }
  }
  if (keep_all) {
    const int n_all = IDS ? nb : L;
    for (int j = tid; j < n_all; j += kThreadsTk) out[j] = j;
    if (tid == 0) n_idx[b] = n_all;
    return;
  }
  if (r > 0) {
    sh.taken[tid] = 0u;  // one round: word t holds blocks 32t .. 32t + 31
    sh.in_bin[tid] = 0u;
    select_stage<true, false>(sh, s_bsum, kMaxSelBlocks, 1, s_end, w_start, (uint32_t)r);
  } else {
    sh.taken[tid] = 0u;
    __syncthreads();
  }

  // Ordered emit: sink positions ++ the chosen middle blocks' positions ++
  // window positions (IDS: the blocks themselves).  Thread t owns the 32
  // blocks of bitmap word t.
  const uint32_t word = sh.taken[tid];
  if (IDS) {
    uint32_t mid;
    uint32_t o = block_exclusive_scan((uint32_t)__builtin_popcount(word), sh.s_wave, mid) +
                 (uint32_t)s_end;
    for (uint32_t bits = word; bits != 0u; bits &= bits - 1u) out[o++] = 32 * tid + __builtin_ctz(bits);
    for (int i = tid; i < s_end; i += kThreadsTk) out[i] = i;
    for (int i = tid; i < nb - w_start; i += kThreadsTk) out[s_end + (int)mid + i] = w_start + i;
    if (tid == 0) n_idx[b] = s_end + (int)mid + (nb - w_start);
    return;
  }
  uint32_t n_mine = 0u, mid_total;
  for (uint32_t bits = word; bits != 0u; bits &= bits - 1u) {
    const int blk = 32 * tid + __builtin_ctz(bits);
    n_mine += (uint32_t)(min(L, blk * block + block) - blk * block);
  }
  uint32_t o = block_exclusive_scan(n_mine, sh.s_wave, mid_total) + (uint32_t)head_pos;
  for (uint32_t bits = word; bits != 0u; bits &= bits - 1u) {
    const int blk = 32 * tid + __builtin_ctz(bits);
    for (int j = blk * block; j < min(L, blk * block + block); ++j)
      if (o < (uint32_t)idx_stride) out[o++] = j;
  }
  const int n_total = head_pos + (int)mid_total + tail_pos;
  for (int i = tid; i < head_pos; i += kThreadsTk)
    if (i < idx_stride) out[i] = i;
  for (int i = tid; i < tail_pos; i += kThreadsTk)
    if (head_pos + (int)mid_total + i < idx_stride) out[head_pos + mid_total + i] = tail0 + i;
  if (tid == 0) n_idx[b] = min(n_total, idx_stride);
}

// ---------------------------------------------------------------------------
// Rows of 2 .. 8 rounds with a workspace: the work of a row is spread over one
// workgroup per round, in three launches (their boundaries make each
// launch's writes visible to the next; no workgroup waits on another):
//   1. select_round_hist_kernel: round rd's 4096-bin histogram of the top 12
//      key bits -> ws_hist[b][rd].
//   2. select_round_mark_kernel: every round's workgroup sums the row's
//      histograms and finds the bin of the r-th largest key (the same result
//      in every workgroup); it writes its round's bitmap of keys above the
//      bin -> ws_bits[b], and its round's bin members as (key << 32 |
//      ~position) -> ws_list[b][rd], their count -> ws_cnt[b][rd].
//   3. select_final_kernel (one workgroup per row): the bin's members (at
//      most kFinalCap, else the one-workgroup selection runs instead) are
//      refined by two more radix passes over the list only and ranked; the
//      ordered output is written from the bitmap.
// Hybrid selection runs the three launches twice: on the draft scores for
// the first min(m, r) positions (picks kept as a bitmap in the workspace),
// then on the target scores with those positions excluded.
// The one-workgroup kernel spends about 17 us per pass over a 131072-position
// row on one CU and needs at least two passes over it plus the marking.
constexpr int kFinalCap = 8192;  // bin members taken through the list

struct SelRow {
  int L, s_end, w_start, r, R;
  bool trivial;  // L <= k, or the forced positions fill the budget
};

__device__ __forceinline__ SelRow sel_row(int b, int32_t max_ctx, const int32_t* seq_lens,
                                          int32_t k, int32_t n_sink, int32_t window) {
  SelRow s;
  s.L = min(max(seq_lens[b], 0), max_ctx);
  s.s_end = min(n_sink, s.L);
  s.w_start = max(s.s_end, s.L - window);
  s.r = k - (s.s_end + (s.L - s.w_start));
  s.R = (s.L + kRoundLen - 1) / kRoundLen;
  s.trivial = s.L <= k || s.r <= 0;
  return s;
}

// Keys of round rd: thread t holds positions rd*32768 + 4096c + 4t + e;
// key 0 outside M = [s_end, w_start) and for positions set in `excl` (the
// row's bitmap of a first stage's picks, or null).
template <bool VEC>
__device__ __forceinline__ void round_keys(const float* __restrict__ sc, int32_t max_ctx, int rd,
                                           const SelRow& s, const uint32_t* __restrict__ excl,
                                           uint32_t (&key)[kSmallChunks][4]) {
  const int tid = threadIdx.x;
  float v[kSmallChunks][4];
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    const int p0 = rd * kRoundLen + c * 4 * kThreadsTk + 4 * tid;
    if (VEC) {
      const float4 x = *reinterpret_cast<const float4*>(sc + min(p0, max_ctx - 4));
      v[c][0] = x.x; v[c][1] = x.y; v[c][2] = x.z; v[c][3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[c][e] = sc[min(p0 + e, max_ctx - 1)];
    }
  }
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    const int p0 = rd * kRoundLen + c * 4 * kThreadsTk + 4 * tid;
    const uint32_t gone = excl != nullptr ? excl[p0 >> 5] >> (p0 & 31) : 0u;  // p0 4-aligned
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = p0 + e;
      key[c][e] = (p >= s.s_end && p < s.w_start && ((gone >> e) & 1u) == 0u) ? order_key(v[c][e]) : 0u;
    }
  }
}

struct SelWorkspace {
  uint32_t* hist;   // [B][Rm][kBins]
  uint32_t* bits;   // [B][Rm * kThreadsTk]
  uint64_t* list;   // [B][Rm][kFinalCap]
  uint32_t* cnt;    // [B][Rm]
  uint32_t* meta;   // [B][4]: bin prefix, rank wanted inside the bin, bin size
  uint32_t* first;  // [B][Rm * kThreadsTk]: the first stage's picks (hybrid)
  int32_t rounds;   // Rm
  // 0: one stage (r positions by `scores`); 1: first hybrid stage (min(m, r)
  // by the draft scores, picks kept in `first`); 2: second hybrid stage (the
  // rest by the target scores, `first` excluded, output written)
  int32_t stage;
  int32_t m;
};

// Positions the stage picks from the row.
__device__ __forceinline__ int stage_want(const SelRow& s, const SelWorkspace& ws) {
  const int m1 = min(max(ws.m, 0), s.r);
  return ws.stage == 0 ? s.r : ws.stage == 1 ? m1 : s.r - m1;
}

__device__ __forceinline__ const uint32_t* stage_excl(const SelWorkspace& ws, int b) {
  return ws.stage == 2 ? ws.first + (size_t)b * ws.rounds * kThreadsTk : nullptr;
}

template <bool VEC>
__global__ __launch_bounds__(kThreadsTk) void select_round_hist_kernel(
    int32_t max_ctx, const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    int32_t k, int32_t n_sink, int32_t window, SelWorkspace ws) {
  __shared__ uint32_t hist[kBins];
  const int rd = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const SelRow s = sel_row(b, max_ctx, seq_lens, k, n_sink, window);
  if (s.trivial || rd >= s.R || stage_want(s, ws) <= 0) return;
  for (int i = tid; i < kBins; i += kThreadsTk) hist[i] = 0u;
  __syncthreads();
  uint32_t key[kSmallChunks][4];
  round_keys<VEC>(scores + (size_t)b * max_ctx, max_ctx, rd, s, stage_excl(ws, b), key);
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (key[c][e] != 0u) atomicAdd(&hist[key[c][e] >> 20], 1u);
  __syncthreads();
  uint32_t* dst = ws.hist + ((size_t)b * ws.rounds + rd) * kBins;
  for (int i = tid; i < kBins; i += kThreadsTk) dst[i] = hist[i];
}

template <bool VEC>
__global__ __launch_bounds__(kThreadsTk) void select_round_mark_kernel(
    int32_t max_ctx, const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    int32_t k, int32_t n_sink, int32_t window, SelWorkspace ws) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t s_wave[kWavesTk];
  __shared__ uint32_t s_out[4];
  __shared__ uint32_t bits[kThreadsTk];  // this round's bitmap words
  __shared__ uint32_t count;
  const int rd = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const SelRow s = sel_row(b, max_ctx, seq_lens, k, n_sink, window);
  const int want_stage = stage_want(s, ws);
  if (s.trivial || rd >= s.R || want_stage <= 0) return;
  for (int i = tid; i < kBins; i += kThreadsTk) {
    uint32_t h = 0u;
    for (int q = 0; q < s.R; ++q) h += ws.hist[((size_t)b * ws.rounds + q) * kBins + i];
    hist[i] = h;
  }
  bits[tid] = 0u;
  if (tid == 0) count = 0u;
  __syncthreads();
  uint32_t prefix = 0u, want = (uint32_t)want_stage;
  find_digit(hist, kBins, 20, prefix, want, s_wave, s_out);  // the stage's keys number >= want
  const uint32_t nbin = s_out[2], pbin = prefix >> 20;
  uint32_t key[kSmallChunks][4];
  round_keys<VEC>(scores + (size_t)b * max_ctx, max_ctx, rd, s, stage_excl(ws, b), key);
  uint64_t* list = ws.list + ((size_t)b * ws.rounds + rd) * kFinalCap;
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    const int p0 = c * 4 * kThreadsTk + 4 * tid;  // position within the round; 4-aligned
    uint32_t above = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t kb = key[c][e] >> 20;
      above |= (key[c][e] != 0u && kb > pbin) ? (1u << e) : 0u;
      if (key[c][e] != 0u && kb == pbin && nbin <= (uint32_t)kFinalCap) {
        const uint32_t slot = atomicAdd(&count, 1u);  // < nbin
        list[slot] = ((uint64_t)key[c][e] << 32) | (uint32_t)~(uint32_t)(rd * kRoundLen + p0 + e);
      }
    }
    if (above != 0u) atomicOr(&bits[p0 >> 5], above << (p0 & 31));
  }
  __syncthreads();
  ws.bits[(size_t)b * ws.rounds * kThreadsTk + (size_t)rd * kThreadsTk + tid] = bits[tid];
  if (tid == 0) {
    ws.cnt[(size_t)b * ws.rounds + rd] = count;
    if (rd == 0) {
      ws.meta[(size_t)b * 4 + 0] = prefix;
      ws.meta[(size_t)b * 4 + 1] = want;
      ws.meta[(size_t)b * 4 + 2] = nbin;
    }
  }
}

__global__ __launch_bounds__(kThreadsTk) void select_final_kernel(
    int32_t max_ctx, const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    int32_t k, int32_t n_sink, int32_t window, int32_t* __restrict__ idx, int32_t idx_stride,
    int32_t* __restrict__ n_idx, SelWorkspace ws) {
  __shared__ SelectLds sh;
  __shared__ uint64_t cand[kFinalCap];
  const int b = blockIdx.x, tid = threadIdx.x;
  const SelRow s = sel_row(b, max_ctx, seq_lens, k, n_sink, window);
  int32_t* out = idx + (size_t)b * idx_stride;
  if (s.L <= k) {
    if (ws.stage == 1) return;  // the second stage writes the output
    for (int j = tid; j < s.L; j += kThreadsTk) out[j] = j;
    if (tid == 0) n_idx[b] = s.L;
    return;
  }
  if (s.r <= 0) {  // the forced positions fill the budget
    if (ws.stage == 1) return;
    for (int i = tid; i < s.s_end; i += kThreadsTk) out[i] = i;
    for (int i = tid; i < s.L - s.w_start; i += kThreadsTk) out[s.s_end + i] = s.w_start + i;
    if (tid == 0) n_idx[b] = k;
    return;
  }
  const int R = s.R;
  const int want_stage = stage_want(s, ws);
  uint32_t* first_row = ws.first + (size_t)b * ws.rounds * kThreadsTk;
  const bool after_first = ws.stage == 2;  // the first stage's picks count as taken
  for (int i = tid; i < R * kThreadsTk; i += kThreadsTk) sh.in_bin[i] = 0u;
  if (want_stage <= 0) {
    // nothing to pick in this stage
    for (int i = tid; i < R * kThreadsTk; i += kThreadsTk) sh.taken[i] = after_first ? first_row[i] : 0u;
    __syncthreads();
  } else if (ws.meta[(size_t)b * 4 + 2] > (uint32_t)kFinalCap) {
    // the bin is too big for the list (massive ties): one-workgroup selection
    for (int i = tid; i < R * kThreadsTk; i += kThreadsTk) sh.taken[i] = after_first ? first_row[i] : 0u;
    if (after_first)
      select_stage<false, true>(sh, scores + (size_t)b * max_ctx, max_ctx, R, s.s_end, s.w_start,
                              (uint32_t)want_stage);
    else
      select_stage<false, false>(sh, scores + (size_t)b * max_ctx, max_ctx, R, s.s_end, s.w_start,
                               (uint32_t)want_stage);
  } else {
    const uint32_t prefix0 = ws.meta[(size_t)b * 4 + 0];
    uint32_t want = ws.meta[(size_t)b * 4 + 1];
    const uint32_t nbin0 = ws.meta[(size_t)b * 4 + 2];
    for (int i = tid; i < R * kThreadsTk; i += kThreadsTk)
      sh.taken[i] = ws.bits[(size_t)b * ws.rounds * kThreadsTk + i] | (after_first ? first_row[i] : 0u);
    // the rounds' lists, concatenated
    uint32_t base = 0u;
    for (int q = 0; q < R; ++q) {
      const uint32_t c = ws.cnt[(size_t)b * ws.rounds + q];
      const uint64_t* lq = ws.list + ((size_t)b * ws.rounds + q) * kFinalCap;
      for (uint32_t j = tid; j < c; j += kThreadsTk) cand[base + j] = lq[j];
      base += c;
    }
    if (tid == 0) sh.count = 0u;
    __syncthreads();
    // further radix passes over the list while the bin is big
    uint32_t prefix = prefix0, mask = 0xFFF00000u, nbin = nbin0;
    int level = 1;
    for (; level <= 2 && nbin > (uint32_t)kBinCapOne; ++level) {
      const int shift = level == 1 ? 8 : 0;
      const uint32_t nb = level == 1 ? (uint32_t)kBins : 256u;
      for (int i = tid; i < (int)nb; i += kThreadsTk) sh.hist[i] = 0u;
      __syncthreads();
      for (uint32_t j = tid; j < nbin0; j += kThreadsTk) {
        const uint32_t kk = (uint32_t)(cand[j] >> 32);
        if ((kk & mask) == prefix) atomicAdd(&sh.hist[(kk >> shift) & (nb - 1u)], 1u);
      }
      __syncthreads();
      find_digit(sh.hist, nb, shift, prefix, want, sh.s_wave, sh.s_out);
      nbin = sh.s_out[2];
      mask |= (nb - 1u) << shift;
    }
    const bool exact = nbin > (uint32_t)kBinCapOne;  // all 32 bits resolved: equal keys
    for (uint32_t j = tid; j < nbin0; j += kThreadsTk) {
      const uint64_t cj = cand[j];
      const uint32_t kk = (uint32_t)(cj >> 32), mk = kk & mask;
      const int pos = (int)~(uint32_t)cj;
      if (mk > prefix) {
        atomicOr(&sh.taken[pos >> 5], 1u << (pos & 31));
      } else if (mk == prefix) {
        if (exact) {
          atomicOr(&sh.in_bin[pos >> 5], 1u << (pos & 31));
        } else {
          const uint32_t slot = atomicAdd(&sh.count, 1u);  // < nbin <= kBinCapOne
          sh.bin_rank_key[slot] = cj;
        }
      }
    }
    resolve_bin(sh, nbin, want, exact, R);
  }
  if (ws.stage == 1) {  // keep the picks for the second stage
    for (int i = tid; i < R * kThreadsTk; i += kThreadsTk) first_row[i] = sh.taken[i];
    return;
  }
  emit_taken(sh, R, s.s_end, s.w_start, s.L, s.r, out, idx_stride);
  if (tid == 0) n_idx[b] = k;
}

// ---------------------------------------------------------------------------
// Finish and select in one launch, for rows of up to eight rounds (262144
// positions).
//   * Workgroups [0, B * pieces) aggregate: workgroup (b, piece) sums the
//     collected logits of positions piece * 4096 .. + 4095 below L_b into
//     the scores (aggregate_values: the arithmetic of the aggregation
//     kernel), stores them with device scope, and counts the top 12 key bits
//     of those in M = [s_end, w_start) into an LDS histogram, which it then
//     adds into the row's histogram in the workspace (device-scope atomics,
//     non-empty bins only).  From its own histogram it finds its threshold
//     bin for r and lists its candidates, the keys at or above that bin, in
//     the workspace (rows with r <= kListMaxR; the others select from every
//     score).  It counts itself in once all of that is out; the last
//     of the row's pieces to do so selects the row: it loads the row's
//     histogram (leaving zeros for the next call) and the pieces' counts,
//     finds the threshold bin, then reads the candidate lists, marking the
//     candidates above the bin and ranking those in it.  A bin too large to
//     rank directly (heavy ties) takes the one-workgroup selection over every
//     score instead.  No workgroup waits on another.  A row whose output does
//     not depend on the scores (L <= k, or the forced positions fill the
//     budget) is written by its piece 0.
//   * The workgroups after them combine the split partials, kThreadsTk / (D
//     / 4) rows each (combine_quad, as the combine kernel).
// Aggregation comes first in the grid: its workgroups are dispatched first,
// and the selections start while the combine runs.
constexpr int kAggPos = 4 * kThreadsTk;  // positions per aggregation workgroup
constexpr int kFusedRoundsShort = 2;  // LDS of the selection for rows of up to 65536 positions

struct FinishSelectArgs {
  int32_t k, n_sink, window;
  int32_t* idx;
  int32_t idx_stride;
  int32_t* n_idx;
  uint32_t* hist;   // [B][kBins] key histograms; zero between calls
  int32_t* arrive;  // [B] pieces counted in; zero between calls
  uint32_t* counts; // [B][pieces] candidates each piece listed
  uint64_t* lists;  // [B][pieces][kAggPos] the pieces' candidates
  int32_t pieces;   // aggregation workgroups per sequence
  int32_t n_agg;    // B * pieces
};
constexpr int kMaxPieces = kMaxRounds * kRoundLen / kAggPos;
// Rows list candidates when r is at most a quarter of a piece: a piece then
// lists about r / kAggPos of its positions; with a larger r the lists cost
// more to write and read than the scores they replace.
constexpr int kListMaxR = kAggPos / 4;

// RM: rounds the LDS bitmaps hold (max_ctx <= RM * 32768).
template <int D, int RM>
__global__ __launch_bounds__(kThreadsTk) void finish_select_kernel(CombineArgs c, AggregateArgs ag,
                                                                   FinishSelectArgs f) {
  __shared__ SelectLdsT<RM> sh;
  __shared__ int s_last;
  __shared__ uint32_t s_cnt[kMaxPieces];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= f.n_agg) {
    constexpr int Q = D / 4;
    const int row = ((int)blockIdx.x - f.n_agg) * (kThreadsTk / Q) + tid / Q;
    const int chunk = min(max(c.header[0], kTile), c.chunk);
    if (row < c.rows) combine_quad<D>(c, row, tid % Q, chunk);
    return;
  }
  const int b = (int)blockIdx.x / f.pieces, piece = (int)blockIdx.x % f.pieces;
  const SelRow s = sel_row(b, ag.max_ctx, ag.seq_lens, f.k, f.n_sink, f.window);
  int32_t* out = f.idx + (size_t)b * f.idx_stride;
  if (s.trivial && piece == 0) {
    if (s.L <= f.k) {
      for (int j = tid; j < s.L; j += kThreadsTk) out[j] = j;
      if (tid == 0) f.n_idx[b] = s.L;
    } else {
      for (int i = tid; i < s.s_end; i += kThreadsTk) out[i] = i;
      for (int i = tid; i < s.L - s.w_start; i += kThreadsTk) out[s.s_end + i] = s.w_start + i;
      if (tid == 0) f.n_idx[b] = f.k;
    }
  }
  const int j0 = piece * kAggPos;
  if (j0 >= s.L) return;  // no position here (and not counted in)

  if (!s.trivial)
    for (int i = tid; i < kBins; i += kThreadsTk) sh.hist[i] = 0u;
  __syncthreads();
  float* srow = ag.scores + (size_t)b * ag.max_ctx;
  float val[4];
  aggregate_values<4>(ag, b, j0 + tid, kThreadsTk, s.L, val);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = j0 + tid + u * kThreadsTk;
    if (j < s.L) {
      store1_device(srow, (uint32_t)j * 4u, val[u]);
      if (!s.trivial && j >= s.s_end && j < s.w_start) atomicAdd(&sh.hist[order_key(val[u]) >> 20], 1u);
    }
  }
  if (s.trivial) return;
  __syncthreads();
  uint32_t* gh = f.hist + (size_t)b * kBins;
  for (int i = tid; i < kBins; i += kThreadsTk) {
    const uint32_t h = sh.hist[i];
    if (h != 0u) atomicAdd(gh + i, h);
  }
  // The piece's candidates: its eligible keys at or above its own threshold
  // bin for r (a key of a lower bin has r keys of this piece above it, so it
  // is never selected; every key when the piece holds fewer than r), listed
  // as key << 32 | ~position in thread order.  The selecting workgroup reads
  // these lists instead of every score of the row.
  const bool lists = s.r <= kListMaxR;
  if (lists) {
    if (tid == 0) sh.s_out[0] = 0u;
    const uint32_t floor_bin =
        find_digit_v(sh.hist, kBins, 20, 0u, (uint32_t)s.r, sh.s_wave, sh.s_out).x >> 20;
    uint32_t key[4], cand = 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + tid + u * kThreadsTk;
      key[u] = order_key(val[u]);
      if (j < s.L && j >= s.s_end && j < s.w_start && (key[u] >> 20) >= floor_bin) cand |= 1u << u;
    }
    const uint2 sc = block_scan((uint32_t)__builtin_popcount(cand), sh.s_wave);
    float* lst = reinterpret_cast<float*>(f.lists + ((size_t)b * f.pieces + piece) * kAggPos);
    uint32_t o = sc.x;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if ((cand >> u) & 1u) {
        const uint64_t e = ((uint64_t)key[u] << 32) | (uint32_t)~(uint32_t)(j0 + tid + u * kThreadsTk);
        store2_device(lst, o++ * 8u, __builtin_bit_cast(float2, e));
      }
    if (tid == 0)
      store1_device(reinterpret_cast<float*>(f.counts), (uint32_t)(b * f.pieces + piece) * 4u,
                    __uint_as_float(sc.y));
  }
  // every store and histogram add of this workgroup has completed before it
  // counts itself in
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int n_pieces = (s.L + kAggPos - 1) / kAggPos;
    const int done = atomicAdd(f.arrive + b, 1) + 1;
    s_last = done == n_pieces;
    if (done == n_pieces) atomicExch(f.arrive + b, 0);  // ready for the next call
  }
  __syncthreads();
  if (!s_last) return;

  // select from the row's histogram (every piece has added to it), then
  // leave it zero for the next call
  for (int i = tid; i < s.R * kThreadsTk; i += kThreadsTk) {
    sh.taken[i] = 0u;
    sh.in_bin[i] = 0u;
  }
  // The histogram and the pieces' candidate counts, loaded together; the
  // threshold bin from the histogram.
  const int np = (s.L + kAggPos - 1) / kAggPos;  // <= kMaxPieces
  if (lists) {
    uint32_t h[kBins / kThreadsTk];
#pragma unroll
    for (int q = 0; q < kBins / kThreadsTk; ++q)
      h[q] = __float_as_uint(load1_device(reinterpret_cast<const float*>(gh), (uint32_t)(tid + q * kThreadsTk) * 4u));
    const uint32_t cn = tid < np ? __float_as_uint(load1_device(reinterpret_cast<const float*>(f.counts),
                                                                (uint32_t)(b * f.pieces + tid) * 4u))
                                 : 0u;
#pragma unroll
    for (int q = 0; q < kBins / kThreadsTk; ++q) sh.hist[tid + q * kThreadsTk] = h[q];
    if (tid < np) s_cnt[tid] = cn;
    if (tid == 0) sh.count = 0u;
    __syncthreads();
  }
  uint32_t prefix = 0u, want = (uint32_t)s.r;
  if (lists) find_digit(sh.hist, kBins, 20, prefix, want, sh.s_wave, sh.s_out);
  if (lists && sh.s_out[2] <= (uint32_t)kBinCapMany) {
    // Candidates above the threshold bin are taken; the bin's are ranked.
    // Every selected position is a candidate of its piece, and so is every
    // member of the bin that ranks among the `want` best, so ranking the
    // listed members decides the bin.  Piece p goes to the wavefronts w with
    // w mod np = p (or w to pieces w, w + 16, .. when np > 16), eight loads
    // per lane in flight.
    const int lane = tid & 63, wave = tid >> 6;
    const uint32_t tb = prefix >> 20;
    for (int p = wave % np; p < np; p += kWavesTk) {
      const int kw = np <= kWavesTk ? (kWavesTk - 1 - p) / np + 1 : 1;  // wavefronts on piece p
      const int k0 = np <= kWavesTk ? wave / np : 0;
      const uint32_t n = s_cnt[p];
      const float* lst = reinterpret_cast<const float*>(f.lists + ((size_t)b * f.pieces + p) * kAggPos);
      const uint32_t stride = (uint32_t)kw * 64u;
      for (uint32_t e0 = (uint32_t)k0 * 64u + lane; e0 < n; e0 += 8u * stride) {
        uint64_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t e = min(e0 + i * stride, n - 1u);
          v[i] = __builtin_bit_cast(uint64_t, load2_device(lst, e * 8u));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (e0 + i * stride >= n) break;
          const uint32_t key = (uint32_t)(v[i] >> 32), pos = ~(uint32_t)v[i];
          if ((key >> 20) > tb) {
            atomicOr(&sh.taken[pos >> 5], 1u << (pos & 31));
          } else if ((key >> 20) == tb) {
            const uint32_t slot = atomicAdd(&sh.count, 1u);  // < the bin's size <= kBinCap
            sh.bin_rank_key[slot] = v[i];
          }
        }
      }
    }
    __syncthreads();
    resolve_bin(sh, sh.count, want, false, s.R);
  } else {
    // no lists (r above kListMaxR), or a bin too large to rank directly
    // (heavy ties): every score of the row
    select_stage<false, false, true, true>(sh, srow, ag.max_ctx, s.R, s.s_end, s.w_start,
                                           (uint32_t)s.r, gh);
  }
  emit_taken(sh, s.R, s.s_end, s.w_start, s.L, s.r, out, f.idx_stride);
  if (tid == 0) f.n_idx[b] = f.k;
  for (int i = tid; i < kBins; i += kThreadsTk) store1_device(reinterpret_cast<float*>(gh), (uint32_t)i * 4u, 0.f);
}

}  // namespace

hipError_t launch_select_topk(int32_t batch, int32_t max_ctx, const float* scores,
                              const float* draft_scores, const int32_t* seq_lens, int32_t k,
                              int32_t m, int32_t n_sink, int32_t window, int32_t* idx,
                              int32_t idx_stride, int32_t* n_idx, hipStream_t stream) {
  const bool hybrid = draft_scores != nullptr;
  const int rounds = (max_ctx + kRoundLen - 1) / kRoundLen;
  const dim3 grid(batch), block(kThreadsTk);
  const auto args = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, max_ctx, scores, draft_scores, seq_lens, k,
                       m, n_sink, window, idx, idx_stride, n_idx);
  };
  if (rounds <= kMaxRounds) {
    if (hybrid) args(select_topk_kernel<true>); else args(select_topk_kernel<false>);
  } else {
    if (hybrid) return hipErrorInvalidValue;  // rows past kMaxRounds rounds: plain selection only
    hipLaunchKernelGGL(select_topk_large_kernel, grid, block, 0, stream, max_ctx, scores, seq_lens,
                       k, n_sink, window, idx, idx_stride, n_idx);
  }
  return hipGetLastError();
}

size_t select_workspace_bytes(int32_t batch, int32_t max_ctx) {
  const int64_t rounds = ((int64_t)max_ctx + kRoundLen - 1) / kRoundLen;
  // Up to 1.5 rounds the one-workgroup kernel is as fast (its rows may well
  // fit one round, e.g. a capacity with headroom for drafted tokens), and
  // one launch beats three.
  if (batch < 1 || max_ctx <= kRoundLen + kRoundLen / 2 || rounds > kMaxRounds) return 0;
  const size_t per_row =
      (size_t)rounds * (kBins * 4 + 2 * kThreadsTk * 4 + (size_t)kFinalCap * 8 + 4) + 16;
  return ((size_t)batch * per_row + 5 * 256 + 255) / 256 * 256;
}

hipError_t launch_select_topk_split(int32_t batch, int32_t max_ctx, const float* scores,
                                    const float* draft_scores, const int32_t* seq_lens, int32_t k,
                                    int32_t m, int32_t n_sink, int32_t window, int32_t* idx,
                                    int32_t idx_stride, int32_t* n_idx, void* workspace,
                                    hipStream_t stream) {
  const int rounds = (max_ctx + kRoundLen - 1) / kRoundLen;
  if (rounds < 2 || rounds > kMaxRounds) return hipErrorInvalidValue;
  const auto al16 = [](const float* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = max_ctx % 4 == 0 && al16(scores) && (draft_scores == nullptr || al16(draft_scores));
  // carve the workspace: 256-byte aligned arrays
  char* p = static_cast<char*>(workspace);
  auto take = [&](size_t bytes) {
    char* q = p;
    p += (bytes + 255) / 256 * 256;
    return q;
  };
  SelWorkspace ws;
  ws.rounds = rounds;
  ws.list = reinterpret_cast<uint64_t*>(take((size_t)batch * rounds * kFinalCap * 8));
  ws.hist = reinterpret_cast<uint32_t*>(take((size_t)batch * rounds * kBins * 4));
  ws.bits = reinterpret_cast<uint32_t*>(take((size_t)batch * rounds * kThreadsTk * 4));
  ws.cnt = reinterpret_cast<uint32_t*>(take((size_t)batch * rounds * 4));
  ws.meta = reinterpret_cast<uint32_t*>(take((size_t)batch * 16));
  ws.first = reinterpret_cast<uint32_t*>(take((size_t)batch * rounds * kThreadsTk * 4));
  ws.m = m;
  const dim3 grid_r(rounds, batch), grid_b(batch), block(kThreadsTk);
  // hybrid: the first stage on the draft scores, then the second on the
  // target scores; otherwise one stage
  const int n_stages = draft_scores != nullptr ? 2 : 1;
  for (int st = 0; st < n_stages; ++st) {
    ws.stage = draft_scores == nullptr ? 0 : st + 1;
    const float* sc = ws.stage == 1 ? draft_scores : scores;
    if (vec) {
      hipLaunchKernelGGL(select_round_hist_kernel<true>, grid_r, block, 0, stream, max_ctx, sc,
                         seq_lens, k, n_sink, window, ws);
      hipLaunchKernelGGL(select_round_mark_kernel<true>, grid_r, block, 0, stream, max_ctx, sc,
                         seq_lens, k, n_sink, window, ws);
    } else {
      hipLaunchKernelGGL(select_round_hist_kernel<false>, grid_r, block, 0, stream, max_ctx, sc,
                         seq_lens, k, n_sink, window, ws);
      hipLaunchKernelGGL(select_round_mark_kernel<false>, grid_r, block, 0, stream, max_ctx, sc,
                         seq_lens, k, n_sink, window, ws);
    }
    hipLaunchKernelGGL(select_final_kernel, grid_b, block, 0, stream, max_ctx, sc, seq_lens, k,
                       n_sink, window, idx, idx_stride, n_idx, ws);
  }
  return hipGetLastError();
}

hipError_t launch_select_blocks(int32_t batch, int32_t max_ctx, const float* scores,
                                const int32_t* seq_lens, int32_t k_blocks, int32_t block,
                                int32_t n_sink, int32_t window, int32_t* idx, int32_t idx_stride,
                                int32_t* n_idx, float* block_sums, bool ids, hipStream_t stream) {
  if ((max_ctx + block - 1) / block > kMaxSelBlocks) return hipErrorInvalidValue;
  const bool vec = max_ctx % 4 == 0 && block % 4 == 0 &&
                   (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  const dim3 grid(batch), block_dim(kThreadsTk);
  const auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block_dim, 0, stream, max_ctx, scores, seq_lens, k_blocks,
                       block, n_sink, window, idx, idx_stride, n_idx, block_sums);
  };
  if (ids) {
    if (vec) go(select_blocks_kernel<true, true>); else go(select_blocks_kernel<false, true>);
  } else {
    if (vec) go(select_blocks_kernel<true, false>); else go(select_blocks_kernel<false, false>);
  }
  return hipGetLastError();
}

// [B][kBins] histograms, [B] arrival counters, [B][pieces] candidate
// counts, [B][pieces][kAggPos] candidates; 256-byte aligned parts.
size_t finish_select_workspace_bytes(int32_t batch, int32_t max_ctx) {
  const size_t pieces = ((size_t)max_ctx + kAggPos - 1) / kAggPos;
  const auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  return al((size_t)batch * kBins * 4) + al((size_t)batch * 4) + al((size_t)batch * pieces * 4) +
         al((size_t)batch * pieces * kAggPos * 8);
}

hipError_t launch_finish_select(const CombineArgs& c, const AggregateArgs& ag, int32_t k,
                                int32_t n_sink, int32_t window, int32_t* idx, int32_t idx_stride,
                                int32_t* n_idx, void* workspace, hipStream_t stream) {
  if (ag.max_ctx > kMaxRounds * kRoundLen || ag.scores == nullptr) return hipErrorInvalidValue;
  FinishSelectArgs f;
  f.k = k;
  f.n_sink = n_sink;
  f.window = window;
  f.idx = idx;
  f.idx_stride = idx_stride;
  f.n_idx = n_idx;
  f.pieces = (ag.max_ctx + kAggPos - 1) / kAggPos;
  const auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  char* w = static_cast<char*>(workspace);
  f.hist = reinterpret_cast<uint32_t*>(w);
  w += al((size_t)ag.batch * kBins * 4);
  f.arrive = reinterpret_cast<int32_t*>(w);
  w += al((size_t)ag.batch * 4);
  f.counts = reinterpret_cast<uint32_t*>(w);
  w += al((size_t)ag.batch * f.pieces * 4);
  f.lists = reinterpret_cast<uint64_t*>(w);
  f.n_agg = ag.batch * f.pieces;
  const int q = c.head_dim / 4;
  const int n_comb = (c.rows + kThreadsTk / q - 1) / (kThreadsTk / q);
  const dim3 grid((unsigned)(f.n_agg + n_comb)), block(kThreadsTk);
  const bool short_rows = ag.max_ctx <= kFusedRoundsShort * kRoundLen;
  const auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, c, ag, f);
  };
  if (c.head_dim == 64) {
    if (short_rows) go(finish_select_kernel<64, kFusedRoundsShort>);
    else go(finish_select_kernel<64, kMaxRounds>);
  } else {
    if (short_rows) go(finish_select_kernel<128, kFusedRoundsShort>);
    else go(finish_select_kernel<128, kMaxRounds>);
  }
  return hipGetLastError();
}

}  // namespace vgsa
