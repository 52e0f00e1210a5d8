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
// Layout of the work: one workgroup per (split, kv-head, sequence); its
// wavefronts (four or eight) take 32-position tiles of the split in turn.  All
// G*T query rows that share the kv-head live in one wavefront as 16-row MFMA
// blocks, so every K/V byte is read from HBM once.  (A sparse pass with one
// split shares the rows between two workgroups on one XCD instead: both
// gather every listed row, the second read coming from that XCD's L2.)  Per
// tile a wavefront:
//   1. loads 32 K rows and 32 V rows with 16-byte loads (prefetched one tile
//      ahead in registers),
//   2. computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (positions are the
//      M side, query rows the N side),
//   3. writes the collected logits: per head straight to HBM, or summed over
//      the kv-group into an LDS copy of the chunk that goes out in one burst
//      after the loop (the sum comes from two extra query columns holding
//      the summed collected queries when the group leaves them free, else
//      from a cross-lane reduction),
//   4. runs an online softmax in log2 units per query row,
//   5. accumulates O^T += V^T P^T with the same MFMA; P comes straight from
//      the S^T accumulators, V^T is read from a per-wavefront LDS tile.
// The wavefronts are merged through LDS at the end and the workgroup writes
// its un-normalised partial (o, m, l) for the combine kernel, or with one
// split the normalised output itself.
#include "internal.h"
#include "merge_ops.h"

namespace vgsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ bf16x8 load16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}


// K/V rows are read once per launch: nontemporal loads stream them past the
// caches.  Each wavefront load instruction covers whole rows (1 KB contiguous
// per instruction for contiguous caches), the shape that streams fastest.
__device__ __forceinline__ u32x4 load16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Waves per SIMD the register budget is sized for: two (<= 256 registers per
// wave) unless four query blocks of d = 128 need more.
template <int D, int QB>
struct Occupancy {
  static constexpr int kWavesPerEU = (D == 128 && QB == 4) ? 1 : 2;
};

// Kv-group-summed logits taken straight from the MFMA: the logit sum over the
// collected rows of the group is K . (sum of their scaled queries), so the
// summed query, split into a bf16 high part and the bf16 rounding of the
// remainder (about 16 significant bits together), rides in the last two
// query columns of the last 16-row block when the group leaves them free.
// Internal emit mode; the layout written is VGSA_LOGITS_KVGROUP_SUM.
constexpr int kEmitSumColumn = 3;

// Lane moves within 16-lane rows (DPP: VALU only, no LDS crossbar traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                                           0xF, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm 1,0,3,2: lane i <- i ^ 1
constexpr int kDppXor2 = 0x4E;        // quad_perm 2,3,0,1: lane i <- i ^ 2
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane i <- i ^ 7 (within 8 lanes)
constexpr int kDppXor8 = 0x128;       // row_ror:8: lane i <- i ^ 8 (within 16 lanes)

__device__ __forceinline__ float swap_adjacent_lanes(float x) {  // lane i <-> lane i ^ 1
  return dpp_move<kDppXor1>(x);
}

// Lanes i and i ^ 16 (ROWS = true) or i and i ^ 32: both values of the pair,
// the lower lane's first, in both lanes (gfx950 permlane swaps: VALU, no LDS
// crossbar traffic).
template <bool ROWS>
__device__ __forceinline__ void lane_pair(float x, float& lo, float& hi) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  if constexpr (ROWS) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    lo = __builtin_bit_cast(float, (unsigned)r[0]);
    hi = __builtin_bit_cast(float, (unsigned)r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __builtin_bit_cast(float, (unsigned)r[0]);
    hi = __builtin_bit_cast(float, (unsigned)r[1]);
  }
}

// Max and sum over lanes i, i ^ 16, i ^ 32, i ^ 48 (one 16-lane column).
__device__ __forceinline__ float column_max(float x) {
  float lo, hi;
  lane_pair<true>(x, lo, hi);
  lane_pair<false>(fmaxf(lo, hi), lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float column_sum(float x) {
  float lo, hi;
  lane_pair<true>(x, lo, hi);
  lane_pair<false>(lo + hi, lo, hi);
  return lo + hi;
}

// Lazy rescaling: a row's running max is only raised (and O, l rescaled)
// when a tile exceeds it by more than 2^kRescaleLog2; otherwise the stale max
// is kept, so p <= 2^kRescaleLog2.  The combine uses the same (m, l, O)
// triple, so the result is exact.
constexpr float kRescaleLog2 = 8.0f;

// D: head dim (64/128); QB: 16-row query blocks (G*T <= 16*QB); SPARSE: index
// list; EMIT: logit layout written by the verify pass (VGSA_LOGITS_*).
// WAVES: wavefronts per workgroup (4 for split launches; 8 for one-split
// sparse launches, so a short index list is covered in fewer serial tiles).
template <int D, int QB, bool SPARSE, int EMIT, int WAVES>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(Occupancy<D, QB>::kWavesPerEU, Occupancy<D, QB>::kWavesPerEU)))
void attn_partials_kernel(AttnArgs a) {
  constexpr int NT = WAVES * 64;   // threads per workgroup
  constexpr int KS = D / 32;       // MFMA steps over the head dimension
  constexpr int DB = D / 16;       // 16-wide blocks of the head dimension
  constexpr int VS = D + 16;       // V tile row stride (elements): rows land 32 B apart in the banks
  // Per-wavefront K/V tiles, [position][d]; reused at the end as the fp32
  // merge buffers.
  __shared__ __align__(16) uint16_t sbuf[WAVES * kTile * VS];
  // Summed collected query (kv-group logits through the MFMA): in the last
  // block's two spare columns, 14 (bf16 high part) and 15 (low part).
  constexpr bool kSumQuery = EMIT == kEmitSumColumn;
  constexpr int kSumCol = 14;
  // Query fragments, already in MFMA operand order: [qb][ks][lane] x 16 B.
  __shared__ __align__(16) u32x4 sq[QB * KS * 64];
  __shared__ int s_idx[WAVES][kTile];           // sparse: positions of the staged tile
  __shared__ uint32_t s_row[WAVES][kTile];      // sparse: cache element offsets of those rows
  // One array, three uses in turn:
  //  * slog, the kv-group logits of the chunk: held here and written out in
  //    contiguous bursts once the loop is done.  Stores issued while the K/V
  //    stream runs cost far more than their bytes: one 4096-position burst
  //    per workgroup in mid-chunk cost 3 % of the verify time.  Wide
  //    layouts hold a whole chunk (kMaxChunkWide positions), contiguous or
  //    paged; narrow ones kLogitBufMax (contiguous) or kLogitBuf (paged)
  //    positions, flushed whenever full;
  //  * s_blk, the paged verify's block ids of the chunk, in the top
  //    kMaxChunk / 16 entries (beyond the logit buffer);
  //  * after the loop (logits out, block ids no longer read): the merge's
  //    per-wavefront row max and sum and the rows' 1 / sum.
  constexpr bool kWide = WAVES == kWavesWide;
  constexpr int kChunkMax = kWide ? kMaxChunkWide : kMaxChunk;
  constexpr int kLogCap = kWide ? kMaxChunkWide : kLogitBufMax;       // contiguous caches
  constexpr int kLogCapPaged = kWide ? kMaxChunkWide : kLogitBuf;     // paged caches
  constexpr bool kGroupLogits = EMIT == VGSA_LOGITS_KVGROUP_SUM || kSumQuery;
  constexpr int kBlkIds = SPARSE ? 0 : kChunkMax / 16;
  constexpr int kRowStats = 2 * WAVES * kMaxRows + kMaxRows;
  constexpr int kShared = kGroupLogits ? (kWide ? kLogCap + kBlkIds : kLogitBufMax)
                                       : (kBlkIds > kRowStats ? kBlkIds : kRowStats);
  static_assert(!kGroupLogits || kLogCapPaged + kBlkIds <= kShared, "logits meet block ids");
  static_assert(!kGroupLogits || kLogCap <= kShared, "logit buffer does not fit");
  static_assert(kRowStats <= kShared, "row statistics do not fit");
  __shared__ __align__(16) float sx[kShared];
  float* const slog = sx;
  int* const s_blk = reinterpret_cast<int*>(sx + kShared - kBlkIds);
  float (*const s_m)[kMaxRows] = reinterpret_cast<float (*)[kMaxRows]>(sx);
  float (*const s_l)[kMaxRows] = reinterpret_cast<float (*)[kMaxRows]>(sx + WAVES * kMaxRows);
  float* const s_inv = sx + 2 * WAVES * kMaxRows;  // 1 / (merged row sum), one-split output
  // Per-head logits: each wavefront turns its 16 x 32 tile of one row block
  // around in LDS so that a store instruction writes two rows' 32 positions
  // as contiguous 128-byte runs (any row alignment); s_lrow[m] is the element
  // offset of query row m's logit row, -1 when the row is not collected.
  constexpr int kHS = kTile + 4;  // row stride of the turned tile (floats)
  constexpr bool kHeadLogits = EMIT == VGSA_LOGITS_PER_HEAD;
  __shared__ __align__(16) float shl[kHeadLogits ? WAVES * 16 * kHS : 4];
  __shared__ int64_t s_lrow[kHeadLogits ? QB * 16 : 1];

  int g = blockIdx.y, split = blockIdx.x, b = blockIdx.z, chunk = a.chunk;
  // Row-split sparse launch (one split): a 1-D grid whose linear ids x + 8*(2j)
  // and x + 8*(2j + 1) (one XCD: ids are dealt to the XCDs in turn) take the
  // two halves of the query rows of (sequence, kv-head) pair x + 8*j; the
  // grid is rounded up to whole rounds of 16, and ids past the pairs leave.
  int half = 0;
  if (SPARSE && a.row_split > 1) {
    const int id = blockIdx.x, pair = (id & 7) + 8 * (id >> 4);
    if (pair >= a.batch * a.hkv) return;
    half = (id >> 3) & 1;
    b = pair / a.hkv;
    g = pair % a.hkv;
    split = 0;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, kg = lane >> 4;
  // Ragged verify batches of up to 64 sequences: lane i holds sequence i's
  // length (a buffer load bounded by the array: lanes past it read 0) and
  // the item is derived across the lanes (below).
  const bool lane_lens = !SPARSE && a.balance && a.batch <= 64;
  int len_lane = 0;
  if (lane_lens)
    len_lane = min(max((int)__builtin_amdgcn_raw_buffer_load_b32(
                           __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.seq_lens), 0, a.batch * 4,
                                                             kRawBufferWord3),
                           (uint32_t)lane * 4u, 0, 0),
                       0),
                   a.max_ctx);

  // Ragged batches (verify): every workgroup derives the same item length
  // from the lengths, short enough that the non-empty items of a kv-head fill
  // its S * B workgroups, and takes one of them (below): the longest
  // workgroup then has about the mean work, not the longest row's.
  int L_item = -1;  // the item's sequence length, when the lanes hold it
  if (lane_lens) {
    // The same item lengths and mapping as below, with lane i standing for
    // sequence i: a count over the sequences is one division per lane and a
    // wave sum.
    const int S = a.num_splits, B = a.batch;
    // (the sum in two 16-bit halves: each half's wave sum fits 32 bits)
    const uint32_t len_u = (uint32_t)len_lane;
    const int64_t total = ((int64_t)wave_total(len_u >> 16) << 16) + (int64_t)wave_total(len_u & 0xFFFFu);
    const int64_t fit = (total + (int64_t)S * B - B - 1) / ((int64_t)S * B - B);  // S > 1 here
    constexpr int MC = (kWide && !SPARSE) ? kTile : WAVES * kTile;
    const int floor_len = (a.chunk / kBalanceSplits + MC - 1) / MC * MC;
    int cp = (int)min((int64_t)a.chunk, max((int64_t)floor_len, (fit + MC - 1) / MC * MC));
    const int SB = S * B;
    // items of this lane's sequence at item length c, capped (the sum then fits 32 bits)
    auto n_items = [&](int c) { return min((len_lane + c - 1) / c, SB + 1); };
    {
      int lo = max(floor_len, (int)(((total + SB - 1) / SB + MC - 1) / MC * MC));
      int hi = cp;
      while (lo < hi) {
        const int mid = max(lo, (lo + hi) / 2 / MC * MC);
        if ((int)wave_total((uint32_t)n_items(mid)) <= SB) hi = mid; else lo = mid + MC;
      }
      cp = hi;
    }
    const int it = (len_lane + cp - 1) / cp;  // items of sequence `lane` (0 past the batch)
    const int nb = __builtin_amdgcn_readlane(it, b);
    int bi = -1, si = 0;
    if (split < nb) {
      bi = b;
      si = split;
    } else {
      // rank among the free workgroups, then the sequence whose items past S
      // hold that rank (in sequence order)
      const int r = split - nb + (int)wave_total(lane < b ? (uint32_t)max(0, S - it) : 0u);
      const int o = max(0, it - S);
      const int pre = (int)wave_inclusive_scan((uint32_t)o);  // items past S of sequences 0 .. lane
      const uint64_t hit = __ballot(r < pre);
      if (hit != 0ull) {
        bi = __builtin_ctzll(hit);
        si = S + (r - (__builtin_amdgcn_readlane(pre, bi) - __builtin_amdgcn_readlane(o, bi)));
      }
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) a.header[0] = cp;
    if (bi < 0) return;  // more workgroups than items
    L_item = __builtin_amdgcn_readlane(len_lane, bi);
    b = bi;
    split = si;
    chunk = cp;
  } else if (!SPARSE && a.balance) {
    const int S = a.num_splits, B = a.batch;
    int64_t total = 0;
    for (int i = 0; i < B; ++i) total += min(max(a.seq_lens[i], 0), a.max_ctx);
    const int64_t fit = (total + (int64_t)S * B - B - 1) / ((int64_t)S * B - B);  // S > 1 here
    // item granularity: a tile when the wavefronts claim tiles, else one
    // step of every wavefront
    constexpr int MC = (kWide && !SPARSE) ? kTile : WAVES * kTile;
    const int floor_len = (a.chunk / kBalanceSplits + MC - 1) / MC * MC;
    int cp = (int)min((int64_t)a.chunk, max((int64_t)floor_len, (fit + MC - 1) / MC * MC));
    // cp above always fits (the items of a sequence number at most L / cp +
    // 1); the smallest item length that still gives at most S * B items is
    // found by bisection in steps of MC.  For lengths 12536, 60439, 51539,
    // 12189 over 32 workgroups per kv-head it gives 32 items of 4320
    // positions (an even split is 4272) instead of 29 of 5120.
    {
      const int64_t SB = (int64_t)S * B;
      auto fits = [&](int c) {
        int64_t n = 0;
        for (int i = 0; i < B; ++i) n += (min(max(a.seq_lens[i], 0), a.max_ctx) + c - 1) / c;
        return n <= SB;
      };
      int lo = max(floor_len, (int)(((total + SB - 1) / SB + MC - 1) / MC * MC));
      int hi = cp;
      while (lo < hi) {
        const int mid = max(lo, (lo + hi) / 2 / MC * MC);
        if (fits(mid)) hi = mid; else lo = mid + MC;
      }
      cp = hi;
    }
    // A sequence keeps its first S items on its own workgroups (split < n),
    // so equal lengths map as without balancing; the items past S of long
    // sequences go, in order, to the workgroups that short sequences leave
    // free (split >= n).  The items number at most S * B, so every one has
    // a workgroup.  (Which K/V rows stream together matters: handing each
    // sequence's items to the next sequence's workgroups measured 17 %
    // slower at 128K x b8 with 17 splits.)
    auto items = [&](int i) { return (min(max(a.seq_lens[i], 0), a.max_ctx) + cp - 1) / cp; };
    const int nb = items(b);
    int bi = -1, si = 0;
    if (split < nb) {
      bi = b;
      si = split;
    } else {
      int r = split - nb;  // rank among the free workgroups, in (sequence, split) order
      for (int i = 0; i < b; ++i) r += max(0, S - items(i));
      int acc = 0;
      for (int i = 0; i < B && bi < 0; ++i) {
        const int o = max(0, items(i) - S);
        if (r < acc + o) {
          bi = i;
          si = S + (r - acc);
        }
        acc += o;
      }
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) a.header[0] = cp;
    if (bi < 0) return;  // more workgroups than items
    b = bi;
    split = si;
    chunk = cp;
  } else if (!a.direct && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 &&
             threadIdx.x == 0) {
    a.header[0] = chunk;
  }

  const int start = split * chunk;
  // Sparse: the list entries of this wavefront's first kPreTiles tiles are
  // loaded (clamped in bounds) together with the lengths, so those tiles
  // need no index round trip of their own.
  // Block lists (id_block = B > 1): entry e of the position list is
  // position ids[e / B] * B + e % B.
  constexpr int kPreTiles = 4;
  const int B_id = SPARSE ? a.id_block : 1;
  int idx_pre[kPreTiles];
#pragma unroll
  for (int i = 0; i < kPreTiles; ++i) {
    idx_pre[i] = 0;
    if (SPARSE && lane < kTile) {
      const int e = start + (i * WAVES + wave) * kTile + lane;
      if (B_id == 1) {
        idx_pre[i] = a.idx[(size_t)b * a.idx_stride + min(e, a.idx_stride - 1)];
      } else {
        const int blk_e = min(e / B_id, a.idx_stride - 1);
        idx_pre[i] = a.idx[(size_t)b * a.idx_stride + blk_e] * B_id + (e - blk_e * B_id);
      }
    }
  }
  const int L = L_item >= 0 ? L_item : min(max(a.seq_lens[b], 0), a.max_ctx);
  const int32_t* btab = a.paged ? a.block_table + (size_t)b * a.max_blocks : nullptr;
  // Paged sparse: block ids of the preloaded entries, fetched together.
  int blk_pre[kPreTiles];
#pragma unroll
  for (int i = 0; i < kPreTiles; ++i) {
    blk_pre[i] = 0;
    if (SPARSE && lane < kTile && a.paged)
      blk_pre[i] = btab[min(max(idx_pre[i], 0), max(L - 1, 0)) >> 4];
  }
  // sparse: the listed entries, then (virtually) the last `tail` positions
  // below L, e.g. the tokens drafted since the selection
  const int tail = SPARSE ? min(a.tail, L) : 0;
  int nlist = SPARSE ? min(max(a.n_idx[b], 0), a.idx_stride) : 0;
  if (SPARSE && B_id > 1 && nlist > 0) {
    // every position of the listed blocks below L - tail (only the last
    // listed block can reach past it)
    const int last = a.idx[(size_t)b * a.idx_stride + nlist - 1];
    nlist = (nlist - 1) * B_id + min(B_id, max(0, L - tail - last * B_id));
  } else if (SPARSE && B_id > 1) {
    nlist = 0;
  }
  const int count = SPARSE ? nlist + tail : L;
  const int G = a.group, T = a.q_len;
  // This workgroup's query rows: the group's G*T, or (row-split sparse) one
  // half of them, from the group's row r0.
  const bool halves = SPARSE && a.row_split > 1;
  const int rows_half = (G * T + 1) / 2;
  const int r0 = halves ? half * rows_half : 0;
  const int rows = halves ? min(G * T - r0, rows_half) : G * T;
  // Rows [B][Hq][T] of this kv-group are contiguous: row r0 + m = hh*T + t of
  // the group (q-head g*G + hh, query t) is row row_base + m.
  const size_t row_base = ((size_t)b * a.hq + (size_t)g * G) * T + r0;
  if (start >= count) {  // whole workgroup: nothing in this split
    // the only split, or (fused merge) an empty list that no workgroup
    // merges: the rows see nothing -> o = 0, lse = -inf
    if (a.direct || (a.fuse && split == 0)) {
      for (int e = threadIdx.x; e < rows * D; e += NT) a.out[row_base * D + e] = 0;
      if (a.lse != nullptr && (int)threadIdx.x < rows) a.lse[row_base + threadIdx.x] = kNegInf;
    }
    return;
  }
  const int end = min(start + chunk, count);

  // Collected heads of this kv-group: bit hh for q-head g*G + hh (a head
  // subset needs Hq <= 64, checked on the host).
  const uint64_t all_g = G >= 64 ? ~0ull : (1ull << G) - 1ull;
  const uint64_t gmask = a.head_mask == kAllHeads ? all_g : (a.head_mask >> (g * G)) & all_g;

  // This lane's query column c16 of block qb: causal limit and collected row.
  int lim[QB], rowc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int m = qb * 16 + c16;
    const bool ok = m < rows;
    const int hh = ok ? (r0 + m) / T : 0, t = ok ? (r0 + m) % T : 0;
    lim[qb] = ok ? L - T + t : 0x7fffffff;  // row t sees positions <= L - T + t
    // collected row of a collected head: its rank among the collected rows
    rowc[qb] = (EMIT != VGSA_LOGITS_NONE && ok && ((a.row_mask >> t) & 1u) && ((gmask >> hh) & 1ull))
                   ? __builtin_popcount(a.row_mask & ((1u << t) - 1u)) : -1;
    if (kHeadLogits && threadIdx.x < 16) {
      // per-head row: [b][collected row][collected head][position]
      const int head = g * G + hh;
      const int hrank = a.head_mask == kAllHeads
                            ? head : __builtin_popcountll(a.head_mask & ((1ull << head) - 1ull));
      s_lrow[m] = rowc[qb] < 0
                      ? -1 : (((int64_t)b * a.n_rows + rowc[qb]) * a.n_heads + hrank) * a.max_ctx;
    }
  }
  const int lim_min = L - T;  // every row sees positions <= L - T
  // kv-group logits: the softmax scale for a collected row of this lane, else 0
  float rowc_w[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) rowc_w[qb] = rowc[qb] >= 0 ? a.scale : 0.f;
  // per-head logits: the collected rows of block qb, bit c16 (wave-uniform),
  // so blocks and row pairs with nothing to write are skipped
  uint32_t cmask[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
    cmask[qb] = kHeadLogits ? (uint32_t)(__ballot(rowc[qb] >= 0) & 0xFFFFull) : 0u;

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

  uint16_t* vt = sbuf + wave * kTile * VS;  // this wavefront's K/V tile
  int* sidx = s_idx[wave];
  uint32_t* srow = s_row[wave];
  const int step = WAVES * kTile;

  // Global -> register loads use whole rows: instruction i of a tile covers
  // rows i*RPI + lane/CPR, 16-byte chunk lane%CPR (RPI rows of D bf16 = 1 KB).
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;       // rows per load instruction
  constexpr int NI = kTile / RPI;     // load instructions per tile (each for K and V)
  const int lrow = lane / CPR, lchunk = lane % CPR;

  // K/V of this (sequence, kv-head) for contiguous caches; the paged pool base
  // otherwise.  Per-lane element offsets from it fit in 32 bits (checked on
  // the host).
  const size_t bg_off = a.paged ? 0 : ((size_t)b * a.hkv + g) * a.max_ctx * D;
  const uint16_t* kbase = a.k + bg_off;
  const uint16_t* vbase = a.v + bg_off;

  // Issue the K/V loads of tile t0 (staging its positions first when sparse).
  // Stage (sparse) the positions of this wavefront's tile number `it`
  // (starting at t0) into sidx.
  auto stage = [&](int t0, int it) {
    if (SPARSE) {
      if (lane < kTile) {
        const int li = t0 + lane;
        const bool listed = li < nlist;
        int p = 0;
        if (listed) {
          if (it < kPreTiles) {
            p = it == 0 ? idx_pre[0] : it == 1 ? idx_pre[1] : it == 2 ? idx_pre[2] : idx_pre[3];
          } else if (B_id == 1) {
            p = a.idx[(size_t)b * a.idx_stride + li];
          } else {
            const int q_ = li / B_id;
            p = a.idx[(size_t)b * a.idx_stride + q_] * B_id + (li - q_ * B_id);
          }
        } else if (li < end) {
          p = L - tail + (li - nlist);  // a trailing position
        }
        p = min(max(p, 0), max(L - 1, 0));
        sidx[lane] = p;
        uint32_t off = (uint32_t)p * D;
        if (a.paged) {
          // entries past the list (p = 0) read row 0 of the sequence's own
          // first block: another block may hold anything, and P = 0 times a
          // non-finite V is NaN
          int blk = !listed ? btab[p >> 4] : it == 0 ? blk_pre[0] : it == 1 ? blk_pre[1]
                  : it == 2 ? blk_pre[2] : it == 3 ? blk_pre[3] : btab[p >> 4];
          blk = min(max(blk, 0), a.num_blocks - 1);
          off = (((uint32_t)blk * a.hkv + g) * 16u + (uint32_t)(p & 15)) * D;
        }
        srow[lane] = off;
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  };
  // Issue the loads of one tensor's rows for the tile starting at t0.
  auto issue = [&](int t0, const uint16_t* base, u32x4 (&dst)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = i * RPI + lrow;
      uint32_t off;
      if (SPARSE) {
        off = srow[r];
      } else {
        const int pos = min(t0 + r, end - 1);
        if (a.paged) {
          off = (((uint32_t)s_blk[(pos >> 4) - (start >> 4)] * a.hkv + g) * 16u +
                 (uint32_t)(pos & 15)) * D;
        } else {
          off = (uint32_t)pos * D;
        }
      }
      // byte offset in 32 bits from the uniform base: a scalar-base load
      const uint32_t boff = (off + (uint32_t)lchunk * 8u) * 2u;
      dst[i] = load16_stream(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(base) + boff));
    }
  };

  // Paged verify: the chunk's block ids (clamped) go to LDS once, so no load
  // address waits on a block-table read inside the loop.  Their loads go out
  // with the query fragments' below (one round trip for both).
  constexpr int kBlkPerThread = (kChunkMax / 16 + NT - 1) / NT;
  const int nblk = (!SPARSE && a.paged) ? (end - 1 - start) / 16 + 1 : 0;  // <= kChunkMax / 16
  int blk_v[kBlkPerThread];
#pragma unroll
  for (int j = 0; j < kBlkPerThread; ++j) {
    const int i = (int)threadIdx.x + j * NT;
    blk_v[j] = i < nblk ? btab[(start >> 4) + i] : 0;
  }

  u32x4 kraw[NI], vraw[NI];
  int ts = start + wave * kTile;
  int tile_no = 0;
  // Wide verify: after its first tile (wavefront w takes tile w) a wavefront
  // claims the next unclaimed tile of the chunk from an LDS counter, so the
  // wavefronts that run faster take more tiles and all finish within about
  // one tile of each other (two wavefronts share each SIMD, and the arbiter
  // favours the older one).  The chunk's logits fit the LDS buffer whole
  // (the plan's chunk is at most kMaxChunkWide), so no mid-chunk flush
  // assumes a fixed tile order.
  constexpr bool kClaim = kWide && !SPARSE;
  __shared__ int s_next_tile;
  if (kClaim && threadIdx.x == 0) s_next_tile = WAVES;

  // Stage the query fragments (B operand of S^T = K Q^T) before the first
  // tile's loads go out: a wavefront's loads complete in issue order, so
  // query loads issued after the first K/V tile would wait for it.
  // Fragment (qb, ks, lane) holds row m = qb*16 + lane%16,
  // d = ks*32 + (lane/16)*8 .. +8; a buffer load bounded by the group's rows
  // (rows past them read 0).
  {
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.q + row_base * D), 0, rows * D * 2, kRawBufferWord3);
    for (int f = threadIdx.x; f < QB * KS * 64; f += NT) {
      const int fl = f & 63, fks = (f >> 6) % KS, fqb = (f >> 6) / KS;
      const int m = fqb * 16 + (fl & 15);
      sq[f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            qr, (uint32_t)((m * D + fks * 32 + (fl >> 4) * 8) * 2), 0, 0));
    }
  }
  if (!SPARSE && a.paged) {
#pragma unroll
    for (int j = 0; j < kBlkPerThread; ++j) {
      const int i = (int)threadIdx.x + j * NT;
      if (i < nblk) s_blk[i] = min(max(blk_v[j], 0), a.num_blocks - 1);
    }
    __syncthreads();  // block ids staged (the first tile's addresses need them)
  }
  if (ts < end) {
    stage(ts, 0);
    issue(ts, kbase, kraw);
    issue(ts, vbase, vraw);
  }
  __syncthreads();  // query fragments staged
  if (kSumQuery) {
    // The summed query of the collected rows of the collected heads (heads
    // ascending, then rows ascending), formed from the staged fragments in
    // LDS (no more HBM round trips before the first tile): thread t < D sums
    // column d = t in fp32 and writes its bf16 rounding to column kSumCol
    // and the bf16 rounding of the remainder to kSumCol + 1 (about 16
    // significant bits together).  A fragment element (row m, column d) sits
    // in block m / 16, step d / 32, lane ((d % 32) / 8) * 16 + m % 16, slot d % 8.
    // Rows are taken in ascending order m = hh*T + t; every candidate row's
    // element is read at once (independent LDS reads) and the rows not
    // collected add exact zeros.
    if ((int)threadIdx.x < D) {
      const int dcol = threadIdx.x, ks = dcol / 32, lq = ((dcol % 32) / 8) * 16, j = dcol % 8;
      const uint16_t* sqh = reinterpret_cast<const uint16_t*>(sq);
      uint64_t take = 0ull;  // bit m: row m is a collected row of a collected head (m < rows <= 64)
      for (int hh = 0; hh < G; ++hh)
        if ((gmask >> hh) & 1ull) take |= (uint64_t)a.row_mask << (hh * T);
      float term[QB * 16];
#pragma unroll
      for (int m = 0; m < QB * 16; ++m)
        term[m] = __builtin_bit_cast(float, (uint32_t)sqh[(((m >> 4) * KS + ks) * 64 + lq + (m & 15)) * 8 + j] << 16);
      float qs = 0.f;
#pragma unroll
      for (int m = 0; m < QB * 16; ++m)
        if ((take >> m) & 1ull) qs += term[m];
      const __bf16 hi = (__bf16)qs, lo = (__bf16)(qs - (float)hi);
      uint16_t* sqw = reinterpret_cast<uint16_t*>(sq);
      sqw[(((QB - 1) * KS + ks) * 64 + lq + kSumCol) * 8 + j] = __builtin_bit_cast(uint16_t, hi);
      sqw[(((QB - 1) * KS + ks) * 64 + lq + kSumCol + 1) * 8 + j] = __builtin_bit_cast(uint16_t, lo);
    }
    __syncthreads();  // summed query staged
  }

  int lbase = start;  // first position held in slog
  // positions of logits slog holds (a multiple of step), and the tile count
  // at which it is full
  const int log_cap = a.paged ? kLogCapPaged : kLogCap;
  int flush_tile = log_cap / step;
  auto flush_logits = [&](int n) {  // slog[0, n) -> logits[lbase, lbase + n), nontemporal
    float* lp = a.logits + ((size_t)b * a.hkv + g) * a.max_ctx + lbase;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // recomputed here, not held across the loop
    if ((reinterpret_cast<uintptr_t>(lp) & 15) == 0) {
      for (int i = tid * 4; i + 4 <= n; i += NT * 4)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(slog + i),
                                    reinterpret_cast<f32x4*>(lp + i));
      for (int i = (n & ~3) + tid; i < n; i += NT) __builtin_nontemporal_store(slog[i], lp + i);
    } else {
      for (int i = tid; i < n; i += NT) __builtin_nontemporal_store(slog[i], lp + i);
    }
  };
  while (ts < end) {
    int claimed = 0;  // the wavefront's next tile (kClaim)
    if (kClaim) {
      if (lane == 0) claimed = atomicAdd(&s_next_tile, 1);
      claimed = __builtin_amdgcn_readfirstlane(claimed);
    }
    // Entry e of the tile (e = pb*16 + 4*kg + r for this lane's S^T values)
    // is visible to query row qb iff e < vis[qb]: positions ascend within a
    // tile, so each row sees a prefix.  `full`: every entry visible to all.
    const int n_in = min(kTile, end - ts);
    const bool full = n_in == kTile && (SPARSE ? sidx[kTile - 1] : ts + kTile - 1) <= lim_min;
    int vis[QB];
    if (!full) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (SPARSE) {
          int lo = 0, hi = n_in;  // count of entries with position <= lim[qb]
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (sidx[mid] <= lim[qb]) lo = mid + 1; else hi = mid;
          }
          vis[qb] = lo;
        } else {
          vis[qb] = max(0, min(lim[qb], ts + n_in - 1) - ts + 1);
        }
      }
    }

    // K tile -> LDS [position][d]; its registers are free at once, so the
    // next tile's K loads go out right away.  Per 16-row half: read the K
    // fragments (A of S^T = K Q^T: lane (c16, kg) of step ks holds row
    // pb*16 + c16, d = ks*32 + kg*8 ..), overwrite those rows with V (LDS
    // executes one wavefront's operations in order), multiply.  V's loads
    // for the next tile go out once V is in LDS.
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<u32x4*>(vt + (i * RPI + lrow) * VS + lchunk * 8) = kraw[i];
    const int tn = kClaim ? start + claimed * kTile : ts + step;
    if (tn < end) {
      stage(tn, tile_no + 1);
      issue(tn, kbase, kraw);
    }
    f32x4 sacc[2][QB];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      bf16x8 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                vt + (pb * 16 + c16) * VS + ks * 32 + kg * 8));
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = pb * (NI / 2); i < (pb + 1) * (NI / 2); ++i)
        *reinterpret_cast<u32x4*>(vt + (i * RPI + lrow) * VS + lchunk * 8) = vraw[i];
      if (pb == 1 && tn < end) issue(tn, vbase, vraw);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kf[ks], __builtin_bit_cast(bf16x8, sq[(qb * KS + ks) * 64 + lane]), acc, 0, 0, 0);
        sacc[pb][qb] = acc;
      }
    }

    // Collect-2-Query epilogue (any set of collected rows): pre-softmax logits.
    if (kHeadLogits) {
      float* hs = shl + wave * 16 * kHS;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (cmask[qb] == 0u) continue;
        // lane (c16, kg) holds row c16 at positions pb*16 + 4*kg .. +3
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
          f32x4 val;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = pb * 16 + 4 * kg + r;
            val[r] = (full || e < vis[qb]) ? sacc[pb][qb][r] * a.scale : kNegInf;
          }
          *reinterpret_cast<f32x4*>(hs + c16 * kHS + pb * 16 + 4 * kg) = val;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const int e = lane & 31;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (((cmask[qb] >> (2 * i)) & 3u) == 0u) continue;
          const int rr = 2 * i + (lane >> 5);
          const int64_t off = s_lrow[qb * 16 + rr];
          const float v = hs[rr * kHS + e];
          if (off >= 0 && e < n_in) __builtin_nontemporal_store(v, a.logits + off + ts + e);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    } else if (EMIT == VGSA_LOGITS_KVGROUP_SUM) {
      // v8[pb*4 + r]: this lane's collected rows summed, at position pb*16 +
      // 4*kg + r: a weight per row (the softmax scale when collected, else 0)
      // times its S^T value, so no branch or select per term.  The earliest
      // collected row sees a prefix of what the later ones see, so a
      // position is hidden from a collected row iff it is hidden from that
      // one: past its causal limit (one wave-uniform count per tile) the sum
      // is -inf, applied once to the reduced sum (the terms summed there are
      // finite products either way).  A kv-group with no collected head sums
      // to 0 at every position.
      const int row_first = __builtin_ctz(a.row_mask);
      const int vis0 = (full || gmask == 0ull)
                           ? kTile : max(0, min(L - T + row_first, ts + n_in - 1) - ts + 1);
      float v8[8];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float acc = 0.f;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc = __builtin_fmaf(rowc_w[qb], sacc[pb][qb][r], acc);
          v8[pb * 4 + r] = acc;
        }
      // Reduce-scatter over the 16 query-row lanes: after the four steps lane
      // c16 holds the full sum of position pb = bit 3, r = 2*bit 2 + bit 1.
      // Each step pairs a lane with one whose bit (8, 4, 2, then 1) differs
      // and whose higher bits agree: lane ^ 8, lane ^ 7 (the mirror within 8
      // lanes: bit 4 differs, bit 8 agrees), lane ^ 2, lane ^ 1; over the
      // steps every lane's partner sets join into all 16 lanes.
      const bool h8 = (c16 >> 3) & 1, h4 = (c16 >> 2) & 1, h2 = (c16 >> 1) & 1;
      float v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float keep = h8 ? v8[4 + i] : v8[i];
        const float give = h8 ? v8[i] : v8[4 + i];
        v4[i] = keep + dpp_move<kDppXor8>(give);
      }
      float v2[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float keep = h4 ? v4[2 + i] : v4[i];
        const float give = h4 ? v4[i] : v4[2 + i];
        v2[i] = keep + dpp_move<kDppHalfMirror>(give);
      }
      float v1 = (h2 ? v2[1] : v2[0]) + dpp_move<kDppXor2>(h2 ? v2[0] : v2[1]);
      v1 += dpp_move<kDppXor1>(v1);
      const int e = (h8 ? 16 : 0) + 4 * kg + 2 * h4 + h2;
      if ((c16 & 1) == 0) slog[ts - lbase + e] = e < vis0 ? v1 : kNegInf;
    }

    if (kSumQuery) {
      // Lanes c16 = 14 / 15 of the last block hold K . (high / low part);
      // after the exchange both hold the sum.  The earlier
      // collected row sees a prefix of what the later one sees, so past its
      // causal limit the sum is -inf.
      // (a kv-group with no collected head sums to 0 at every position)
      const int row_first = __builtin_ctz(a.row_mask);  // the earliest collected row
      const int vis0 = (full || gmask == 0ull)
                           ? kTile : max(0, min(L - T + row_first, ts + n_in - 1) - ts + 1);
      f32x4 lv[2];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = sacc[pb][QB - 1][r];
          x += swap_adjacent_lanes(x);
          lv[pb][r] = (pb * 16 + 4 * kg + r) < vis0 ? x * a.scale : kNegInf;
        }
      if (c16 == kSumCol) {
#pragma unroll
        for (int pb = 0; pb < 2; ++pb)
          *reinterpret_cast<f32x4*>(slog + (ts - lbase) + pb * 16 + 4 * kg) = lv[pb];
      }
    }

    // Online softmax (log2 units, lazily rescaled) and the P fragments
    // (B operand of O^T = V^T P^T).
    // x holds the unscaled S values (-inf where hidden); the scale is applied
    // to the row maximum (rounding is monotonic, so that is the maximum of the
    // scaled values) and inside the exponent's fused multiply-add.  Tiles that
    // every row sees in full skip the mask (one wave-uniform branch).
    bf16x8 pf[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float x[2][4];
      float mx = kNegInf;
      if (full) {
#pragma unroll
        for (int pb = 0; pb < 2; ++pb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[pb][r] = sacc[pb][qb][r];
            mx = fmaxf(mx, x[pb][r]);
          }
      } else {
#pragma unroll
        for (int pb = 0; pb < 2; ++pb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[pb][r] = (pb * 16 + 4 * kg + r) < vis[qb] ? sacc[pb][qb][r] : kNegInf;
            mx = fmaxf(mx, x[pb][r]);
          }
      }
      mx = column_max(mx) * a.scale_log2;
      const bool grow = mx > m_run[qb] + kRescaleLog2;
      if (__any(grow)) {
        const float m_new = grow ? mx : m_run[qb];
        if (__any(grow && m_run[qb] != kNegInf)) {  // a row still at -inf holds O = 0, l = 0
          const float alpha = grow ? fast_exp2(m_run[qb] - m_new) : 1.f;
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
        }
        m_run[qb] = m_new;
      }
      const float m_use = m_run[qb] == kNegInf ? 0.f : m_run[qb];
      float psum = 0.f;
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = fast_exp2(__builtin_fmaf(x[pb][r], a.scale_log2, -m_use));
          pf[qb][pb * 4 + r] = (__bf16)pv;
          psum += pv;
        }
      l_run[qb] += psum;
    }

    // O^T += V^T P^T.  A operand: row d = db*16 + c16, k slots 0..3 are
    // positions 4*kg + j, slots 4..7 are positions 16 + 4*kg + j -- the
    // positions the P fragment holds.  The LDS transpose read hands lane
    // (c16 = 4*j + q) the 4 values of d = db*16 + c16 from the 4 rows whose
    // 8-byte pieces (row 4*kg + j, d = db*16 + 4*q ..) the 16 lanes point at.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int trow = 4 * kg + (c16 >> 2), tcol = 4 * (c16 & 3);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS s16x4*)(vt + trow * VS + db * 16 + tcol));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS s16x4*)(vt + (16 + trow) * VS + db * 16 + tcol));
      const bf16x8 vf = __builtin_bit_cast(
          bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb], oacc[db][qb], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    ++tile_no;
    if (!kClaim && kGroupLogits && tile_no == flush_tile &&
        start + (tile_no - 1) * step + (WAVES - 1) * kTile < end) {
      // the last wavefront has a tile_no-th tile, so every wavefront reaches
      // this point (the condition is the same for all): the buffer is full
      __syncthreads();
      flush_logits(min(log_cap, end - lbase));
      __syncthreads();
      lbase += log_cap;
      flush_tile += log_cap / step;
    }
    ts = tn;
  }

  // Row sums: combine the four 16-lane groups.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l_run[qb] = column_sum(l_run[qb]);
  }
  __syncthreads();  // every wavefront's logits are in slog; no block id is read again
  if (kGroupLogits && end > lbase) {
    flush_logits(end - lbase);  // the rest (read once, later)
    __syncthreads();            // slog read out: its space takes the row statistics
  }
  if (kg == 0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      s_m[wave][qb * 16 + c16] = m_run[qb];
      s_l[wave][qb * 16 + c16] = l_run[qb];
    }
  }
  __syncthreads();

  // Merge the wavefronts, relative to each row's workgroup max M, in rounds
  // of D/kRounds head-dim columns (two when the parked blocks of half the
  // columns fit in the K/V tiles, which are free now, else four): every
  // wavefront parks its scaled accumulators for those columns of the real
  // rows in LDS, then all threads sum the wavefronts element by element and
  // write the result.
  constexpr int RP = QB * 16;      // rows held by the accumulators
  constexpr int kRounds = WAVES * RP * (D / 2 + 4) * 4 <= (int)sizeof(sbuf) ? 2 : 4;
  constexpr int DC = D / kRounds;  // columns per round
  constexpr int DBR = DB / kRounds;  // 16-wide column blocks per round
  constexpr int CS = DC + 4;       // row stride of a parked block (floats)
  static_assert(WAVES * RP * CS * 4 <= (int)sizeof(sbuf), "merge rounds must fit in the K/V tiles");
  float* obuf = reinterpret_cast<float*>(sbuf);  // [WAVES][RP][CS]
  float scl[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qb * 16 + c16;
    float M = s_m[0][row];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) M = fmaxf(M, s_m[w][row]);
    scl[qb] = m_run[qb] == kNegInf ? 0.f : fast_exp2(m_run[qb] - M);
  }
  float rowM = kNegInf, rowL = 0.f;  // threads < rows: their row's merged (M, l)
  if ((int)threadIdx.x < rows) {
    const int m = threadIdx.x;
    rowM = s_m[0][m];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) rowM = fmaxf(rowM, s_m[w][m]);
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
      if (s_m[w][m] != kNegInf) rowL += s_l[w][m] * fast_exp2(s_m[w][m] - rowM);
    s_inv[m] = rowL > 0.f ? 1.f / rowL : 0.f;
  }
  const int S = a.part_splits;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
#pragma unroll
    for (int j = 0; j < DBR; ++j)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        if (qb < QB - 1 || qb * 16 + c16 < rows)  // rows past the real ones are never read
          *reinterpret_cast<f32x4*>(obuf + (wave * RP + qb * 16 + c16) * CS + j * 16 + 4 * kg) =
              oacc[r * DBR + j][qb] * scl[qb];
    __syncthreads();
    // four consecutive columns per thread: 16-byte LDS reads, 16-byte partial
    // stores, 8-byte output stores
    constexpr int DQ = DC / 4;
    for (int e = threadIdx.x; e < rows * DQ; e += NT) {
      const int m = e / DQ, dq = e % DQ;
      f32x4 acc = *reinterpret_cast<const f32x4*>(obuf + m * CS + dq * 4);
#pragma unroll
      for (int w = 1; w < WAVES; ++w) acc += *reinterpret_cast<const f32x4*>(obuf + (w * RP + m) * CS + dq * 4);
      const int d = r * DC + dq * 4;
      const size_t po = ((row_base + m) * S + split) * D + d;  // partial element offset
      if (a.direct) {
        const float inv = s_inv[m];
        const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)(acc[0] * inv)) |
                            (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[1] * inv)) << 16;
        const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)(acc[2] * inv)) |
                            (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[3] * inv)) << 16;
        *reinterpret_cast<u32x2*>(a.out + (row_base + m) * D + d) = u32x2{lo, hi};
      } else if (SPARSE && a.fuse) {  // read back in this launch, maybe from another XCD
        store4_device(a.part_o, (uint32_t)(po * 4), make_float4(acc[0], acc[1], acc[2], acc[3]));
      } else {  // written once, read once (next launch)
        __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(a.part_o + po));
      }
    }
    __syncthreads();
  }
  if ((int)threadIdx.x < rows) {
    if (a.direct) {
      if (a.lse != nullptr)
        a.lse[row_base + threadIdx.x] = rowL > 0.f ? (rowM + __log2f(rowL)) * kLn2 : kNegInf;
    } else {
      const size_t prow = (row_base + threadIdx.x) * S + split;
      if (SPARSE && a.fuse) {
        store2_device(a.part_ml, (uint32_t)(prow * 8), make_float2(rowM, rowL));
      } else {
        a.part_ml[prow * 2 + 0] = rowM;
        a.part_ml[prow * 2 + 1] = rowL;
      }
    }
  }

  if (SPARSE && a.fuse) {
    // Fused merge: every non-empty split of this (sequence, kv-head) counts
    // itself in once its partials are out; the one that completes the count
    // merges them all (no workgroup waits on another).  The partials were
    // stored with device scope (write-through, no cache-wide flush needed);
    // every thread waits for its stores to complete before the count, and
    // the merging workgroup reads them with device-scope loads after it.
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const int nvalid = (count + chunk - 1) / chunk;
      int* ctr = a.sync + (size_t)b * a.hkv + g;
      const int done = atomicAdd(ctr, 1) + 1;
      s_last = done == nvalid;
      if (done == nvalid) atomicExch(ctr, 0);  // every split has counted: ready for the next call
    }
    __syncthreads();
    if (s_last) {
      CombineArgs c{};
      c.part_o = a.part_o;
      c.part_ml = a.part_ml;
      c.lengths = a.n_idx;
      c.tail = tail;
      c.rows_per_seq = a.hq * T;
      c.span = a.idx_stride;
      c.chunk = chunk;
      c.part_splits = S;
      c.out = a.out;
      c.lse = a.lse;
      constexpr int Q = D / 4;
      for (int e = threadIdx.x; e < rows * Q; e += NT)
        combine_quad<D, true>(c, (int)row_base + e / Q, e % Q, chunk, count);
    }
  }
}

// One block of D threads per (sequence, head, row): exact merge of the splits.
template <int D>
__global__ __launch_bounds__(kMergeBlock) void combine_kernel(CombineArgs a) {
  combine_block<D>(a, blockIdx.x);
}

template <int D, bool SPARSE, int EMIT, int WAVES>
hipError_t launch_d(const AttnArgs& a, dim3 grid, hipStream_t s) {
  // rows of one workgroup
  const int rows = (SPARSE && a.row_split > 1) ? (a.group * a.q_len + 1) / 2 : a.group * a.q_len;
  const dim3 block(WAVES * 64);
  if constexpr (WAVES == kWaves) {
    // narrow: only d = 128 with four row blocks (one wavefront per SIMD)
    if constexpr (D != 128) return hipErrorInvalidValue;
    else {
      if (rows <= 48) return hipErrorInvalidValue;
      hipLaunchKernelGGL((attn_partials_kernel<D, 4, SPARSE, EMIT, WAVES>), grid, block, 0, s, a);
    }
  } else {
    if (rows <= 16) {
      hipLaunchKernelGGL((attn_partials_kernel<D, 1, SPARSE, EMIT, WAVES>), grid, block, 0, s, a);
    } else if (rows <= 32) {
      hipLaunchKernelGGL((attn_partials_kernel<D, 2, SPARSE, EMIT, WAVES>), grid, block, 0, s, a);
    } else if (rows <= 48) {
      hipLaunchKernelGGL((attn_partials_kernel<D, 3, SPARSE, EMIT, WAVES>), grid, block, 0, s, a);
    } else {
      // four row blocks of d = 128 leave registers for one wavefront per
      // SIMD: the narrow layout (not instantiated wide)
      if constexpr (D == 128) return hipErrorInvalidValue;
      else hipLaunchKernelGGL((attn_partials_kernel<D, 4, SPARSE, EMIT, WAVES>), grid, block, 0, s, a);
    }
  }
  return hipGetLastError();
}

template <int D, int WAVES>
hipError_t launch_layout(const AttnArgs& a, bool sparse, dim3 grid, hipStream_t s) {
  if (sparse) return launch_d<D, true, VGSA_LOGITS_NONE, WAVES>(a, grid, s);
  switch (a.layout) {
    case VGSA_LOGITS_PER_HEAD: return launch_d<D, false, VGSA_LOGITS_PER_HEAD, WAVES>(a, grid, s);
    case VGSA_LOGITS_KVGROUP_SUM: {
      // the summed query fits in the last block's two spare columns;
      // otherwise a lane reduction sums the collected rows (an extra block
      // entering only S^T measured slower at d = 64 x 48 rows: +11.7 %
      // against +9.4 %, and +28 % with every row collected)
      const int rows = a.group * a.q_len;
      if (rows + 2 <= (rows + 15) / 16 * 16)
        return launch_d<D, false, kEmitSumColumn, WAVES>(a, grid, s);
      return launch_d<D, false, VGSA_LOGITS_KVGROUP_SUM, WAVES>(a, grid, s);
    }
    default: return launch_d<D, false, VGSA_LOGITS_NONE, WAVES>(a, grid, s);
  }
}

template <int D>
hipError_t launch_dim(const AttnArgs& a, bool sparse, dim3 grid, hipStream_t s) {
  return a.waves == kWavesWide ? launch_layout<D, kWavesWide>(a, sparse, grid, s)
                               : launch_layout<D, kWaves>(a, sparse, grid, s);
}

}  // namespace

hipError_t launch_attention_partials(const AttnArgs& a, bool sparse, hipStream_t s) {
  // the split plan never makes these: LDS logit buffer and mid-chunk flush
  const bool wide = a.waves == kWavesWide;
  if (!wide && a.waves != kWaves) return hipErrorInvalidValue;
  if (a.chunk > (wide ? kMaxChunkWide : kMaxChunk) || a.chunk % (wide ? kMinChunkWide : kMinChunk) != 0)
    return hipErrorInvalidValue;
  if (a.row_split > 1 && (!sparse || !wide || a.num_splits != 1 || !a.direct)) return hipErrorInvalidValue;
  // row split: two workgroups per (sequence, kv-head), in whole rounds of 16
  const int pairs = a.batch * a.hkv;
  const dim3 grid = a.row_split > 1 ? dim3((unsigned)((pairs + 7) / 8 * 16))
                                    : dim3(a.num_splits, a.hkv, a.batch);
  return a.head_dim == 64 ? launch_dim<64>(a, sparse, grid, s) : launch_dim<128>(a, sparse, grid, s);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.head_dim == 64) {
    hipLaunchKernelGGL(combine_kernel<64>, dim3(combine_blocks<64>(a.rows)), dim3(kMergeBlock), 0,
                       s, a);
  } else {
    hipLaunchKernelGGL(combine_kernel<128>, dim3(combine_blocks<128>(a.rows)), dim3(kMergeBlock),
                       0, s, a);
  }
  return hipGetLastError();
}

}  // namespace vgsa
