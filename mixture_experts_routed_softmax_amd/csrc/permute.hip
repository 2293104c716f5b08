// Ordering (token, slot) pairs by selected expert, and the row gathers.
//
// "Experts backends", backend table, rows grouped_mm and deepgemm: tokens are
// ordered (sorted) by their selected expert so that all experts run as one
// grouped GEMM.  The order inside an expert is ascending (token, slot), i.e. a
// stable counting sort of the flattened top-k ids:
//   counts[e]  = #{p : ids[p] == e}
//   offsets[e] = sum_{e' < e} counts[e']            (E+1 entries)
//   row(p)     = offsets[ids[p]] + #{p' < p : ids[p'] == ids[p]}
//   perm[row(p)] = p,  inv[p] = row(p)
// Three launches, no atomics on global memory and no host synchronisation:
//   hist    : per-chunk expert histograms (chunks of 1024 pairs)
//   scan    : counts, offsets, per-chunk bases (offsets + earlier chunks), the
//             touched-expert list and the grouped-GEMM work schedules
//   scatter : stable in-chunk ranks (wave ballots per distinct id + per-wave counts)
// or, when all pairs fit one chunk, a single workgroup that does all three.
#include "common.h"
#include "kernels.h"
#include "topk_select.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                   int E, int32_t* __restrict__ block_counts) {
  __shared__ int s_hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) s_hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kPermChunk;
#pragma unroll
  for (int q = 0; q < kPermChunk / 256; ++q) {
    int64_t p = base + q * 256 + threadIdx.x;
    if (p < P) {
      const int e = ids[p];
      if ((unsigned)e < (unsigned)E) atomicAdd(&s_hist[e], 1);   // out-of-range ids are ignored
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    block_counts[(int64_t)blockIdx.x * E + e] = s_hist[e];
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves:
// shifts by 1, 2, 4 and 8 inside rows of 16 lanes, then the row broadcasts of
// lanes 15 and 31 carry the earlier rows' totals forward.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int scan_step(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xf, true);
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v = scan_step<0x111, 0xf>(v);   // row_shr:1
  v = scan_step<0x112, 0xf>(v);   // row_shr:2
  v = scan_step<0x114, 0xf>(v);   // row_shr:4
  v = scan_step<0x118, 0xf>(v);   // row_shr:8
  v = scan_step<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v = scan_step<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// In-place exclusive scans of N arrays v[j][0..n) (n <= 256) in LDS by the
// first wave of the block (lane l: entries 4l .. 4l+3), then a barrier of the
// whole block; total[j] gets each array's sum in every thread.  The arrays'
// entries must be written before (with a barrier); tmp: LDS scratch of N ints.
template <int N>
__device__ void block_exclusive_scan_n(int* const (&v)[N], int n, int* tmp, int (&total)[N]) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      int x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = 4 * lane + q < n ? v[j][4 * lane + q] : 0;
      const int t = x[0] + x[1] + x[2] + x[3];
      const int inc = wave_inclusive_scan(t);
      int run = inc - t;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (4 * lane + q < n) v[j][4 * lane + q] = run;
        run += x[q];
      }
      if (lane == 63) tmp[j] = inc;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < N; ++j) total[j] = tmp[j];
}

// Rank of this lane's id among the earlier lanes of its wave holding the same
// id, and (n_same) how many lanes of the wave hold it: one round per distinct
// id in the wave (a wave of decode-sized batches holds few).
__device__ __forceinline__ int wave_rank_same(int e, int lane, int& n_same) {
  int rank = 0;
  n_same = 0;
  uint64_t todo = ~0ull;
  while (todo != 0) {
    const int leader = __builtin_ctzll(todo);
    const int el = __builtin_amdgcn_readlane(e, leader);
    const uint64_t same = __ballot(e == el);
    if (e == el) {
      rank = __popcll(same & ((1ull << lane) - 1ull));
      n_same = __popcll(same);
    }
    todo &= ~same;
  }
  return rank;
}

// Item idx of one schedule: experts in ascending order; inside an expert (M
// row tiles x N output-channel tiles) blocks of up to block_m row tiles x
// block_n channel tiles, the blocks channel-major, inside a block the channel
// tile major and the row tile fastest.  Consecutive items then share a weight
// tile, and a run of block_m * block_n items (one XCD chunk of the grouped
// GEMMs) reads only block_n weight tiles and block_m token tiles.  With
// block_m = block_n = 1 this is channel tile major, row tile fastest.
// s_tiles[e]: row tiles of expert e; s_base[e]: its first item; rows_total:
// the row count (the end of the last expert's rows).
__device__ void write_schedule_item(const int* s_offsets, int E, int rows_total, SchedRequest rq,
                                    const int* s_tiles, const int* s_base, int idx) {
  // largest e with base[e] <= idx
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_base[mid] <= idx) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int M = s_tiles[e];
  const int bm = rq.block_m, bn = rq.block_n;
  int r = idx - s_base[e];
  int nt, mt;
  if (bm == 1 && bn == 1) {
    nt = r / M;
    mt = r - nt * M;
  } else {
    // channel block: bn columns (the last one possibly fewer) of M row tiles
    const int jb = r / (bn * M);
    const int cols = min(bn, rq.ntiles - jb * bn);
    r -= jb * bn * M;
    // row block inside it: bm rows (the last one possibly fewer)
    const int ib = r / (cols * bm);
    const int rows = min(bm, M - ib * bm);
    r -= ib * cols * bm;
    nt = jb * bn + r / rows;
    mt = ib * bm + r % rows;
  }
  const int BM = rq.rows_per_tile;
  const int rb = s_offsets[e] + mt * BM;
  const int re = min(rb + BM, e + 1 < E ? s_offsets[e + 1] : rows_total);
  ((WorkItem*)(rq.sched + 1))[idx] = WorkItem{rb, re, e, nt};
}

// LDS scratch of scan_counts_and_schedules, in ints
constexpr int kSchedWork = 6 * (kMaxExperts + 1);

// Sources of the expert counts for scan_counts_and_schedules
struct CountsInLds {      // s[e] (may be the offsets array itself)
  const int* s;
  __device__ int operator()(int e) const { return s[e]; }
};
struct CountsOfWaves {    // sum of the per-wave counts w[0..nw)[e]
  const int (*w)[kMaxExperts];
  int nw;
  __device__ int operator()(int e) const {
    int c = 0;
    for (int i = 0; i < nw; ++i) c += w[i][e];
    return c;
  }
};
struct CountsOfOffsets {  // differences of global offsets
  const int32_t* o;
  __device__ int operator()(int e) const { return o[e + 1] - o[e]; }
};

// Layout of the schedule tables one launch hands to another (ints): row
// offsets (E + 1), row tiles and first items of schedule 0, then of schedule
// 1 (E each, at strides of kMaxExperts + 1), then the two item counts and
// the row count.
constexpr int kTabOff = 0, kTabTiles0 = kMaxExperts + 1, kTabBase0 = 2 * (kMaxExperts + 1),
              kTabTiles1 = 3 * (kMaxExperts + 1), kTabBase1 = 4 * (kMaxExperts + 1),
              kTabTotals = 5 * (kMaxExperts + 1);
static_assert(kTabTotals + 3 == kSchedTablesInts, "schedule table layout");

// From the expert counts count_of(e), e < E (written, if in LDS, before a
// barrier): the counts in counts_out (if not null), the exclusive offsets in
// s_offsets[0..E) and their total (the row count, also stored at s_offsets[E]
// by thread 0: read it there only after a barrier), the touched-expert list
// (ascending, its length in touched[E]; touched may be null) and up to two
// grouped-GEMM schedules (a null sched skips one), with a single four-way scan.
// With `tables` the schedules' items are left to another launch: their item
// counts go to the headers and the tables they are computed from to `tables`.
template <class CountOf>
__device__ int scan_counts_and_schedules(CountOf count_of, int32_t* __restrict__ counts_out, int* s_offsets, int E,
                                         int32_t* __restrict__ touched, SchedRequest s0, SchedRequest s1,
                                         int* s_work, int* s_tmp, int32_t* __restrict__ tables = nullptr) {
  const int tid = threadIdx.x;
  int* s_tiles0 = s_work;
  int* s_tiles1 = s_work + (kMaxExperts + 1);
  int* s_base0 = s_work + 2 * (kMaxExperts + 1);
  int* s_base1 = s_work + 3 * (kMaxExperts + 1);
  int* s_tpos = s_work + 4 * (kMaxExperts + 1);
  int* s_c = s_work + 5 * (kMaxExperts + 1);
  for (int e = tid; e < E; e += 1024) {
    const int c = count_of(e);
    if (counts_out != nullptr) counts_out[e] = c;
    const int m0 = s0.sched != nullptr ? (c + s0.rows_per_tile - 1) / s0.rows_per_tile : 0;
    const int m1 = s1.sched != nullptr ? (c + s1.rows_per_tile - 1) / s1.rows_per_tile : 0;
    s_c[e] = c;
    s_offsets[e] = c;
    s_tiles0[e] = m0;
    s_base0[e] = m0 * s0.ntiles;
    s_tiles1[e] = m1;
    s_base1[e] = m1 * s1.ntiles;
    s_tpos[e] = c > 0 ? 1 : 0;
  }
  __syncthreads();
  int* const arrays[4] = {s_offsets, s_base0, s_base1, s_tpos};
  int total[4];
  block_exclusive_scan_n<4>(arrays, E, s_tmp, total);
  if (tid == 0) s_offsets[E] = total[0];
  if (touched != nullptr) {
    if (tid < E && s_c[tid] > 0) touched[s_tpos[tid]] = tid;
    if (tid == 0) touched[E] = total[3];
  }
  if (tid == 0) {
    if (s0.sched != nullptr) s0.sched->total = total[1];
    if (s1.sched != nullptr) s1.sched->total = total[2];
  }
  // a streaming schedule gets one entry per touched expert (at its place in
  // the touched list) and no per-item entries
  for (int e = tid; e < E; e += 1024)
    if (s_c[e] > 0) {
      const WorkItem ent{s_offsets[e], s_offsets[e] + s_c[e], e, 0};
      if (s0.implicit_items) ((WorkItem*)(s0.sched + 1))[s_tpos[e]] = ent;
      if (s1.implicit_items) ((WorkItem*)(s1.sched + 1))[s_tpos[e]] = ent;
    }
  const int w0 = s0.implicit_items ? 0 : total[1], w1 = s1.implicit_items ? 0 : total[2];
  if (tables != nullptr) {
    for (int e = tid; e < E; e += 1024) {
      tables[kTabOff + e] = s_offsets[e];
      tables[kTabTiles0 + e] = s_tiles0[e];
      tables[kTabBase0 + e] = s_base0[e];
      tables[kTabTiles1 + e] = s_tiles1[e];
      tables[kTabBase1 + e] = s_base1[e];
    }
    if (tid == 0) {
      tables[kTabOff + E] = total[0];
      tables[kTabTotals] = w0;
      tables[kTabTotals + 1] = w1;
      tables[kTabTotals + 2] = total[0];
    }
    return total[0];
  }
  // both schedules' items in one pass (totals of a null schedule are 0)
  for (int idx = tid; idx < w0 + w1; idx += 1024) {
    const bool first = idx < w0;
    write_schedule_item(s_offsets, E, total[0], first ? s0 : s1, first ? s_tiles0 : s_tiles1,
                        first ? s_base0 : s_base1, first ? idx : idx - w0);
  }
  return total[0];
}

// kFusedHist: the histogram of every chunk is taken here too, from the ids
// (at most kFusedHistBlocks chunks, chunk c by wave c % 16 with LDS atomics
// into its own row of counts), so that no histogram launch precedes the scan.
template <bool kFusedHist>
__global__ __launch_bounds__(1024) void scan_kernel(
    const int32_t* __restrict__ ids, int64_t P, const int32_t* __restrict__ block_counts, int64_t nblocks, int E,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ block_base,
    int32_t* __restrict__ touched, SchedRequest s0, SchedRequest s1, int32_t* __restrict__ tables) {
  __shared__ int s_part[4][kMaxExperts];
  __shared__ int s_offsets[kMaxExperts + 1];
  __shared__ int s_work[kSchedWork];
  __shared__ int s_tmp[4];   // the scans' totals
  __shared__ int s_cnt[kFusedHist ? kFusedHistBlocks * kMaxExperts : 1];
  const int tid = threadIdx.x;
  if constexpr (kFusedHist) {
    for (int x = tid; x < (int)nblocks * E; x += 1024) s_cnt[x] = 0;
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6;
    for (int c = wave; c < (int)nblocks; c += 16) {
      int v[kPermChunk / 64];
#pragma unroll
      for (int q = 0; q < kPermChunk / 64; ++q) {
        const int64_t p = (int64_t)c * kPermChunk + q * 64 + lane;
        v[q] = p < P ? ids[p] : -1;
      }
#pragma unroll
      for (int q = 0; q < kPermChunk / 64; ++q)
        if ((unsigned)v[q] < (unsigned)E) atomicAdd(&s_cnt[c * E + v[q]], 1);   // out-of-range ids are ignored
    }
    __syncthreads();
  }
  auto chunk_count = [&](int64_t b, int ex) {
    if constexpr (kFusedHist) return s_cnt[b * E + ex];
    else return block_counts[b * E + ex];
  };
  const int e = tid & 255;
  const int part = tid >> 8;
  const int64_t per = (nblocks + 3) / 4;
  const int64_t b0 = part * per;
  const int64_t b1 = min(nblocks, b0 + per);
  // the chunk counts are read 8 at a time so that their load latencies overlap
  int sum = 0;
  if (e < E)
    for (int64_t b = b0; b < b1; b += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = b + u < b1 ? chunk_count(b + u, e) : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += c[u];
    }
  s_part[part][e] = sum;
  __syncthreads();
  if (tid < E) {
    int c = s_part[0][tid] + s_part[1][tid] + s_part[2][tid] + s_part[3][tid];
    s_offsets[tid] = c;
    counts[tid] = c;
  }
  __syncthreads();
  const int total =
      scan_counts_and_schedules(CountsInLds{s_offsets}, nullptr, s_offsets, E, touched, s0, s1, s_work, s_tmp, tables);
  for (int i = tid; i <= E; i += 1024) offsets[i] = i < E ? s_offsets[i] : total;
  // per-chunk bases
  if (e < E) {
    int run = s_offsets[e];
    for (int p = 0; p < part; ++p) run += s_part[p][e];
    for (int64_t b = b0; b < b1; b += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = b + u < b1 ? chunk_count(b + u, e) : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b + u < b1) {
          block_base[(b + u) * E + e] = run;
          run += c[u];
        }
    }
  }
}

// All of the above in one workgroup when the pairs fit one chunk (P <= 1024,
// e.g. decode batches): histogram, counts and offsets, stable ranks, the
// touched-expert list and the schedules, with a single launch.
// Body of the one-workgroup permutation (1024 threads): thread p < P holds the
// expert e of pair p (-1 for none).
__device__ void permute_small_body(int e, int P, int E, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                   int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                   int32_t* __restrict__ touched, SchedRequest s0, SchedRequest s1) {
  __shared__ int s_wcount[16][kMaxExperts];
  __shared__ int s_offsets[kMaxExperts + 1];
  __shared__ int s_work[kSchedWork];
  __shared__ int s_tmp[4];   // the scans' totals
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // per-wave counts of the waves that hold pairs (the others are never read)
  const int nw = (P + 63) >> 6;
  for (int x = tid; x < nw * kMaxExperts; x += 1024) (&s_wcount[0][0])[x] = 0;
  __syncthreads();
  if ((unsigned)e >= (unsigned)E) e = -1;   // out-of-range ids get no row
  int n_same;
  const int rank = wave_rank_same(e, lane, n_same);
  if (e >= 0 && rank == n_same - 1) s_wcount[wave][e] = n_same;   // the wave's last lane with this id
  __syncthreads();
  const int total = scan_counts_and_schedules(CountsOfWaves{s_wcount, nw}, counts, s_offsets, E, touched, s0, s1,
                                              s_work, s_tmp);
  for (int x = tid; x <= E; x += 1024) offsets[x] = x < E ? s_offsets[x] : total;
  if (e >= 0) {
    int row = s_offsets[e] + rank;
    for (int w = 0; w < wave; ++w) row += s_wcount[w][e];
    perm[row] = tid;
    inv[tid] = row;
  } else if (tid < P) {
    inv[tid] = -1;   // a pair with an out-of-range id has no row
  }
}

__global__ __launch_bounds__(1024) void permute_small_kernel(
    const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ touched, SchedRequest s0,
    SchedRequest s1) {
  const int tid = threadIdx.x;
  permute_small_body(tid < P ? ids[tid] : -1, P, E, counts, offsets, perm, inv, touched, s0, s1);
}

// Small batches (T <= kSelectPermuteMaxT = 16, T * k <= 1024): the top-k selection
// of every token (wave w selects tokens w, w + 16, ..., exactly as the
// router's selection launch does) and the permutation of the selected pairs
// in one workgroup; the ids reach the permutation through LDS.
__global__ __launch_bounds__(1024) void select_permute_small_kernel(
    const float* __restrict__ part, int slices, int T, int E, const float* __restrict__ bias, int k, int score,
    int renorm, float routed_scale, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ touched, SchedRequest s0, SchedRequest s1) {
  __shared__ int s_ids[kPermChunk];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int tok = wave; tok < T; tok += 16) {
    float key[4];
    bool taken[4];
    token_keys(part, slices, T, tok, E, bias, lane, key, taken);
    select_topk(key, taken, lane, E, k, score, renorm, routed_scale, ids_out + (int64_t)tok * k,
                w_out + (int64_t)tok * k, s_ids + tok * k);
  }
  __syncthreads();
  const int P = T * k, tid = threadIdx.x;
  permute_small_body(tid < P ? s_ids[tid] : -1, P, E, counts, offsets, perm, inv, touched, s0, s1);
}

__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* __restrict__ offsets, int E,
                                                        SchedRequest rq) {
  // (offsets as moe_permute writes them: offsets[0] = 0)
  __shared__ int s_offsets[kMaxExperts + 1];
  __shared__ int s_work[kSchedWork];
  __shared__ int s_tmp[4];   // the scans' totals
  scan_counts_and_schedules(CountsOfOffsets{offsets}, nullptr, s_offsets, E, nullptr, rq, SchedRequest{}, s_work,
                            s_tmp);
}

// One workgroup of 1024 threads per chunk of 1024 pairs (one pair each): the
// rank among the wave's earlier lanes with the same id, the wave's count of
// each id (written by its last lane with that id), then the row: the
// chunk's base for the expert + the earlier waves' counts + the rank.  The
// workgroups also write the schedules' items from the tables scan_kernel
// left (item idx by thread idx of the grid): spread over the grid, the
// per-item arithmetic costs a fraction of what it costs one workgroup.
__global__ __launch_bounds__(1024) void scatter_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                       int E, const int32_t* __restrict__ block_base,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv, SchedRequest s0,
                                                       SchedRequest s1, const int32_t* __restrict__ tables) {
  static_assert(kPermChunk == 1024, "one pair per thread");
  __shared__ int s_cursor[kMaxExperts];
  __shared__ int s_wcount[16][kMaxExperts];
  __shared__ int s_tab[kSchedTablesInts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t p = (int64_t)blockIdx.x * kPermChunk + tid;
  int e = p < P ? ids[p] : -1;
  for (int x = tid; x < 16 * kMaxExperts; x += 1024) (&s_wcount[0][0])[x] = 0;
  for (int x = tid; x < E; x += 1024) s_cursor[x] = block_base[(int64_t)blockIdx.x * E + x];
  for (int x = tid; x < 5 * (E + 1); x += 1024) {
    const int t = x / (E + 1), i = x - t * (E + 1);   // table t, entry i <= E
    const int o = t * (kMaxExperts + 1) + i;
    if (t == 0 || i < E) s_tab[o] = tables[o];
  }
  if (tid < 3) s_tab[kTabTotals + tid] = tables[kTabTotals + tid];
  __syncthreads();
  if ((unsigned)e >= (unsigned)E) e = -1;   // out-of-range ids get no row
  int n_same;
  const int rank = wave_rank_same(e, lane, n_same);
  if (e >= 0 && rank == n_same - 1) s_wcount[wave][e] = n_same;   // the wave's last lane with this id
  __syncthreads();
  if (e >= 0) {
    int row = s_cursor[e] + rank;
    for (int w = 0; w < wave; ++w) row += s_wcount[w][e];
    perm[row] = (int32_t)p;
    inv[p] = row;
  } else if (p < P) {
    inv[p] = -1;   // a pair with an out-of-range id has no row
  }
  const int n0 = s_tab[kTabTotals], n1 = s_tab[kTabTotals + 1], rows_total = s_tab[kTabTotals + 2];
  for (int idx = blockIdx.x * 1024 + tid; idx < n0 + n1; idx += gridDim.x * 1024) {
    const bool first = idx < n0;
    write_schedule_item(s_tab + kTabOff, E, rows_total, first ? s0 : s1, s_tab + (first ? kTabTiles0 : kTabTiles1),
                        s_tab + (first ? kTabBase0 : kTabBase1), first ? idx : idx - n0);
  }
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ src,
                                                          const int32_t* __restrict__ perm, int k,
                                                          int64_t row_bytes, uint8_t* __restrict__ dst) {
  const int64_t r = blockIdx.x;
  const int64_t t = perm[r] / k;
  const i32x4* s = (const i32x4*)(src + t * row_bytes);
  i32x4* d = (i32x4*)(dst + r * row_bytes);
  for (int64_t c = threadIdx.x; c < row_bytes / 16; c += 256) d[c] = s[c];
}

__global__ __launch_bounds__(256) void gather_scales_kernel(const float* __restrict__ src,
                                                            const int32_t* __restrict__ perm, int k,
                                                            int64_t P, int n, float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= P * n) return;
  const int64_t r = i / n;
  const int c = (int)(i % n);
  dst[i] = src[(int64_t)(perm[r] / k) * n + c];
}

// Dynamic fp8 quantization of bf16 rows, per 128 channels: s = amax/448,
// code = RNE_e4m3(x/s); amax = 0 gives s = 1 and zero codes.  A thread takes
// 8 channels (one 16-byte load), 16 threads a group, a workgroup 16 groups
// (2048 channels) of one row.  (One 4-byte load per lane and a wave per group
// ran at 2.5 TB/s: 71 us for the DeepSeek-like 8192 x 7168 rows.)
__global__ __launch_bounds__(256) void quant_rows_fp8_kernel(const uint16_t* __restrict__ x,
                                                             int n, uint8_t* __restrict__ codes,
                                                             float* __restrict__ scales) {
  const int64_t row = blockIdx.x;
  const int groups = n / 128;
  const int c8 = blockIdx.y * 256 + threadIdx.x;   // 8-channel piece of the row
  const int g = c8 >> 4;                           // its 128-channel group
  const bool live = g < groups;                    // (uniform per 16 lanes)
  i32x4 v = {0, 0, 0, 0};
  if (live) v = *(const i32x4*)(x + row * n + c8 * 8);
  float f[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = bf16_bits_to_f32((uint16_t)((uint32_t)v[q] & 0xffff));
    f[2 * q + 1] = bf16_bits_to_f32((uint16_t)((uint32_t)v[q] >> 16));
  }
  float m = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(f[q]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float s = m > 0.f ? m / 448.0f : 1.0f;
  if (live) {
    *(i32x2*)(codes + row * n + c8 * 8) = i32x2{(int)pack_fp8x4(f[0] / s, f[1] / s, f[2] / s, f[3] / s),
                                                (int)pack_fp8x4(f[4] / s, f[5] / s, f[6] / s, f[7] / s)};
    if ((c8 & 15) == 0) scales[row * groups + g] = s;
  }
}

}  // namespace

hipError_t launch_hist(const int32_t* ids, int64_t P, int E, int32_t* block_counts,
                       hipStream_t stream) {
  int64_t nb = perm_blocks(P);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(hist_kernel, dim3((unsigned)nb), dim3(256), 0, stream, ids, P, E, block_counts);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* block_counts, int64_t nblocks, int E, int32_t* counts,
                       int32_t* offsets, int32_t* block_base, int32_t* touched, SchedRequest s0,
                       SchedRequest s1, int32_t* tables, hipStream_t stream) {
  if (tables == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL(scan_kernel<false>, dim3(1), dim3(1024), 0, stream, nullptr, (int64_t)0, block_counts, nblocks,
                     E, counts, offsets, block_base, touched, s0, s1, tables);
  return hipGetLastError();
}

hipError_t launch_hist_scan(const int32_t* ids, int64_t P, int E, int32_t* counts, int32_t* offsets,
                            int32_t* block_base, int32_t* touched, SchedRequest s0, SchedRequest s1,
                            int32_t* tables, hipStream_t stream) {
  const int64_t nb = perm_blocks(P);
  if (tables == nullptr || nb > kFusedHistBlocks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(scan_kernel<true>, dim3(1), dim3(1024), 0, stream, ids, P, nullptr, nb, E, counts, offsets,
                     block_base, touched, s0, s1, tables);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* ids, int64_t P, int E, const int32_t* block_base,
                          int32_t* perm, int32_t* inv, SchedRequest s0, SchedRequest s1,
                          const int32_t* tables, hipStream_t stream) {
  int64_t nb = perm_blocks(P);
  if (nb == 0) return hipSuccess;
  if (tables == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)nb), dim3(1024), 0, stream, ids, P, E,
                     block_base, perm, inv, s0, s1, tables);
  return hipGetLastError();
}

hipError_t launch_select_permute_small(const float* part, int slices, int64_t T, int E, const float* bias, int k,
                                       int score, int renorm, float routed_scale, int32_t* ids, float* w,
                                       int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                       int32_t* touched, SchedRequest s0, SchedRequest s1, hipStream_t stream) {
  if (T <= 0 || T > kSelectPermuteMaxT || T * k > kPermChunk || E > kMaxExperts || k > 64)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(select_permute_small_kernel, dim3(1), dim3(1024), 0, stream, part, slices, (int)T, E, bias, k,
                     score, renorm, routed_scale, ids, w, counts, offsets, perm, inv, touched, s0, s1);
  return hipGetLastError();
}

hipError_t launch_permute_small(const int32_t* ids, int64_t P, int E, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* inv, int32_t* touched, SchedRequest s0, SchedRequest s1,
                                hipStream_t stream) {
  if (P > kPermChunk) return hipErrorInvalidValue;
  hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), 0, stream, ids, (int)P, E, counts, offsets, perm,
                     inv, touched, s0, s1);
  return hipGetLastError();
}

hipError_t launch_schedule(const int32_t* offsets, int E, SchedRequest s, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, stream, offsets, E, s);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, const int32_t* perm, int k, int64_t P,
                              int64_t row_bytes, void* dst, hipStream_t stream) {
  if (P == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)P), dim3(256), 0, stream,
                     (const uint8_t*)src, perm, k, row_bytes, (uint8_t*)dst);
  return hipGetLastError();
}

hipError_t launch_gather_scales(const float* src, const int32_t* perm, int k, int64_t P, int n,
                                float* dst, hipStream_t stream) {
  if (P == 0) return hipSuccess;
  int64_t total = P * n;
  hipLaunchKernelGGL(gather_scales_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, src, perm, k, P, n, dst);
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp8(const uint16_t* x_bf16, int64_t rows, int n, uint8_t* codes,
                                 float* scales, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3((unsigned)rows, (unsigned)((n / 8 + 255) / 256)), dim3(256), 0,
                     stream, x_bf16, n, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
