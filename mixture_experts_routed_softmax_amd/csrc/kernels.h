// Host-side launchers of the libmoe kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct WorkItem;
struct Schedule;

// ---- router
// bf16: `part` is a workspace of route_workspace_bytes() for the partial logits
hipError_t launch_route_topk(const void* x, const void* w_router, const float* bias, int64_t T,
                             int H, int E, int k, int act_bf16, int score, int renorm,
                             float routed_scale, int32_t* ids, float* w, float* part, hipStream_t stream);
int route_slices(int64_t T, int H, int E);
bool route_big(int64_t T, int H);
// bf16 logits of a batch the small-batch router takes (!route_big): partial
// sums of route_slices() K slices, part[slice][T][E]
hipError_t launch_route_logits(const void* x, const void* w_router, int64_t T, int H, int E, float* part,
                               hipStream_t stream);
size_t route_workspace_bytes(int64_t T, int H, int E, int act_bf16);

// ---- permutation
constexpr int kPermChunk = 1024;   // (token, slot) pairs per histogram / scatter block

inline int64_t perm_blocks(int64_t P) { return (P + kPermChunk - 1) / kPermChunk; }

// One grouped-GEMM schedule to be built by the scan kernel.
struct SchedRequest {
  Schedule* sched;    // header + items, or nullptr
  int rows_per_tile;  // BM (token rows per tile)
  int ntiles;         // output-channel tiles per expert
  int capacity;       // items the buffer holds
  int block_m = 1;    // an expert's items run in blocks of block_m row tiles
  int block_n = 1;    //   x block_n channel tiles (see build_schedule)
  // weight streaming (every expert's rows form one row tile): one entry per
  // touched expert (its rows, channel tile 0) instead of one per item; item w
  // is entry w / ntiles with channel tile w % ntiles (GemmArgs::per_expert_items)
  bool implicit_items = false;
};

// work items per XCD chunk of the one-wave-per-SIMD grouped GEMMs
// (xcd_work_index<kGroupedXcdChunk>; their grid is a multiple of 8 times it)
constexpr int kGroupedXcdChunk = 16;

hipError_t launch_hist(const int32_t* ids, int64_t P, int E, int32_t* block_counts,
                       hipStream_t stream);
// counts, offsets, block bases, touched-expert list and the item counts of
// up to two schedules; the tables their items are computed from go to
// `tables` (kSchedTablesInts ints), and launch_scatter writes the items.
constexpr int kSchedTablesInts = 5 * (kMaxExperts + 1) + 3;
hipError_t launch_scan(const int32_t* block_counts, int64_t nblocks, int E, int32_t* counts,
                       int32_t* offsets, int32_t* block_base, int32_t* touched,
                       SchedRequest s0, SchedRequest s1, int32_t* tables, hipStream_t stream);
// launch_hist + launch_scan in one workgroup for at most kFusedHistBlocks
// chunks of pairs (the chunk histograms stay in LDS).  qwen_prefill, 16
// chunks: 15.8 -> 13.9 us; at 64 chunks (dsv3) the one workgroup reading
// every id took longer than the two launches (20.3 against 17 us)
constexpr int kFusedHistBlocks = 32;
hipError_t launch_hist_scan(const int32_t* ids, int64_t P, int E, int32_t* counts, int32_t* offsets,
                            int32_t* block_base, int32_t* touched, SchedRequest s0, SchedRequest s1,
                            int32_t* tables, hipStream_t stream);
hipError_t launch_scatter(const int32_t* ids, int64_t P, int E, const int32_t* block_base,
                          int32_t* perm, int32_t* inv, SchedRequest s0, SchedRequest s1,
                          const int32_t* tables, hipStream_t stream);
// top-k selection of every token from the partial logits of
// launch_route_logits, then hist + scan + scatter, in one workgroup, for
// T <= kSelectPermuteMaxT and T * k <= kPermChunk
constexpr int kSelectPermuteMaxT = 16;   // one token per wave: 32 tokens measured slower than two launches
hipError_t launch_select_permute_small(const float* part, int slices, int64_t T, int E, const float* bias, int k,
                                       int score, int renorm, float routed_scale, int32_t* ids, float* w,
                                       int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                       int32_t* touched, SchedRequest s0, SchedRequest s1, hipStream_t stream);
// hist + scan + scatter in one workgroup, for P <= kPermChunk
hipError_t launch_permute_small(const int32_t* ids, int64_t P, int E, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* inv, int32_t* touched, SchedRequest s0, SchedRequest s1,
                                hipStream_t stream);
// schedule from offsets alone (staged entry points)
hipError_t launch_schedule(const int32_t* offsets, int E, SchedRequest s, hipStream_t stream);

// gather rows: dst[r] = src[perm[r] / k]  (row_bytes multiple of 16)
hipError_t launch_gather_rows(const void* src, const int32_t* perm, int k, int64_t P,
                              int64_t row_bytes, void* dst, hipStream_t stream);
// gather fp32 scale rows: dst[r, :] = src[perm[r] / k, :]
hipError_t launch_gather_scales(const float* src, const int32_t* perm, int k, int64_t P, int n,
                                float* dst, hipStream_t stream);

// ---- fp8 activation quantization (per row, per 128 channels)
hipError_t launch_quant_rows_fp8(const uint16_t* x_bf16, int64_t rows, int n, uint8_t* codes,
                                 float* scales, hipStream_t stream);

// ---- grouped GEMMs
struct GemmArgs {
  const void* act;          // activation rows
  const float* act_scales;  // fp8: [rows_src, K/128]
  const int32_t* gather;    // nullptr, or sorted row -> perm entry (token = entry / gather_div)
  int gather_div;
  const void* w0;           // gate (or down) weights
  const void* w1;           // up weights (gate/up only)
  const void* s0;           // fp8 block scales of w0
  const void* s1;           // fp8 block scales of w1
  int scale_ue8m0;
  int K;                    // reduction length
  int N;                    // output channels (I for gate/up, H for down)
  void* out;                // [P, N]
  float* out_scales;        // fp8 h: [P, N/128]
  int out_f32;              // 1: fp32 output rows, 0: bf16
  const Schedule* sched;
  const int32_t* offsets;   // f32 path: expert of a row
  int E;
  int64_t P;
  int wtiles;               // packed weights: row tiles per expert
  float* partial;           // weight streaming: split-K partial tiles
  int gate_act;             // moe_gate_act of the gate/up epilogue
  int gu_out;               // row-major bf16 gate/up: store g and u (fp32 [P, 2N]) instead of h
  int64_t act_rows;         // rows of `act` (bounds of the activation buffer resource)
  int32_t* rowinfo;         // streaming down without its reduction launch: sorted row -> item * 64 + row in item
  int per_expert_items;     // streaming: the schedule holds one entry per touched expert (see SchedRequest)
};

// tile geometry of the grouped GEMMs
constexpr int kGemmRowsPerTile = 128;          // token rows per tile (all dtypes)
constexpr int kGemmGateUpChannelsBf16 = 256;   // h channels per bf16 gate/up tile (512 weight rows)
constexpr int kGemmDownChannelsBf16 = 512;     // output channels per bf16 down tile
constexpr int kGemmGateUpChannelsFp8 = 128;    // h channels per fp8 gate/up tile (256 weight rows)
constexpr int kGemmDownChannelsFp8 = 256;      // output channels per fp8 down tile

hipError_t launch_gate_up_bf16(const GemmArgs& a, int grid, hipStream_t stream);
hipError_t launch_down_bf16(const GemmArgs& a, int grid, hipStream_t stream);
hipError_t launch_gate_up_fp8(const GemmArgs& a, int grid, hipStream_t stream);
hipError_t launch_down_fp8(const GemmArgs& a, int grid, hipStream_t stream);
hipError_t launch_gate_up_f32(const GemmArgs& a, hipStream_t stream);
// grouped GEMM on tile-packed weights (bf16 or fp8), mode 0 gate/up, 1 down
// wfmt: weight format, 0 bf16, 1 fp8, 2 fp4 (e4m3 activations for 1 and 2)
hipError_t launch_gemm_packed(const GemmArgs& a, int wfmt, int mode, int grid, hipStream_t stream);
// bf16 grouped GEMM on packed weights with one wave per SIMD (weights loaded
// straight into registers, token rows through LDS); mode 0 gate/up, 1 down.
// Takes K a multiple of 64 and activations of act_rows rows spanning at most
// 4 GiB (32-bit row offsets); gemm_packed_kernel serves the rest.
bool gemm_grouped_bf16_fits(int64_t act_rows, int K);
hipError_t launch_gemm_grouped_bf16(const GemmArgs& a, int64_t act_rows, int mode, int grid, hipStream_t stream);
// fp8 (e4m3, 128 x 128 block scales) or, with fp4, e2m1 (UE8M0 scales per
// 32 K) grouped GEMM on packed weights and e4m3 activations with one wave per
// SIMD, 128 token rows per tile; takes K a multiple of 128 up to
// 128 * kStreamMaxScaleBlocks and activations spanning at most 4 GiB.
// Mode 0 gate/up (fp8 h and its scales), mode 1 down (bf16 y only).
bool gemm_grouped_fp8_fits(int64_t act_rows, int K);
hipError_t launch_gemm_grouped_fp8(const GemmArgs& a, int64_t act_rows, int mode, bool fp4, int grid,
                                   hipStream_t stream);
constexpr int kPackedGateUpChannels = 128;   // h channels per packed gate/up tile (256 weight rows)
constexpr int kPackedDownChannels = 256;     // output channels per packed down tile
// weight-streaming GEMM for T <= 64 on packed weights (one 64-row tile per
// touched expert), split over K when there are few items, plus its split-K
// reduction launch (reduce_grid >= min(item capacity, kStreamTarget): only
// fewer than kStreamTarget items are ever split)
// wfmt: weight format, 0 bf16, 1 fp8, 2 fp4 (fp8 activations for 1 and 2)
// one_tile: every expert holds at most 32 of the batch's rows (T <= 32)
// with_reduce = 0 (down only): no reduction launch; a split launch leaves
// y in the partial tiles (a.rowinfo says where) for launch_combine_stream
hipError_t launch_gemm_stream(const GemmArgs& a, int wfmt, int mode, int grid, int reduce_grid, int one_tile,
                              hipStream_t stream, int with_reduce = 1);
// workgroups resident at once and K steps of the streaming GEMM (they fix its splits)
int stream_slots(int wfmt, int one_tile);
int stream_ksteps(int wfmt, int K);
constexpr int kStreamMaxTokens = 64;
constexpr int kStreamMaxScaleBlocks = 64;   // fp8 streaming: K / 128 at most (K <= 8192)
constexpr int kStreamTarget = 1024;      // work units the split aims for (two rounds of 2 per CU)
constexpr int kStreamSlots = 512;        // workgroups resident at once (256 CUs x 2)
constexpr int kStreamMaxSplit = 16;
constexpr int kStreamMinSteps = 4;       // K steps per split at least
constexpr int kStreamPartFloats = 2 * 2 * 16 * 256;   // fp32 partial tile of one work unit
// K splits per work item for `items` items of KT steps (host and device agree):
// none when the items fill a whole round of kStreamSlots resident workgroups
// or at least 90% of their rounds (a split would only add the partial-tile
// traffic and the reduction launch: qwen_decode T=64 gate/up, 660 items on
// 512 slots, 134 us with 3 splits and their reduction, 131.5 us unsplit);
// else about kStreamTarget units, or one split more when that fills the last
// round clearly better.  Units stay below kStreamTarget + 2 * items.  Every
// workgroup evaluates this at its start, so it stays free of loops and
// variable divisions.
__host__ __device__ inline int stream_splits(int items, int KT, int slots = kStreamSlots) {
  if (items <= 0 || items >= kStreamTarget || items >= slots) return 1;
  const int r1 = (items + slots - 1) / slots;
  if (items * 10 >= r1 * slots * 9) return 1;
  int smax = KT / kStreamMinSteps;
  smax = smax < kStreamMaxSplit ? smax : kStreamMaxSplit;
  smax = smax < 1 ? 1 : smax;
  int s = (kStreamTarget + items - 1) / items;
  s = s < smax ? s : smax;
  if (s + 1 <= smax) {
    const int u0 = items * s, u1 = items * (s + 1);
    const int r0 = (u0 + slots - 1) / slots, r1b = (u1 + slots - 1) / slots;
    // fill(s) = u / (rounds * slots); take s + 1 if it fills at least 5 points better
    if ((int64_t)u1 * r0 * 100 >= (int64_t)u0 * r1b * 105) s = s + 1;
  }
  return s;
}
constexpr int kPackedTokBf16 = 256;          // token rows per packed bf16 tile
constexpr int kPackedTokFp8 = 128;           // token rows per packed fp8 tile

// ---- weight packing (one-time layout transform)
int64_t packed_tiles(int which_gate_up, int N);
hipError_t launch_pack(const void* w0, const void* w1, int gate_up, int E, int N, int64_t row_bytes,
                       void* dst, hipStream_t stream);
hipError_t launch_down_f32(const GemmArgs& a, hipStream_t stream);

// ---- backward (gemm_bwd.hip)
// C[n][m] = sum_k A[m][k] B[n][k], stored out[n][m].  A is MN-major (K index
// = memory row).  ragged N: B K-major token rows [row_begin, row_end) of a
// schedule item (or of 128-row tiles over n_total when sched is null), A rows
// k < a_split from a + e*a_gs, a_split <= k < a_krows from a2 + e*a_gs,
// zeros past a_krows; K = a.K.  ragged K: A and B MN-major, K rows
// [offsets[e], offsets[e+1]) (or [0, K) when offsets is null), zeros past
// the end; item = (e, m tile, n tile) from blockIdx; rows n >= n_split go to
// out2; rows n >= n_valid are not stored.  Tiles are kBwdTile x kBwdTile;
// columns past M (A) or n_total (B) read zeros and are not stored.
// Without offsets, k_chunk > 0 splits K: group e takes K rows
// [e k_chunk, (e+1) k_chunk) (partial sums, one output slice per group).
constexpr int kBwdTile = 256;
struct BwdGemmArgs {
  const uint16_t* a;
  const uint16_t* a2;
  int64_t lda;
  int64_t a_gs;
  int a_split;
  int a_krows;
  const uint16_t* b;
  int64_t ldb;
  const int32_t* b_gather;
  int b_div;
  const uint16_t* zeros;     // >= 8 zero bf16
  int M, K;
  int n_total, n_valid;
  const Schedule* sched;
  const int32_t* offsets;
  void* out;
  void* out2;
  int64_t ldo;
  int64_t o_gs;
  int n_split;
  int out_f32;
  int k_chunk;
};
// router: the router's two GEMMs (a separate instantiation, same code)
hipError_t launch_gemm_bwd(const BwdGemmArgs& a, int ragged_k, int router, int grid, hipStream_t stream);
hipError_t launch_swiglu_bwd(const float* ev, const float* gu, const int32_t* perm, const float* w, int64_t P,
                             int I, int act, float* dw, uint16_t* ap, uint16_t* dgu, hipStream_t stream);
hipError_t launch_router_bwd(const float* part, int slices, int64_t T, int E, int Epad, const float* bias,
                             const int32_t* ids, const float* dw, int k, int score, int renorm, float routed_scale,
                             float* dkey, uint16_t* dkey_b, hipStream_t stream);
hipError_t launch_bias_grad(const float* dkey, int64_t T, int E, float* dbias, hipStream_t stream);
hipError_t launch_dx_combine(const float* dxp, const float* dxr, const int32_t* inv, int64_t T, int k, int H,
                             uint16_t* dx, hipStream_t stream);
// bytes: multiple of 4
hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t stream);
// out[i] = bf16(sum over c < chunks of part[c * n + i]), n a multiple of 4
hipError_t launch_chunk_sum(const float* part, int chunks, int64_t n, uint16_t* out, hipStream_t stream);

// ---- combine
hipError_t launch_combine(const void* y, int y_f32, const int32_t* inv, const float* w, int64_t T,
                          int k, int H, void* out, int out_f32, hipStream_t stream);
// after a streaming down launch without its reduction: y rows from y when the
// launch was not split, else summed from its partial tiles (split order) and
// rounded to y's type first; then the combine above, same arithmetic
// Batches of at most kCombineFineMaxT tokens take one workgroup per (token, 32
// channels) when H is a multiple of 32, whose threads read the (slot, split)
// partial rows in parallel.
constexpr int kCombineFineMaxT = 16;
hipError_t launch_combine_stream(const void* y, int y_f32, const float* partial, const int32_t* rowinfo,
                                 const Schedule* sched, int ksteps, int slots, const int32_t* inv, const float* w,
                                 int64_t T, int k, int H, void* out, int out_f32, hipStream_t stream);

}  // namespace moe
