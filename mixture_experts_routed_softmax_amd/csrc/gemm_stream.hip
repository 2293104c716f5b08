// Weight-streaming expert GEMMs for decode-sized batches (T <= 64, so every
// expert owns at most 64 token rows), on tile-packed weights, bf16 or fp8.
//
// "Experts backends", section "Decode-stage switching": small token counts
// call for a different execution scheme than the grouped GEMM of large
// batches.  At T <= 64 the layer is bound by reading the touched experts'
// weights from HBM; this kernel reads every weight byte exactly once, spread
// over all compute units, and multiplies it against the (L2-resident) token
// rows of its expert:
//   gate/up : h[r, j] = act(x_r . w_gate[e, j]) * (x_r . w_up[e, j]),
//             act = silu, gelu or relu (GemmArgs.gate_act)
//   down    : y[r, o] = h_r . w_down[e, o]
//
// Work item = (touched expert, packed 256-row tile); 4 waves, each owning 64
// weight rows (gate/up: the gate and up rows of 32 channels) for all of the
// expert's tokens (one or two 32-token MFMA tiles).  Weights go from the
// contiguous packed chunks straight into registers in MFMA layout through a
// register ring of 4 (bf16) or 3 (fp8) K steps (no LDS, no barriers); token
// fragments are loaded from global memory (they stay in L2).  FP8: the
// partial sum of every 64-deep step is promoted with the s_w * s_x of its
// 128-deep scale block (both loaded with the step); the gate/up epilogue
// quantizes h per row over the block's 128 channels (s = amax / 448).
//
// Split K: when there are few work items (few touched experts) each item's K
// steps are split over S workgroups so that the stream occupies every CU;
// the S fp32 partial tiles are summed in split order by a second launch that
// also runs the epilogue.  S depends only on the item count, so results do
// not depend on timing.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kRowB = 64;       // packed bytes per row per K step
constexpr int kChunk = 256 * kRowB;
template <int kW>
constexpr int kRing = kW == 0 ? 4 : (kW == 1 ? 3 : 5);   // K steps in flight per wave (bf16, fp8, fp4)
// waves per SIMD: fp4 steps carry twice the token bytes, so its deeper ring
// takes the whole register file with one wave per SIMD
template <int kW>
constexpr int kWavesPerSimd = kW == 2 ? 1 : 2;
// batches of at most 32 tokens (one 32-token tile per item): without the
// second token tile a bf16 workgroup fits three to a CU (fp8 would spill)
template <int kW, bool kOneTile>
constexpr int kBlocksPerCu = kOneTile && kW == 0 ? 3 : kWavesPerSimd<kW>;   // 0: bf16
template <int kW, bool kOneTile>
constexpr int kSlots = 256 * kBlocksPerCu<kW, kOneTile>;   // resident workgroups

__device__ __forceinline__ int pswz(int row, int chunk) {
  return row * kRowB + ((chunk ^ ((row >> 2) & 3)) << 4);
}

__device__ __forceinline__ float wscale(const void* s, int ue8m0, int64_t idx) {
  return ue8m0 ? e8m0_to_f32(((const uint8_t*)s)[idx]) : ((const float*)s)[idx];
}

// weight formats of the streaming GEMM
constexpr int kWBf16 = 0, kWFp8 = 1, kWFp4 = 2;

// K steps of 64 packed weight bytes: 32 bf16, 64 fp8 or 128 fp4 values
template <int kW>
__host__ __device__ inline int stream_steps(int K) {
  return kW == kWBf16 ? K * 2 / kRowB : (kW == kWFp8 ? K / kRowB : K / (2 * kRowB));
}

template <int kW, int NT>
struct Step {
  i32x4 a[2][2];                       // [weight tile][16-byte piece]
  i32x4 b[NT][kW == kWFp4 ? 4 : 2];    // [token tile][16-byte piece]
  uint32_t s[kW == kWFp4 ? 2 : 1];     // fp4: the 4 UE8M0 block scales of each weight row's step
};

// Epilogue of one work item from its fp32 accumulators.  Lane holds token
// l32 of each token tile and channels (r/4)*8 + hl*4 + r%4 of each 32-row
// weight tile.
template <bool kFp8, int kMode, bool kOutF32, int NT>
__device__ __forceinline__ void stream_epilogue(const GemmArgs& a, const WorkItem& it, const f32x16 (&acc)[2][NT]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int N = a.N;
  if (kMode == 0) {
    const int ch0 = it.ntile * 128 + wave * 32;
    if constexpr (kFp8) {
      __shared__ float s_amax[4][64];
      float hv[NT][16];
      with_gate_act(a.gate_act, [&](auto k) {
#pragma unroll
        for (int j = 0; j < NT; ++j) gated16<decltype(k)::value>(acc[0][j], acc[1][j], hv[j]);
      });
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        float m = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(hv[j][r]));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (hl == 0) s_amax[wave][j * 32 + l32] = m;
      }
      __syncthreads();
      const int NG = N / 128;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int row = it.row_begin + j * 32 + l32;
        if (row >= it.row_end) continue;
        const int tk = j * 32 + l32;
        const float amax = fmaxf(fmaxf(s_amax[0][tk], s_amax[1][tk]), fmaxf(s_amax[2][tk], s_amax[3][tk]));
        const float s = amax > 0.f ? amax / 448.0f : 1.0f;
        uint8_t* h = (uint8_t*)a.out + (int64_t)row * N;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(uint32_t*)(h + ch0 + q * 8 + hl * 4) =
              pack_fp8x4(hv[j][q * 4 + 0] / s, hv[j][q * 4 + 1] / s, hv[j][q * 4 + 2] / s, hv[j][q * 4 + 3] / s);
        if (wave == 0 && hl == 0) a.out_scales[(int64_t)row * NG + it.ntile] = s;
      }
    } else {
      float hv[NT][16];
      with_gate_act(a.gate_act, [&](auto k) {
#pragma unroll
        for (int j = 0; j < NT; ++j) gated16<decltype(k)::value>(acc[0][j], acc[1][j], hv[j]);
      });
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int row = it.row_begin + j * 32 + l32;
        if (row >= it.row_end) continue;
        uint16_t* h = (uint16_t*)a.out + (int64_t)row * N;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = ch0 + q * 8 + hl * 4;
          if (ch >= N) continue;
          *(i32x2*)(h + ch) = i32x2{(int)pack_bf16x2(hv[j][q * 4 + 0], hv[j][q * 4 + 1]),
                                    (int)pack_bf16x2(hv[j][q * 4 + 2], hv[j][q * 4 + 3])};
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int row = it.row_begin + j * 32 + l32;
      if (row >= it.row_end) continue;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = it.ntile * 256 + wave * 64 + t * 32 + q * 8 + hl * 4;
          if (ch >= N) continue;
          const f32x16& y = acc[t][j];
          if (kOutF32) {
            *(f32x4*)((float*)a.out + (int64_t)row * N + ch) = f32x4{y[q * 4 + 0], y[q * 4 + 1], y[q * 4 + 2], y[q * 4 + 3]};
          } else {
            *(i32x2*)((uint16_t*)a.out + (int64_t)row * N + ch) =
                i32x2{(int)pack_bf16x2(y[q * 4 + 0], y[q * 4 + 1]), (int)pack_bf16x2(y[q * 4 + 2], y[q * 4 + 3])};
          }
        }
    }
  }
}

// K steps [kt_begin, kt_end) of one work item.  With `part` the fp32
// accumulators of the item's valid rows are stored there; otherwise the
// epilogue runs.
template <int kW, int kMode, bool kOutF32, int NT>
__device__ __forceinline__ void stream_tile(const GemmArgs& a, const WorkItem& it, int kt_begin, int kt_end,
                                            float* part) {
  constexpr bool kFp8 = kW != kWBf16;   // fp8 activations (fp8 and fp4 weights)
  constexpr bool kFp4 = kW == kWFp4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int e = it.expert;
  const int K = a.K, N = a.N;
  const int elt = kFp8 ? 1 : 2;         // bytes per activation element
  const int KT = stream_steps<kW>(K);
  const int kstep_b = kFp4 ? 2 * kRowB : kRowB;   // activation bytes per K step

  // weight rows (packed tile rows) of this lane
  int arow[2];
  if (kMode == 0) {
    arow[0] = wave * 32 + l32;
    arow[1] = 128 + wave * 32 + l32;
  } else {
    arow[0] = wave * 64 + l32;
    arow[1] = wave * 64 + 32 + l32;
  }
  const uint8_t* abase = (const uint8_t*)a.w0 + ((int64_t)e * a.wtiles + it.ntile) * KT * (int64_t)kChunk;
  // byte offsets of the two 16-byte pieces this lane needs per weight row:
  // bf16: logical chunks 2*kk + hl (kk = 0, 1); fp8: 2*hl and 2*hl + 1;
  // fp4: 2*m + hl for the step's two 64-deep MFMAs m (the fp4 A operand of a
  // lane half holds 32 consecutive K)
  int aoff[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int q = 0; q < 2; ++q) aoff[t][q] = pswz(arow[t], (kFp8 && !kFp4) ? hl * 2 + q : q * 2 + hl);
  // fp4: UE8M0 scales [rows, K/32] of this lane's two weight rows
  const uint8_t* srow[2] = {nullptr, nullptr};
  if constexpr (kFp4) {
    const int KS = K / 32;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      int ch;
      const uint8_t* sm;
      if (kMode == 0) {
        ch = it.ntile * 128 + (arow[t] & 127);
        sm = (const uint8_t*)(arow[t] < 128 ? a.s0 : a.s1);
      } else {
        ch = it.ntile * 256 + arow[t];
        sm = (const uint8_t*)a.s0;
      }
      ch = ch < N ? ch : N - 1;   // rows past N are zero in the packed tile
      srow[t] = sm + ((int64_t)e * N + ch) * KS;
    }
  }
  // token rows of this lane
  int64_t src_row[NT];
  const uint8_t* brow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int r = it.row_begin + j * 32 + l32;
    r = r < it.row_end ? r : it.row_end - 1;
    src_row[j] = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
    brow[j] = (const uint8_t*)a.act + src_row[j] * (int64_t)K * elt;
  }
  // byte offsets (within a K step) of the token pieces, same K mapping as A;
  // fp4 steps hold two 64-deep MFMAs, whose fp8 B operand of a lane half is
  // K hb*16 .. +16 and 32 + hb*16 .. +16 of the MFMA's 64
  constexpr int kBP = kFp4 ? 4 : 2;
  int boff[kBP];
#pragma unroll
  for (int q = 0; q < kBP; ++q)
    boff[q] = kFp4 ? q * 32 + hl * 16 : ((kFp8 ? hl * 2 + q : q * 2 + hl) * 16);

  const int KB = K / 128;

  typedef Step<kW, NT> S;
  auto load = [&](S& st, int kt) {
    const uint8_t* ck = abase + (int64_t)kt * kChunk;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q) st.a[t][q] = *(const i32x4*)(ck + aoff[t][q]);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < kBP; ++q) st.b[j][q] = *(const i32x4*)(brow[j] + (int64_t)kt * kstep_b + boff[q]);
    if constexpr (kFp4) {
#pragma unroll
      for (int t = 0; t < 2; ++t) st.s[t] = *(const uint32_t*)(srow[t] + kt * 4);
    }
  };

  f32x16 acc[2][NT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[t][j] = f32x16{};

  // fp8 scales of the whole K range, staged in LDS once: activation scales of
  // the item's rows (s_sx[row][kb]) and the block scales of the weight rows
  // (gate/up: s_sw[0] gate, s_sw[1] up; down: s_sw[h] for the tile's half h)
  __shared__ float s_sx[kFp8 ? kStreamMaxTokens * kStreamMaxScaleBlocks : 1];
  __shared__ float s_sw[2][kFp8 ? kStreamMaxScaleBlocks : 1];
  auto stage_scales = [&]() {
    if constexpr (kFp8) {
      const int NBr = (N + 127) / 128;
      for (int i = tid; i < kStreamMaxTokens * KB; i += 256) {
        const int row = i / KB, kb = i - row * KB;
        int r = it.row_begin + row;
        r = r < it.row_end ? r : it.row_end - 1;
        const int64_t src = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
        s_sx[i] = a.act_scales[src * KB + kb];
      }
      for (int i = tid; i < (kFp4 ? 0 : 2 * KB); i += 256) {
        const int h = i / KB, kb = i - h * KB;
        if (kMode == 0) {
          s_sw[h][kb] = wscale(h == 0 ? a.s0 : a.s1, a.scale_ue8m0, ((int64_t)e * NBr + it.ntile) * KB + kb);
        } else {
          int br = it.ntile * 2 + h;
          br = br < NBr ? br : NBr - 1;
          s_sw[h][kb] = wscale(a.s0, a.scale_ue8m0, ((int64_t)e * NBr + br) * KB + kb);
        }
      }
      __syncthreads();
    }
  };

  auto consume = [&](const S& st, int kt) {
    if constexpr (kFp4) {
      // two 64-deep MFMAs per step, the weights' block scales applied by the
      // MFMA (lane half hl: block 2*m + hl of the step), the activation scale
      // of the step's 128-deep block by promotion
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float sx = s_sx[(j * 32 + l32) * KB + kt];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x16 p = {};
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const i32x8 av = {st.a[t][m].x, st.a[t][m].y, st.a[t][m].z, st.a[t][m].w, 0, 0, 0, 0};
            const i32x8 bv = {st.b[j][2 * m].x, st.b[j][2 * m].y, st.b[j][2 * m].z, st.b[j][2 * m].w,
                              st.b[j][2 * m + 1].x, st.b[j][2 * m + 1].y, st.b[j][2 * m + 1].z,
                              st.b[j][2 * m + 1].w};
            const int sa = (int)((st.s[t] >> (8 * (2 * m + hl))) & 0xff);
            p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, p, 4, 0, 0, sa, 0, 127);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[t][j][r] = __builtin_fmaf(p[r], sx, acc[t][j][r]);
        }
      }
    } else if constexpr (kFp8) {
      // each step's partial sum is promoted on its own (both 64-deep halves
      // of a 128-deep scale block carry the same scales)
      const int kb = kt >> 1;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const i32x8 bv = {st.b[j][0].x, st.b[j][0].y, st.b[j][0].z, st.b[j][0].w,
                          st.b[j][1].x, st.b[j][1].y, st.b[j][1].z, st.b[j][1].w};
        const float sx = s_sx[(j * 32 + l32) * KB + kb];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const i32x8 av = {st.a[t][0].x, st.a[t][0].y, st.a[t][0].z, st.a[t][0].w,
                            st.a[t][1].x, st.a[t][1].y, st.a[t][1].z, st.a[t][1].w};
          const f32x16 p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, f32x16{}, 0, 0, 0, 127, 0, 127);
          const float m = s_sw[kMode == 0 ? t : (wave >> 1)][kb] * sx;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[t][j][r] = __builtin_fmaf(p[r], m, acc[t][j][r]);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[t][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((bf16x8)st.a[t][q], (bf16x8)st.b[j][q], acc[t][j],
                                                                0, 0, 0);
    }
  };

  // register ring: K steps kt .. kt+kRing-1 in flight
  constexpr int R = kRing<kW>;
  S ring[R];
  int kt0 = kt_begin;
  if (kt_end - kt_begin >= 2 * R) {
    // steady state: every slot is consumed and refilled with no conditions
    // (prologue included), so each wait knows exactly how many loads are
    // younger than the slot's own
#pragma unroll
    for (int d = 0; d < R; ++d) load(ring[d], kt_begin + d);
    stage_scales();
    for (; kt0 + 2 * R <= kt_end; kt0 += R) {
#pragma unroll
      for (int d = 0; d < R; ++d) {
        consume(ring[d], kt0 + d);
        load(ring[d], kt0 + d + R);
        __builtin_amdgcn_sched_barrier(0);   // keep the slots in ring order
      }
    }
  } else {
#pragma unroll
    for (int d = 0; d < R; ++d)
      if (kt_begin + d < kt_end) load(ring[d], kt_begin + d);
    stage_scales();
  }
  for (; kt0 < kt_end; kt0 += R) {
#pragma unroll
    for (int d = 0; d < R; ++d) {
      const int kt = kt0 + d;
      if (kt < kt_end) {
        consume(ring[d], kt);
        if (kt + R < kt_end) load(ring[d], kt + R);
      }
    }
  }

  if (part != nullptr) {
    // partial tile, token-row major: part[row * 256 + channel of the 256-row
    // weight tile]; only the item's valid rows are written
    const int rows = it.row_end - it.row_begin;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (j * 32 + l32 >= rows) continue;
      float* prow = part + (j * 32 + l32) * 256 + wave * 64 + hl * 4;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(f32x4*)(prow + t * 32 + q * 8) =
              f32x4{acc[t][j][q * 4 + 0], acc[t][j][q * 4 + 1], acc[t][j][q * 4 + 2], acc[t][j][q * 4 + 3]};
    }
    return;
  }
  stream_epilogue<kFp8, kMode, kOutF32, NT>(a, it, acc);
}

// Work item w: the schedule's entry, or with one entry per touched expert
// (its whole segment: every expert holds at most 64 rows here) entry
// w / wtiles with channel tile w % wtiles
__device__ __forceinline__ WorkItem stream_item(const GemmArgs& a, int w) {
  const WorkItem* items = (const WorkItem*)(a.sched + 1);
  if (!a.per_expert_items) return items[w];
  const int te = w / a.wtiles;
  WorkItem it = items[te];
  it.ntile = w - te * a.wtiles;
  return it;
}

template <int kW, int kMode, bool kOutF32, bool kOneTile>
__global__ __launch_bounds__(256, (kBlocksPerCu<kW, kOneTile>)) void gemm_stream_kernel(GemmArgs a) {
  const int items = a.sched->total;
  const int KT = stream_steps<kW>(a.K);
  const int S = stream_splits(items, KT, kSlots<kW, kOneTile>);
  const int u = xcd_work_index(items * S);
  if (u < 0) return;
  const int w = u / S, sp = u - w * S;
  const WorkItem it = stream_item(a, w);
  // down without its reduction launch: where each sorted row's partial rows
  // are (the items of an expert's channel tiles are consecutive)
  if (kMode == 1 && a.rowinfo != nullptr && sp == 0 && it.ntile == 0 &&
      (int)threadIdx.x < it.row_end - it.row_begin)
    a.rowinfo[it.row_begin + threadIdx.x] = w * 64 + threadIdx.x;
  const int kt0 = (int)((int64_t)KT * sp / S), kt1 = (int)((int64_t)KT * (sp + 1) / S);
  float* part = S > 1 ? a.partial + (int64_t)u * kStreamPartFloats : nullptr;
  if (!kOneTile && it.row_end - it.row_begin > 32)
    stream_tile<kW, kMode, kOutF32, 2>(a, it, kt0, kt1, part);
  else
    stream_tile<kW, kMode, kOutF32, 1>(a, it, kt0, kt1, part);
}

// Split-K reduction: one workgroup per work item sums its S partial tiles in
// split order and runs the epilogue, one thread per (row, output channel).
// Nothing to do when S == 1.  Partial tile layout: part[row * 256 + c] with,
// for gate/up, the gate value of channel ntile*128 + w*32 + x at c = w*64 + x
// and its up value at c = w*64 + 32 + x; for down, channel ntile*256 + c.
template <int kW, int kMode, bool kOutF32, bool kOneTile>
__global__ __launch_bounds__(256) void stream_reduce_kernel(GemmArgs a) {
  constexpr bool kFp8 = kW != kWBf16;   // fp8 activations and h (fp8 and fp4 weights)
  const int items = a.sched->total;
  const int KT = stream_steps<kW>(a.K);
  const int S = stream_splits(items, KT, kSlots<kW, kOneTile>);
  const int w = blockIdx.x;
  if (S == 1 || w >= items) return;
  const WorkItem it = stream_item(a, w);
  const int rows = it.row_end - it.row_begin;
  const float* part = a.partial + (int64_t)w * S * kStreamPartFloats;
  const int tid = threadIdx.x, N = a.N;
  // sums of the S (<= kStreamMaxSplit) partials at offsets o0 and o1, in
  // split order; all loads are issued before the first add
  auto total2 = [&](int o0, int o1, float& z0, float& z1) {
    float v0[kStreamMaxSplit], v1[kStreamMaxSplit];
#pragma unroll
    for (int u = 0; u < kStreamMaxSplit; ++u) {
      v0[u] = u < S ? part[(int64_t)u * kStreamPartFloats + o0] : 0.f;
      v1[u] = u < S ? part[(int64_t)u * kStreamPartFloats + o1] : 0.f;
    }
    z0 = 0.f;
    z1 = 0.f;
#pragma unroll
    for (int u = 0; u < kStreamMaxSplit; ++u) {
      z0 += v0[u];
      z1 += v1[u];
    }
  };
  if (kMode == 0) {
    // 128 channels per row: two waves per row, rows two at a time
    for (int base = 0; base < rows * 128; base += 256) {
      const int idx = base + tid;
      const int row = idx >> 7, c = idx & 127;
      const bool live = row < rows;
      float hv = 0.f;
      if (live) {
        const int o = row * 256 + (c >> 5) * 64 + (c & 31);
        float g, u;
        total2(o, o + 32, g, u);
        hv = gate_fn(g, a.gate_act) * u;
      }
      const int ch = it.ntile * 128 + c;
      if constexpr (kFp8) {
        // per-row quantization over the 128 channels (one activation group)
        __shared__ float s_m[4];
        float m = fabsf(hv);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if ((tid & 63) == 0) s_m[tid >> 6] = m;
        __syncthreads();
        const float amax = fmaxf(s_m[(tid >> 7) * 2], s_m[(tid >> 7) * 2 + 1]);
        __syncthreads();
        if (live) {
          const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
          const int64_t r = it.row_begin + row;
          ((uint8_t*)a.out)[r * N + ch] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(hv / sc, 0.f, 0, false) & 0xff);
          if (c == 0) a.out_scales[r * (N / 128) + it.ntile] = sc;
        }
      } else {
        if (live && ch < N) ((uint16_t*)a.out)[(int64_t)(it.row_begin + row) * N + ch] = f32_to_bf16_bits(hv);
      }
    }
  } else {
    // two rows per pass
    for (int idx = tid; idx < rows * 256; idx += 512) {
      const int row = idx >> 8, c = idx & 255;
      const bool second = row + 1 < rows;
      float y, y2;
      total2(row * 256 + c, (second ? row + 1 : row) * 256 + c, y, y2);
      const int ch = it.ntile * 256 + c;
      if (ch >= N) continue;
      if (second) {
        const int64_t o2 = (int64_t)(it.row_begin + row + 1) * N + ch;
        if (kOutF32) ((float*)a.out)[o2] = y2;
        else ((uint16_t*)a.out)[o2] = f32_to_bf16_bits(y2);
      }
      const int64_t o = (int64_t)(it.row_begin + row) * N + ch;
      if (kOutF32) ((float*)a.out)[o] = y;
      else ((uint16_t*)a.out)[o] = f32_to_bf16_bits(y);
    }
  }
}

}  // namespace

int stream_slots(int wfmt, int one_tile) {
  if (wfmt == kWFp4) return one_tile ? kSlots<kWFp4, true> : kSlots<kWFp4, false>;
  if (wfmt == kWFp8) return one_tile ? kSlots<kWFp8, true> : kSlots<kWFp8, false>;
  return one_tile ? kSlots<kWBf16, true> : kSlots<kWBf16, false>;
}

int stream_ksteps(int wfmt, int K) {
  return wfmt == kWFp4 ? stream_steps<kWFp4>(K) : (wfmt == kWFp8 ? stream_steps<kWFp8>(K) : stream_steps<kWBf16>(K));
}

hipError_t launch_gemm_stream(const GemmArgs& a, int wfmt, int mode, int grid, int reduce_grid, int one_tile,
                              hipStream_t stream, int with_reduce) {
  if (grid == 0) return hipSuccess;
  if (!with_reduce && (mode != 1 || a.rowinfo == nullptr)) return hipErrorInvalidValue;
  dim3 g(grid), rg(reduce_grid), b(256);
#define MOE_STREAM_LAUNCH_T(W, M, F32, ONE)                                              \
  do {                                                                                   \
    hipLaunchKernelGGL((gemm_stream_kernel<W, M, F32, ONE>), g, b, 0, stream, a);        \
    if (with_reduce)                                                                     \
      hipLaunchKernelGGL((stream_reduce_kernel<W, M, F32, ONE>), rg, b, 0, stream, a);   \
  } while (0)
#define MOE_STREAM_LAUNCH(W, M, F32)                      \
  do {                                                    \
    if (one_tile) MOE_STREAM_LAUNCH_T(W, M, F32, true);   \
    else MOE_STREAM_LAUNCH_T(W, M, F32, false);           \
  } while (0)
  if (wfmt == kWFp4) {
    if (mode == 0) MOE_STREAM_LAUNCH(kWFp4, 0, false);
    else if (a.out_f32) MOE_STREAM_LAUNCH(kWFp4, 1, true);
    else MOE_STREAM_LAUNCH(kWFp4, 1, false);
  } else if (wfmt == kWFp8) {
    if (mode == 0) MOE_STREAM_LAUNCH(kWFp8, 0, false);
    else if (a.out_f32) MOE_STREAM_LAUNCH(kWFp8, 1, true);
    else MOE_STREAM_LAUNCH(kWFp8, 1, false);
  } else {
    if (mode == 0) MOE_STREAM_LAUNCH(kWBf16, 0, false);
    else if (a.out_f32) MOE_STREAM_LAUNCH(kWBf16, 1, true);
    else MOE_STREAM_LAUNCH(kWBf16, 1, false);
  }
#undef MOE_STREAM_LAUNCH
#undef MOE_STREAM_LAUNCH_T
  return hipGetLastError();
}

}  // namespace moe
