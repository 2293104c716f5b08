// Grouped GEMMs of the expert MLPs on tile-packed weights (bf16, OCP fp8 or
// fp4).  The one-wave-per-SIMD grouped kernels (gemm_grouped.hip,
// gemm_grouped_fp8.hip) take every shape they can address; this kernel runs
// the rest: activations past 4 GiB and down projections with an f32 y.
//
// "Experts backends": each expert is a gated MLP (backend table, row
// deepgemm_megamoe: up projection, SwiGLU, down projection) and all experts
// run as one grouped GEMM over the expert-sorted token rows (rows grouped_mm /
// deepgemm); FP8 experts carry 128 x 128 block scales (float32 or UE8M0) and
// dynamic per-row activation scales (section "FP8 and FP4 quantized experts").
//
//   gate/up : h[r, j] = act(x_r . w_gate[e, j]) * (x_r . w_up[e, j]),
//             act = silu, gelu or relu (GemmArgs.gate_act)
//   down    : y[r, o] = h_r . w_down[e, o]
//
// The weights are in the packed layout written by pack.hip: for every
// (expert, 256-row tile, 64-byte K step) one contiguous 16 KB chunk that is
// the LDS image of the step, so the weight operand streams from HBM in long
// contiguous runs.
//
// Tile = 256 weight rows x 256 token rows (bf16) or x 128 (fp8).  8 waves
// (two per SIMD) in a 4 (weight rows) x 2 (tokens) grid, each wave 64 weight
// rows x 128 (bf16) or 64 (fp8) tokens in 32 x 32 tiles
// (v_mfma_f32_32x32x16_bf16, or v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// scales for fp8).  For gate/up the
// two weight tiles of a wave are the gate and up rows of the same 32
// channels, so SwiGLU is applied in registers.
//
// Pipeline: an LDS ring of 32 KB (bf16: 16 KB weights + 16 KB tokens, 5
// stages) or 24 KB (fp8, 6 stages) stages filled with global_load_lds_dwordx4
// several K steps ahead (issued late in the step, see kDmaAt); one
// barrier per step; the fragments of step s+1 are read from LDS while the
// MFMAs of step s run.  Token rows are read through the expert permutation
// when a gather index is given; token tiles past the expert's last row skip
// their MFMAs.
//
// FP8: per 128-deep K block (two steps) the MFMA partial sums are promoted
// into the fp32 accumulators with s_w(block) * s_x(row, block); the gate/up
// epilogue quantizes h per row over the tile's 128 channels (one activation
// group) with s = amax / 448, codes = RNE_e4m3(h / s).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kThreads = 512;
constexpr int kRows = 256;               // weight rows per tile
constexpr int kRowB = 64;                // bytes per LDS row per K step
constexpr int kA = kRows * kRowB;        // 16 KB of weights per stage
constexpr int kLdsBudget = 160 * 1024;

// weight formats: bf16, fp8 (e4m3) and fp4 (e2m1, two per byte); fp8 and
// fp4 experts take e4m3 activations
constexpr int kWBf16 = 0, kWFp8 = 1, kWFp4 = 2;

// token rows per tile: 256 for bf16 (each wave 64 weight rows x 128 tokens),
// 128 for fp8 / fp4 (each wave 64 x 64; the per-block promotion needs a
// second set of accumulators).  A K step is 64 weight bytes per row: 32 bf16,
// 64 fp8 or 128 fp4 values, so an fp4 step carries 128 activation bytes per
// token row and the weight rows' 4 UE8M0 block scales (one dword per row).
template <int kW>
struct Geo {
  static constexpr int kTok = kW != kWBf16 ? 128 : 256;
  static constexpr int kNTW = kTok / 64;            // token tiles per wave
  static constexpr int kTokRowB = kW == kWFp4 ? 128 : kRowB;   // activation bytes per token row and step
  static constexpr int kB = kTok * kTokRowB;        // token bytes per stage
  static constexpr int kSc = kW == kWFp4 ? kRows * 4 : 0;      // fp4 weight scales per stage
  static constexpr int kStage = kA + kB + kSc;
  static constexpr int kAmax = kW != kWBf16 ? 4 * kTok * 4 : 0;     // fp8 epilogue scratch
  static constexpr int kStages = (kLdsBudget - kAmax) / kStage;   // 6 (fp8), 5 (bf16) or 4 (fp4)
  static constexpr int kLoads = 2 + kB / 8192 + (kW == kWFp4 ? 1 : 0);   // DMA instructions per thread per stage
};

// fp4 token rows: 128 bytes, 16-byte chunk c of row r at chunk c ^ (r & 7)
__device__ __forceinline__ int swz128(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowB + ((chunk ^ ((row >> 2) & 3)) << 4);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ void lds_load16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds_wave_base, 16, 0, 0);
}

template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(n): at most n LDS reads of this wave still in flight
template <int n>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(n >= 0 && n < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (n << 8));
}

template <int kLoads>
__device__ __forceinline__ void wait_steps(int ahead) {
  switch (ahead) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<kLoads>(); break;
    case 2: wait_vmcnt<2 * kLoads>(); break;
    case 3: wait_vmcnt<3 * kLoads>(); break;
    case 4: wait_vmcnt<4 * kLoads>(); break;
    default: wait_vmcnt<5 * kLoads>(); break;
  }
}

__device__ __forceinline__ float wscale(const void* s, int ue8m0, int64_t idx) {
  return ue8m0 ? e8m0_to_f32(((const uint8_t*)s)[idx]) : ((const float*)s)[idx];
}

// fragments of one K step: two weight tiles and the wave's token tiles
// (fp4: 16-byte e2m1 weight fragments and the rows' scale dwords)
template <int kW>
struct Frag {
  typedef typename std::conditional<kW != kWBf16, i32x8, bf16x8>::type T;
  typedef typename std::conditional<kW == kWFp4, i32x4, T>::type TA;
  static constexpr int kK = kW == kWFp8 ? 1 : 2;   // MFMAs along K per step
  TA a[kK][2];
  T b[kK][Geo<kW>::kNTW];
  uint32_t s[kW == kWFp4 ? 2 : 1];
};

template <int kW, int kMode, bool kOutF32>
__global__ __launch_bounds__(kThreads, 1) void gemm_packed_kernel(GemmArgs a) {
  constexpr bool kFp8 = kW != kWBf16;   // e4m3 activations (fp8 and fp4 weights)
  constexpr bool kFp4 = kW == kWFp4;
  typedef Geo<kW> G;
  constexpr int kTok = G::kTok, kNTW = G::kNTW, kB = G::kB, kStage = G::kStage, kStages = G::kStages;
  constexpr int kLoads = G::kLoads, kTokRowB = G::kTokRowB;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage];
  const int w = xcd_work_index(a.sched->total);
  if (w < 0) return;
  const WorkItem it = ((const WorkItem*)(a.sched + 1))[w];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int rg = wave & 3, tg = wave >> 2;
  const int e = it.expert;
  const int K = a.K, N = a.N;
  const int elt = kFp8 ? 1 : 2;            // bytes per activation element
  const int KT = kFp4 ? K / 128 : K * elt / kRowB;   // K steps
  const int valid = it.row_end - it.row_begin;
  const int ntok = (valid + 31) >> 5;
  int my_nt = ntok - kNTW * tg;            // live token tiles of this wave (0..kNTW)
  my_nt = my_nt < 0 ? 0 : (my_nt > kNTW ? kNTW : my_nt);

  // ---- loaders
  const uint8_t* abase = (const uint8_t*)a.w0 + ((int64_t)e * a.wtiles + it.ntile) * KT * (int64_t)kA;
  // token rows: DMA instruction i of wave w fills LDS rows (i*8 + w)*16 .. +16
  // (fp4: 128-byte rows, (i*8 + w)*8 .. +8)
  constexpr int kBI = kB / 8192;
  const uint8_t* bsrc[kBI];
#pragma unroll
  for (int i = 0; i < kBI; ++i) {
    const int row = kFp4 ? (i * 8 + wave) * 8 + (lane >> 3) : (i * 8 + wave) * 16 + (lane >> 2);
    int r = it.row_begin + row;
    r = r < it.row_end ? r : it.row_end - 1;
    const int64_t src_row = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
    const int c = kFp4 ? ((lane & 7) ^ (row & 7)) : ((lane & 3) ^ ((row >> 2) & 3));
    bsrc[i] = (const uint8_t*)a.act + src_row * (int64_t)K * elt + c * 16;
  }
  // fp4: UE8M0 scale dword (the step's 4 blocks) of tile row (wave & 3)*64 + lane;
  // waves 4-7 repeat waves 0-3 so that every wave issues the same loads
  const uint8_t* ssrc = nullptr;
  if constexpr (kFp4) {
    const int row = (wave & 3) * 64 + lane;
    int ch;
    const uint8_t* sm;
    if (kMode == 0) {
      ch = it.ntile * 128 + (row & 127);
      sm = (const uint8_t*)(row < 128 ? a.s0 : a.s1);
    } else {
      ch = it.ntile * 256 + row;
      sm = (const uint8_t*)a.s0;
    }
    ch = ch < N ? ch : N - 1;   // rows past N are zero in the packed tile
    ssrc = sm + ((int64_t)e * N + ch) * (K / 32);
  }
  // token DMA instructions that carry live rows: the second one (rows
  // kTok/2 .. kTok-1) is skipped when the tile holds no row there; its LDS
  // rows are then read by no wave (their waves have no live token tile)
  const int live_bi = __builtin_amdgcn_readfirstlane(kBI == 2 && valid <= kTok / 2 ? 1 : kBI);
  const bool full_loads = live_bi == kBI;
  // wave-uniform parts of the DMA addresses (M0 takes the LDS address)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint8_t* asrc = abase + lane * 16 + wv * 1024;
  auto issue = [&](int stage, int kt) {
    uint8_t* sb = smem + stage * kStage + wv * 1024;
    const uint8_t* src = asrc + (int64_t)kt * kA;
    lds_load16(src, sb);
    lds_load16(src + 8192, sb + 8192);
#pragma unroll
    for (int i = 0; i < kBI; ++i)
      if (i < live_bi) lds_load16(bsrc[i] + (int64_t)kt * kTokRowB, sb + kA + i * 8192);
    if constexpr (kFp4)
      __builtin_amdgcn_global_load_lds(ssrc + kt * 4, (lds_ptr)(smem + stage * kStage + kA + kB + (wv & 3) * 256), 4,
                                       0, 0);
  };

  // LDS rows of this wave's tiles
  int arow[2];
  if (kMode == 0) {
    arow[0] = rg * 32;          // gate rows of channels rg*32 .. +31
    arow[1] = 128 + rg * 32;    // up rows of the same channels
  } else {
    arow[0] = rg * 64;
    arow[1] = rg * 64 + 32;
  }
  const int brow = tg * kNTW * 32;

  typedef Frag<kW> F;
  // The fragments of a K step are consumed in two halves (bf16: the two
  // 16-deep MFMA K slices; fp4: the two 64-deep MFMA K slices; fp8: token
  // tile 0, then the weight tiles with the other token tiles).  A half is refilled from the next step's stage as
  // soon as its MFMAs are issued, so the LDS reads of step s+1 overlap the
  // MFMAs of step s without a second register set.
  auto read_half = [&](int stage, F& f, auto h_const, auto nt_const) {
    constexpr int NT = decltype(nt_const)::value, h = decltype(h_const)::value;
    const uint8_t* sa = smem + stage * kStage;
    const uint8_t* sb = sa + kA;
    if constexpr (kFp4) {
      // K slice h (64 deep): the e2m1 A operand of a lane half holds 32
      // consecutive K (weight chunk 2h + hl); the e4m3 B operand holds K
      // hl*16 .. +16 and 32 + hl*16 .. +16 of the slice (token chunks
      // 4h + hl and 4h + 2 + hl).  The scale dwords of the weight rows are
      // read first in the second slice's refill: the current step's second
      // slice has used them by then, and the next step's first slice waits
      // for them together with its own fragments
      if constexpr (h == 1) {
#pragma unroll
        for (int t = 0; t < 2; ++t) f.s[t] = *(const uint32_t*)(sb + kB + (arow[t] + l32) * 4);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) f.a[h][t] = *(const i32x4*)(sa + swz(arow[t] + l32, h * 2 + hl));
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int row = brow + j * 32 + l32;
        const i32x4 lo = *(const i32x4*)(sb + swz128(row, 4 * h + hl));
        const i32x4 hi = *(const i32x4*)(sb + swz128(row, 4 * h + 2 + hl));
        f.b[h][j] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
    } else if constexpr (kFp8) {
      auto ld8 = [&](const uint8_t* base, int row) {
        i32x4 lo = *(const i32x4*)(base + swz(row, hl * 2));
        i32x4 hi = *(const i32x4*)(base + swz(row, hl * 2 + 1));
        return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      };
      if constexpr (h == 0) {
        if constexpr (NT >= 1) f.b[0][0] = ld8(sb, brow + l32);
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) f.a[0][t] = ld8(sa, arow[t] + l32);
#pragma unroll
        for (int j = 1; j < NT; ++j) f.b[0][j] = ld8(sb, brow + j * 32 + l32);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) f.a[h][t] = *(const bf16x8*)(sa + swz(arow[t] + l32, h * 2 + hl));
#pragma unroll
      for (int j = 0; j < NT; ++j) f.b[h][j] = *(const bf16x8*)(sb + swz(brow + j * 32 + l32, h * 2 + hl));
    }
  };

  f32x16 acc[2][kNTW], part[2][kFp8 ? kNTW : 1];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int j = 0; j < kNTW; ++j) acc[t][j] = f32x16{};
    if constexpr (kFp8)
#pragma unroll
      for (int j = 0; j < kNTW; ++j) part[t][j] = f32x16{};
  }

  // fp8 scales
  const int KB = K / 128;
  int64_t sw_idx0 = 0, sw_idx1 = 0;
  const float* sa_row[kNTW] = {};
  if constexpr (kFp8) {
    const int NBr = (N + 127) / 128;
    if (kMode == 0) {
      sw_idx0 = ((int64_t)e * NBr + it.ntile) * KB;
      sw_idx1 = sw_idx0;
    } else {
      int br = it.ntile * 2 + (rg >> 1);
      br = br < NBr ? br : NBr - 1;
      sw_idx0 = ((int64_t)e * NBr + br) * KB;
      sw_idx1 = sw_idx0;
    }
#pragma unroll
    for (int j = 0; j < kNTW; ++j) {
      int r = it.row_begin + brow + j * 32 + l32;
      r = r < it.row_end ? r : it.row_end - 1;
      const int64_t src_row = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
      sa_row[j] = a.act_scales + src_row * KB;
    }
  }

  auto mfma_half = [&](const F& f, auto h_const, auto nt_const) {
    constexpr int NT = decltype(nt_const)::value, h = decltype(h_const)::value;
    if constexpr (kFp4) {
      // e2m1 x e4m3, the weight row's block scale (block 2h + hl of the step)
      // applied by the MFMA; the activation scale by the promotion
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int sc = (int)((f.s[t] >> (8 * (2 * h + hl))) & 0xff);
        const i32x8 av = {f.a[h][t].x, f.a[h][t].y, f.a[h][t].z, f.a[h][t].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < NT; ++j)
          part[t][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, f.b[h][j], part[t][j], 4, 0, 0, sc, 0, 127);
      }
    } else if constexpr (kFp8) {
      constexpr int j0 = h == 0 ? 0 : 1, j1 = h == 0 ? (NT < 1 ? NT : 1) : NT;
#pragma unroll
      for (int j = j0; j < j1; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          part[t][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[0][t], f.b[0][j], part[t][j], 0, 0,
                                                                        0, 127, 0, 127);
    } else {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[h][t], f.b[h][j], acc[t][j], 0, 0, 0);
    }
  };
  // fp8: at the end of a 128-deep scale block (every second step) fold the
  // block's partial sums into the accumulators with s_w(block) * s_x(row, block);
  // fp4: every step is one 128-deep activation block, weights already scaled
  auto promote = [&](int kt, auto nt_const) {
    constexpr int NT = decltype(nt_const)::value;
    if constexpr (kFp4) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float sx = sa_row[j][kt];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[t][j][r] = __builtin_fmaf(part[t][j][r], sx, acc[t][j][r]);
          part[t][j] = f32x16{};
        }
      }
    } else if constexpr (kFp8) {
      if (kt & 1) {
        const int kb = kt >> 1;
        const float s0 = wscale(a.s0, a.scale_ue8m0, sw_idx0 + kb);
        const float s1 = wscale(kMode == 0 ? a.s1 : a.s0, a.scale_ue8m0, sw_idx1 + kb);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const float sx = sa_row[j][kb];
          const float m0 = s0 * sx, m1 = s1 * sx;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[0][j][r] = __builtin_fmaf(part[0][j][r], m0, acc[0][j][r]);
            acc[1][j][r] = __builtin_fmaf(part[1][j][r], m1, acc[1][j][r]);
          }
          part[0][j] = part[1][j] = f32x16{};
        }
      }
    }
  };

  // s_waitcnt until at most `ahead` K steps of this thread's DMA are in flight
  auto wait_ahead = [&](int ahead) {
    if (full_loads) wait_steps<kLoads>(ahead);
    else wait_steps<kLoads - 1>(ahead);
  };
  // where a step's DMA is issued: 0 right after the barrier, 1 after the
  // first MFMA half, 2 after the second, 3 after the step's LDS reads, 4
  // after the fp8 block promotion (measured per format, dsv3 shapes: fp8
  // gate/up 4.20 ms at 4, 4.57 at 3, 4.85 at 0, 5.15 at 1; fp8 down 2.23 ms
  // at 4, 2.38 at 0; fp4 gate/up 3.73 ms at 2, 3.92 at 1, 4.08 at 3)
  constexpr int kDmaAt = kW == kWFp8 ? 4 : 2;
  constexpr bool kDmaLate = kDmaAt != 0;
  auto mainloop = [&](auto nt_const) {
    constexpr int NT = decltype(nt_const)::value;
    constexpr std::integral_constant<int, 0> h0{};
    constexpr std::integral_constant<int, 1> h1{};
    // prologue: K steps 0..kStages-2 in flight
#pragma unroll
    for (int p = 0; p < kStages - 1; ++p)
      if (p < KT) issue(p, p);
    wait_ahead((KT < kStages - 1 ? KT : kStages - 1) - 1);
    __builtin_amdgcn_s_barrier();   // bare barrier: __syncthreads would wait for every step in flight
    F f;
    read_half(0, f, h0, nt_const);
    read_half(0, f, h1, nt_const);
    wait_lgkm<0>();
    // One K step: the MFMAs of step s, with the fragments of step s+1 read
    // from LDS stage `next` half by half as the MFMAs free their registers.
    // The DMA of step fkt into stage fst (fkt < 0: none) is issued at
    // position kDmaAt of the step.  Right after the barrier it delays the
    // MFMAs: bf16 and fp4 issue it after the last MFMA (gate/up: dsv3_bf16
    // 4.85 -> 4.77 ms, expert-parallel shard 3.56 -> 3.43 ms, dsv3_fp4 3.98
    // -> 3.72 ms), fp8 after the block promotion that ends the step.
    auto body = [&](int s, int next, int fst, int fkt) {
      __builtin_amdgcn_sched_barrier(0);
      // this step's first half landed (fp4: and the scales, read before the
      // second half's fragments, which may still be in flight)
      wait_lgkm<kFp4 ? 2 + 2 * NT : (kFp8 ? 0 : 2 + NT)>();
      mfma_half(f, h0, nt_const);
      __builtin_amdgcn_sched_barrier(0);
      if (kDmaAt == 1 && fkt >= 0) issue(fst, fkt);
      __builtin_amdgcn_sched_barrier(0);
      read_half(next, f, h0, nt_const);
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkm<kFp4 ? 2 + 2 * NT : (kFp8 ? (NT >= 1 ? 2 : 0) : 2 + NT)>();   // ... and its second half
      mfma_half(f, h1, nt_const);
      __builtin_amdgcn_sched_barrier(0);
      if (kDmaAt == 2 && fkt >= 0) issue(fst, fkt);
      __builtin_amdgcn_sched_barrier(0);
      read_half(next, f, h1, nt_const);
      __builtin_amdgcn_sched_barrier(0);
      if (kDmaAt == 3 && fkt >= 0) issue(fst, fkt);
      __builtin_amdgcn_sched_barrier(0);
      promote(s, nt_const);
      __builtin_amdgcn_sched_barrier(0);
      if (kDmaAt == 4 && fkt >= 0) issue(fst, fkt);
    };
    int stage = 0;                  // LDS stage of step s
    int fill = kStages - 1;         // stage that receives step s + kStages - 1
    int s = 0;
    // steady state: every step refills the stage freed by step s-1, so the
    // number of steps still in flight behind step s+1 is constant
    for (; s < KT - (kStages - 1); ++s) {
      const int next = stage + 1 == kStages ? 0 : stage + 1;
      wait_ahead(kStages - 3);                // step s+1 landed for this thread
      __builtin_amdgcn_s_barrier();           // ... and for all; step s-1's stage is free (refilled in body)
      const int fst = fill;
      fill = fill + 1 == kStages ? 0 : fill + 1;
      if constexpr (kDmaLate) {
        body(s, next, fst, s + kStages - 1);
      } else {
        issue(fst, s + kStages - 1);
        body(s, next, 0, -1);
      }
      stage = next;
    }
    // drain: nothing left to issue
    for (; s + 1 < KT; ++s) {
      const int next = stage + 1 == kStages ? 0 : stage + 1;
      wait_ahead(KT - 2 - s);
      __builtin_amdgcn_s_barrier();
      body(s, next, 0, -1);
      stage = next;
    }
    mfma_half(f, h0, nt_const);
    mfma_half(f, h1, nt_const);
    promote(KT - 1, nt_const);
  };
  switch (my_nt) {
    case 0: mainloop(std::integral_constant<int, 0>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 3: mainloop(std::integral_constant<int, (kNTW > 2 ? 3 : 2)>{}); break;
    default: mainloop(std::integral_constant<int, kNTW>{}); break;
  }

  // ---- epilogue.  Lane holds token l32 of each token tile and channels
  // (r/4)*8 + hl*4 + r%4 of each 32-row weight tile.
  if (kMode == 0) {
    const int ch0 = it.ntile * 128 + rg * 32;
    if constexpr (kFp8) {
      __shared__ float s_amax[4][kTok];
      float hv[kNTW][16];
      with_gate_act(a.gate_act, [&](auto k) {
#pragma unroll
        for (int j = 0; j < kNTW; ++j) gated16<decltype(k)::value>(acc[0][j], acc[1][j], hv[j]);
      });
#pragma unroll
      for (int j = 0; j < kNTW; ++j) {
        float m = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(hv[j][r]));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (hl == 0) s_amax[rg][brow + j * 32 + l32] = m;
      }
      __syncthreads();
      const int NG = N / 128;
#pragma unroll
      for (int j = 0; j < kNTW; ++j) {
        const int row = it.row_begin + brow + j * 32 + l32;
        if (j >= my_nt || row >= it.row_end) continue;
        const int tk = brow + j * 32 + l32;
        const float amax = fmaxf(fmaxf(s_amax[0][tk], s_amax[1][tk]), fmaxf(s_amax[2][tk], s_amax[3][tk]));
        const float s = amax > 0.f ? amax / 448.0f : 1.0f;
        uint8_t* h = (uint8_t*)a.out + (int64_t)row * N;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = ch0 + q * 8 + hl * 4;
          *(uint32_t*)(h + ch) = pack_fp8x4(hv[j][q * 4 + 0] / s, hv[j][q * 4 + 1] / s, hv[j][q * 4 + 2] / s,
                                            hv[j][q * 4 + 3] / s);
        }
        if (rg == 0 && hl == 0) a.out_scales[(int64_t)row * NG + it.ntile] = s;
      }
    } else {
      // activations of every live token tile first (straight-line code),
      // then the stores of the lane's rows
      float hv[kNTW][16];
      with_gate_act(a.gate_act, [&](auto k) {
#pragma unroll
        for (int j = 0; j < kNTW; ++j) {
          if (j >= my_nt) break;
          gated16<decltype(k)::value>(acc[0][j], acc[1][j], hv[j]);
        }
      });
#pragma unroll
      for (int j = 0; j < kNTW; ++j) {
        const int row = it.row_begin + brow + j * 32 + l32;
        if (j >= my_nt || row >= it.row_end) continue;
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
    for (int j = 0; j < kNTW; ++j) {
      const int row = it.row_begin + brow + j * 32 + l32;
      if (j >= my_nt || row >= it.row_end) continue;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = it.ntile * 256 + rg * 64 + t * 32 + q * 8 + hl * 4;
          if (ch >= N) continue;
          if (kOutF32) {
            *(f32x4*)((float*)a.out + (int64_t)row * N + ch) =
                f32x4{acc[t][j][q * 4 + 0], acc[t][j][q * 4 + 1], acc[t][j][q * 4 + 2], acc[t][j][q * 4 + 3]};
          } else {
            const f32x16& y = acc[t][j];
            *(i32x2*)((uint16_t*)a.out + (int64_t)row * N + ch) =
                i32x2{(int)pack_bf16x2(y[q * 4 + 0], y[q * 4 + 1]), (int)pack_bf16x2(y[q * 4 + 2], y[q * 4 + 3])};
          }
        }
    }
  }
}

}  // namespace

hipError_t launch_gemm_packed(const GemmArgs& a, int wfmt, int mode, int grid, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  dim3 g(grid), b(kThreads);
#define MOE_PACKED_LAUNCH(W)                                                                   \
  do {                                                                                         \
    if (mode == 0) hipLaunchKernelGGL((gemm_packed_kernel<W, 0, false>), g, b, 0, stream, a);  \
    else if (a.out_f32) hipLaunchKernelGGL((gemm_packed_kernel<W, 1, true>), g, b, 0, stream, a); \
    else hipLaunchKernelGGL((gemm_packed_kernel<W, 1, false>), g, b, 0, stream, a);            \
  } while (0)
  if (wfmt == kWFp4) MOE_PACKED_LAUNCH(kWFp4);
  else if (wfmt == kWFp8) MOE_PACKED_LAUNCH(kWFp8);
  else MOE_PACKED_LAUNCH(kWBf16);
#undef MOE_PACKED_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
