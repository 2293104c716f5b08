// Grouped GEMMs of the expert MLPs on tile-packed weights (bf16 or OCP fp8).
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
// several K steps ahead; one barrier per step; the fragments of step s+1 are
// read from LDS while the MFMAs of step s run.  Token rows are read through the expert permutation when a gather
// index is given; token tiles past the expert's last row skip their MFMAs.
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

// token rows per tile: 256 for bf16 (each wave 64 weight rows x 128 tokens),
// 128 for fp8 (each wave 64 x 64; the per-block promotion needs a second set
// of accumulators)
template <bool kFp8>
struct Geo {
  static constexpr int kTok = kFp8 ? 128 : 256;
  static constexpr int kNTW = kTok / 64;            // token tiles per wave
  static constexpr int kB = kTok * kRowB;           // token bytes per stage
  static constexpr int kStage = kA + kB;
  static constexpr int kAmax = kFp8 ? 4 * kTok * 4 : 0;     // fp8 epilogue scratch
  static constexpr int kStages = (kLdsBudget - kAmax) / kStage;   // 6 (fp8) or 5 (bf16)
  static constexpr int kLoads = 2 + kTok / 128;     // DMA instructions per thread per stage
};

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
    default: wait_vmcnt<4 * kLoads>(); break;
  }
}

__device__ __forceinline__ float wscale(const void* s, int ue8m0, int64_t idx) {
  return ue8m0 ? e8m0_to_f32(((const uint8_t*)s)[idx]) : ((const float*)s)[idx];
}

// fragments of one K step: two weight tiles and the wave's token tiles
template <bool kFp8>
struct Frag {
  typedef typename std::conditional<kFp8, i32x8, bf16x8>::type T;
  static constexpr int kK = kFp8 ? 1 : 2;   // MFMAs along K per step
  T a[kK][2];
  T b[kK][Geo<kFp8>::kNTW];
};

template <bool kFp8, int kMode, bool kOutF32>
__global__ __launch_bounds__(kThreads, 1) void gemm_packed_kernel(GemmArgs a) {
  typedef Geo<kFp8> G;
  constexpr int kTok = G::kTok, kNTW = G::kNTW, kB = G::kB, kStage = G::kStage, kStages = G::kStages;
  constexpr int kLoads = G::kLoads;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage];
  const int w = xcd_work_index(a.sched->total);
  if (w < 0) return;
  const WorkItem it = ((const WorkItem*)(a.sched + 1))[w];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int rg = wave & 3, tg = wave >> 2;
  const int e = it.expert;
  const int K = a.K, N = a.N;
  const int elt = kFp8 ? 1 : 2;
  const int KT = K * elt / kRowB;          // K steps
  const int valid = it.row_end - it.row_begin;
  const int ntok = (valid + 31) >> 5;
  int my_nt = ntok - kNTW * tg;            // live token tiles of this wave (0..kNTW)
  my_nt = my_nt < 0 ? 0 : (my_nt > kNTW ? kNTW : my_nt);

  // ---- loaders
  const uint8_t* abase = (const uint8_t*)a.w0 + ((int64_t)e * a.wtiles + it.ntile) * KT * (int64_t)kA;
  // token rows: DMA instruction i of wave w fills LDS rows (i*8 + w)*16 .. +16
  constexpr int kBI = kTok / 128;
  const uint8_t* bsrc[kBI];
#pragma unroll
  for (int i = 0; i < kBI; ++i) {
    const int row = (i * 8 + wave) * 16 + (lane >> 2);
    int r = it.row_begin + row;
    r = r < it.row_end ? r : it.row_end - 1;
    const int64_t src_row = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    bsrc[i] = (const uint8_t*)a.act + src_row * (int64_t)K * elt + c * 16;
  }
  // wave-uniform parts of the DMA addresses (M0 takes the LDS address)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint8_t* asrc = abase + lane * 16 + wv * 1024;
  auto issue = [&](int stage, int kt) {
    uint8_t* sb = smem + stage * kStage + wv * 1024;
    const uint8_t* src = asrc + (int64_t)kt * kA;
    lds_load16(src, sb);
    lds_load16(src + 8192, sb + 8192);
#pragma unroll
    for (int i = 0; i < kBI; ++i) lds_load16(bsrc[i] + (int64_t)kt * kRowB, sb + kA + i * 8192);
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

  typedef Frag<kFp8> F;
  // The fragments of a K step are consumed in two halves (bf16: the two
  // 16-deep MFMA K slices; fp8: token tile 0, then the weight tiles with the
  // other token tiles).  A half is refilled from the next step's stage as
  // soon as its MFMAs are issued, so the LDS reads of step s+1 overlap the
  // MFMAs of step s without a second register set.
  auto read_half = [&](int stage, F& f, auto h_const, auto nt_const) {
    constexpr int NT = decltype(nt_const)::value, h = decltype(h_const)::value;
    const uint8_t* sa = smem + stage * kStage;
    const uint8_t* sb = sa + kA;
    if constexpr (kFp8) {
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
    if constexpr (kFp8) {
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
  // block's partial sums into the accumulators with s_w(block) * s_x(row, block)
  auto promote = [&](int kt, auto nt_const) {
    constexpr int NT = decltype(nt_const)::value;
    if constexpr (kFp8) {
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

  auto mainloop = [&](auto nt_const) {
    constexpr int NT = decltype(nt_const)::value;
    constexpr std::integral_constant<int, 0> h0{};
    constexpr std::integral_constant<int, 1> h1{};
    // prologue: K steps 0..kStages-2 in flight
#pragma unroll
    for (int p = 0; p < kStages - 1; ++p)
      if (p < KT) issue(p, p);
    wait_steps<kLoads>((KT < kStages - 1 ? KT : kStages - 1) - 1);
    __builtin_amdgcn_s_barrier();   // bare barrier: __syncthreads would wait for every step in flight
    F f;
    read_half(0, f, h0, nt_const);
    read_half(0, f, h1, nt_const);
    wait_lgkm<0>();
    // One K step: the MFMAs of step s, with the fragments of step s+1 read
    // from LDS stage `next` half by half as the MFMAs free their registers.
    auto body = [&](int s, int next) {
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkm<kFp8 ? 0 : 2 + NT>();   // this step's first half landed
      mfma_half(f, h0, nt_const);
      __builtin_amdgcn_sched_barrier(0);
      read_half(next, f, h0, nt_const);
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkm<kFp8 ? (NT >= 1 ? 2 : 0) : 2 + NT>();   // ... and its second half
      mfma_half(f, h1, nt_const);
      __builtin_amdgcn_sched_barrier(0);
      read_half(next, f, h1, nt_const);
      __builtin_amdgcn_sched_barrier(0);
      promote(s, nt_const);
    };
    int stage = 0;                  // LDS stage of step s
    int fill = kStages - 1;         // stage that receives step s + kStages - 1
    int s = 0;
    // steady state: every step refills the stage freed by step s-1, so the
    // number of steps still in flight behind step s+1 is constant
    for (; s < KT - (kStages - 1); ++s) {
      const int next = stage + 1 == kStages ? 0 : stage + 1;
      wait_vmcnt<(kStages - 3) * kLoads>();   // step s+1 landed for this thread
      __builtin_amdgcn_s_barrier();           // ... and for all; step s-1's stage is free
      issue(fill, s + kStages - 1);
      fill = fill + 1 == kStages ? 0 : fill + 1;
      body(s, next);
      stage = next;
    }
    // drain: nothing left to issue
    for (; s + 1 < KT; ++s) {
      const int next = stage + 1 == kStages ? 0 : stage + 1;
      wait_steps<kLoads>(KT - 2 - s);
      __builtin_amdgcn_s_barrier();
      body(s, next);
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
#pragma unroll
      for (int j = 0; j < kNTW; ++j) {
        float m = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          hv[j][r] = gate_fn(acc[0][j][r], a.gate_act) * acc[1][j][r];
          m = fmaxf(m, fabsf(hv[j][r]));
        }
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
#pragma unroll
      for (int j = 0; j < kNTW; ++j) {
        const int row = it.row_begin + brow + j * 32 + l32;
        if (j >= my_nt || row >= it.row_end) continue;
        uint16_t* h = (uint16_t*)a.out + (int64_t)row * N;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = ch0 + q * 8 + hl * 4;
          if (ch >= N) continue;
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = gate_fn(acc[0][j][q * 4 + c], a.gate_act) * acc[1][j][q * 4 + c];
          *(i32x2*)(h + ch) = i32x2{(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
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

hipError_t launch_gemm_packed(const GemmArgs& a, int fp8, int mode, int grid, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  dim3 g(grid), b(kThreads);
  if (fp8) {
    if (mode == 0) hipLaunchKernelGGL((gemm_packed_kernel<true, 0, false>), g, b, 0, stream, a);
    else if (a.out_f32) hipLaunchKernelGGL((gemm_packed_kernel<true, 1, true>), g, b, 0, stream, a);
    else hipLaunchKernelGGL((gemm_packed_kernel<true, 1, false>), g, b, 0, stream, a);
  } else {
    if (mode == 0) hipLaunchKernelGGL((gemm_packed_kernel<false, 0, false>), g, b, 0, stream, a);
    else if (a.out_f32) hipLaunchKernelGGL((gemm_packed_kernel<false, 1, true>), g, b, 0, stream, a);
    else hipLaunchKernelGGL((gemm_packed_kernel<false, 1, false>), g, b, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace moe
