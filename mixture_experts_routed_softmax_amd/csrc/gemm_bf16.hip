// bf16 grouped GEMMs of the expert MLPs, one launch for all experts.
//
// "Experts backends": the selected tokens of every expert are projected
// through that expert's gated MLP (backend table, row deepgemm_megamoe:
// up projection, SwiGLU, down projection) as one grouped GEMM over the
// expert-sorted rows (rows grouped_mm / deepgemm).
//
//   gate/up : h[r, j] = act(x_r . w_gate[e, j]) * (x_r . w_up[e, j]),
//             act = silu, gelu or relu (GemmArgs.gate_act)
//   down    : y[r, o] = h_r . w_down[e, o]
//
// Tile = 512 weight rows x 128 token rows, K step 32, 4 waves stacked along
// the weight rows: wave w owns 128 weight rows (four 32-row MFMA tiles) and
// all 128 tokens (four 32-token tiles): 16 accumulators of
// v_mfma_f32_32x32x16_bf16 held in AGPRs, one wave per SIMD.
//
// * Both operands travel global -> LDS with global_load_lds_dwordx4 (no
//   staging registers): each wave instruction fills 1 KB of LDS = 16 rows of
//   64 B, every row read as one contiguous 64-byte segment.  Four LDS stages
//   (40 KB each) keep three K steps in flight; one barrier per step.
// * LDS rows are 64 B; the four 16-byte chunks of row r are stored at
//   chunk ^ ((r >> 2) & 3), which makes the 16-lane groups of every MFMA
//   fragment read hit 16 distinct 16-byte bank groups (64 banks).
// * Token rows are read through the expert permutation when a gather index
//   is given (the fused forward never materialises a sorted copy of x).
// * Token tiles past the last row of the expert are skipped (wave-uniform),
//   so a ragged tail costs at most 31 padded rows of MFMA work.
// * For gate/up the four weight tiles of a wave are gate and up rows of the
//   same 64 channels, so SwiGLU is applied in registers.  Every lane ends with
//   16 channels of one token: 4 runs of 4 consecutive channels, stored as 8-
//   (bf16) or 16-byte (fp32) writes.
// * Work items (expert, token tile, channel tile) come from the device
//   schedule built from the scanned expert offsets; consecutive items share an
//   expert's weight tile and land on the same XCD (and L2).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kTok = 128;                 // token rows per tile
constexpr int kWRows = 512;               // weight rows per tile
constexpr int kRowB = 64;                 // bytes per LDS row = 32 bf16 of K
constexpr int kABytes = kWRows * kRowB;   // 32 KB
constexpr int kBBytes = kTok * kRowB;     // 8 KB
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kStages = 4;
constexpr int kThreads = 512;             // 8 waves, two per SIMD
constexpr int kLoadsPerStage = 5;         // per thread: 4 weight + 1 token instructions

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowB + ((chunk ^ ((row >> 2) & 3)) << 4);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ void lds_load16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds_wave_base, 16, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int kMode, bool kOutF32>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];
  const int w = xcd_work_index(a.sched->total);
  if (w < 0) return;
  const WorkItem it = ((const WorkItem*)(a.sched + 1))[w];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int K = a.K, N = a.N;
  const int e = it.expert;
  const int valid = it.row_end - it.row_begin;
  const int ntok = (valid + 31) >> 5;   // live 32-token tiles, wave-uniform

  // ---- loader geometry: lane L of a wave instruction fills LDS row L/4 (of
  // 16) at physical chunk L%4, i.e. logical chunk (L%4) ^ swizzle(row).
  const int lrow = lane >> 2;
  const int lchunk = lane & 3;
  // weight rows: wave w instruction i covers rows (w*4 + i)*16 .. +16
  const uint16_t* ag[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wave * 4 + i) * 16 + lrow;
    int ch;
    const uint16_t* src;
    if (kMode == 0) {
      ch = it.ntile * kGemmGateUpChannelsBf16 + (row & 255);
      src = (const uint16_t*)(row < 256 ? a.w0 : a.w1);
    } else {
      ch = it.ntile * kGemmDownChannelsBf16 + row;
      src = (const uint16_t*)a.w0;
    }
    ch = ch < N ? ch : N - 1;   // rows past N are computed but never stored
    const int c = lchunk ^ ((row >> 2) & 3);
    ag[i] = src + ((int64_t)e * N + ch) * K + c * 8;
  }
  // token rows: wave w covers rows w*16 .. +16
  const uint16_t* bg[1];
#pragma unroll
  for (int i = 0; i < 1; ++i) {
    const int row = (wave + i) * 16 + lrow;
    int r = it.row_begin + row;
    r = r < it.row_end ? r : it.row_end - 1;
    const int64_t src_row = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
    const int c = lchunk ^ ((row >> 2) & 3);
    bg[i] = (const uint16_t*)a.act + src_row * K + c * 8;
  }

  auto issue_stage = [&](int stage, int k0) {
    uint8_t* sb = smem + stage * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_load16(ag[i] + k0, sb + (wave * 4 + i) * 1024);
    lds_load16(bg[0] + k0, sb + kABytes + wave * 1024);
  };

  // LDS rows of this wave's two weight tiles: gate and up rows of channels
  // 32w .. 32w+31 (gate/up), or output channels 64w .. 64w+63 (down)
  int arow[2];
  if (kMode == 0) {
    arow[0] = wave * 32;
    arow[1] = 256 + wave * 32;
  } else {
    arow[0] = wave * 64;
    arow[1] = wave * 64 + 32;
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = f32x16{};

  // main loop, specialised on the number of live token tiles so that the
  // MFMA block is straight-line code.  Fragment reads are software-pipelined:
  // the second half-step's fragments (kk = 1) are read while the first
  // half's MFMAs run, and the barrier for the next stage sits between the two
  // halves so that the next step's first fragments are in flight during the
  // second half's MFMAs.
  auto mainloop = [&](auto nt_const) {
    constexpr int NT = decltype(nt_const)::value;
    const int KS = K / 32;
    auto read_frags = [&](int stage, int kk, bf16x8 (&af)[2], bf16x8 (&bf)[NT]) {
      const uint8_t* sa = smem + stage * kStageBytes;
      const uint8_t* sb = sa + kABytes;
      const int chunk = kk * 2 + hl;
#pragma unroll
      for (int t = 0; t < 2; ++t) af[t] = *(const bf16x8*)(sa + swz(arow[t] + l32, chunk));
#pragma unroll
      for (int j = 0; j < NT; ++j) bf[j] = *(const bf16x8*)(sb + swz(j * 32 + l32, chunk));
    };
    auto mfmas = [&](const bf16x8 (&af)[2], const bf16x8 (&bf)[NT]) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t], bf[j], acc[t][j], 0, 0, 0);
    };
    // wait until this thread's loads of step `s` landed; `ahead` = steps issued after it
    auto wait_step = [&](int ahead) {
      if (ahead >= 2) wait_vmcnt<2 * kLoadsPerStage>();
      else if (ahead == 1) wait_vmcnt<kLoadsPerStage>();
      else wait_vmcnt<0>();
    };
    // prologue: K steps 0 .. kStages-2 in flight, then step 0's first fragments
#pragma unroll
    for (int p = 0; p < kStages - 1; ++p)
      if (p < KS) issue_stage(p, p * 32);
    int issued = KS < kStages - 1 ? KS : kStages - 1;   // steps issued so far
    wait_step(issued - 1);
    __builtin_amdgcn_s_barrier();   // bare barrier: __syncthreads would wait for every step in flight
    bf16x8 a0[2], b0[NT], a1[2], b1[NT];
    read_frags(0, 0, a0, b0);
    int stage = 0;
    for (int s = 0; s + 1 < KS; ++s) {
      read_frags(stage, 1, a1, b1);
      mfmas(a0, b0);
      const int next = stage + 1 == kStages ? 0 : stage + 1;
      wait_step(issued - 1 - (s + 1));   // step s+1 landed for this thread
      __builtin_amdgcn_s_barrier();      // ... and for every thread; step s-1's buffer is free
      // the DMA of step `issued` into the stage of step s-1 goes out after
      // the step's last MFMAs (right after the barrier it delayed them:
      // qwen_prefill row-major gate/up 345 -> 335 us)
      const bool do_issue = issued < KS;
      int stn = stage + kStages - 1;
      stn = stn >= kStages ? stn - kStages : stn;
      const int k_issue = issued * 32;
      issued += do_issue ? 1 : 0;
      read_frags(next, 0, a0, b0);
      mfmas(a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      if (do_issue) issue_stage(stn, k_issue);
      __builtin_amdgcn_sched_barrier(0);
      stage = next;
    }
    read_frags(stage, 1, a1, b1);   // last step
    mfmas(a0, b0);
    mfmas(a1, b1);
  };
  switch (ntok) {
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 3: mainloop(std::integral_constant<int, 3>{}); break;
    default: mainloop(std::integral_constant<int, 4>{}); break;
  }

  // ---- epilogue.  Lane holds token l32 of each token tile and channels
  // (r/4)*8 + hl*4 + r%4 of each 32-row weight tile.  The gated activations
  // of every live token tile come first, as straight-line code.
  float hv[4][16];
  if (kMode == 0 && !a.gu_out)
    with_gate_act(a.gate_act, [&](auto k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j >= ntok) break;
        gated16<decltype(k)::value>(acc[0][j], acc[1][j], hv[j]);
      }
    });
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = it.row_begin + j * 32 + l32;
    if (j >= ntok || row >= it.row_end) continue;
    if (kMode == 0 && a.gu_out) {
      // g and u themselves in fp32 (the backward recomputes them): [P, 2N], g first
      float* h = (float*)a.out + (int64_t)row * 2 * N;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = it.ntile * kGemmGateUpChannelsBf16 + wave * 32 + q * 8 + hl * 4;
        if (ch >= N) continue;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f32x16& c = acc[t][j];
          *(f32x4*)(h + t * N + ch) = f32x4{c[q * 4 + 0], c[q * 4 + 1], c[q * 4 + 2], c[q * 4 + 3]};
        }
      }
    } else if (kMode == 0) {
      uint16_t* h = (uint16_t*)a.out + (int64_t)row * N;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
          const int ch = it.ntile * kGemmGateUpChannelsBf16 + wave * 32 + q * 8 + hl * 4;
          if (ch >= N) continue;
          uint16_t v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = f32_to_bf16_bits(hv[j][q * 4 + c]);
          i32x2 pk = {(int)(v[0] | ((uint32_t)v[1] << 16)), (int)(v[2] | ((uint32_t)v[3] << 16))};
          *(i32x2*)(h + ch) = pk;
        }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = it.ntile * kGemmDownChannelsBf16 + wave * 64 + t * 32 + q * 8 + hl * 4;
          if (ch >= N) continue;
          if (kOutF32) {
            f32x4 v = {acc[t][j][q * 4 + 0], acc[t][j][q * 4 + 1], acc[t][j][q * 4 + 2],
                       acc[t][j][q * 4 + 3]};
            *(f32x4*)((float*)a.out + (int64_t)row * N + ch) = v;
          } else {
            uint16_t v[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = f32_to_bf16_bits(acc[t][j][q * 4 + c]);
            i32x2 pk = {(int)(v[0] | ((uint32_t)v[1] << 16)), (int)(v[2] | ((uint32_t)v[3] << 16))};
            *(i32x2*)((uint16_t*)a.out + (int64_t)row * N + ch) = pk;
          }
        }
    }
  }
}

}  // namespace

hipError_t launch_gate_up_bf16(const GemmArgs& a, int grid, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<0, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_down_bf16(const GemmArgs& a, int grid, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  if (a.out_f32)
    hipLaunchKernelGGL((gemm_bf16_kernel<1, true>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<1, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
