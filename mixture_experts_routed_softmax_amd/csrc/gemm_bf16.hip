// bf16 grouped GEMMs of the expert MLPs, one launch for all experts.
//
// "Experts backends": the selected tokens of every expert are projected
// through that expert's gated MLP (backend table, row deepgemm_megamoe:
// up projection, SwiGLU, down projection) as one grouped GEMM over the
// expert-sorted rows (rows grouped_mm / deepgemm).
//
//   gate/up : h[r, j] = silu(x_r . w_gate[e, j]) * (x_r . w_up[e, j])
//   down    : y[r, o] = h_r . w_down[e, o]
//
// Tile = 256 weight rows x 128 token rows, K step 64, 4 waves (2 x 2), each
// wave 128 weight rows x 64 tokens = 4 x 2 tiles of v_mfma_f32_32x32x16_bf16.
// Weights are the A operand (32 output channels per MFMA tile) and tokens the
// B operand, so every lane ends with 16 channels of one token: 4 runs of 4
// consecutive channels, written as 8-byte (bf16) or 16-byte (fp32) stores.
// For gate/up the 256 weight rows are the gate and up rows of the same 128
// channels, and each wave holds matching gate/up accumulators, so SwiGLU is
// applied in registers.
//
// Both tiles are staged through LDS (48 KB, one buffer, register prefetch of
// the next K step during the MFMAs), rows of 128 B with the 16-byte chunks
// XOR-swizzled by (row & 7) so that the MFMA fragment reads are bank-conflict
// free.  The work items (expert, row tile, channel tile) come from a device
// schedule built from the scanned expert offsets; consecutive items share an
// expert's weights and are mapped to the same XCD.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBMW = 256;   // weight rows per tile
constexpr int kBNT = 128;   // token rows per tile
constexpr int kBK = 64;     // bf16 elements per K step (128 B per row)

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int kMode, bool kOutF32>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[(kBMW + kBNT) * 128];
  const int w = xcd_work_index(a.sched->total);
  if (w < 0) return;
  const WorkItem it = ((const WorkItem*)(a.sched + 1))[w];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int K = a.K, N = a.N;
  const int e = it.expert;

  // ---- global -> register assignment: row r0 + 32 i, 16-byte chunk `col`
  const int col = tid & 7;
  const int r0 = tid >> 3;
  const uint16_t* aptr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r0 + 32 * i;
    const uint16_t* src;
    int ch;
    if (kMode == 0) {
      ch = it.ntile * kGemmGateUpChannels + (row & 127);
      src = (const uint16_t*)(row < 128 ? a.w0 : a.w1);
    } else {
      ch = it.ntile * kGemmDownChannels + row;
      src = (const uint16_t*)a.w0;
    }
    ch = ch < N ? ch : N - 1;   // rows past N are computed but never stored
    aptr[i] = src + ((int64_t)e * N + ch) * K + col * 8;
  }
  const uint16_t* bptr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = it.row_begin + r0 + 32 * i;
    r = r < it.row_end ? r : it.row_end - 1;
    const int64_t src_row = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
    bptr[i] = (const uint16_t*)a.act + src_row * K + col * 8;
  }

  i32x4 ra[8], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = *(const i32x4*)(aptr[i] + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = *(const i32x4*)(bptr[i] + k0);
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) *(i32x4*)(smem + swz(r0 + 32 * i, col)) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *(i32x4*)(smem + kBMW * 128 + swz(r0 + 32 * i, col)) = rb[i];
  };

  // LDS rows of this wave's four weight tiles and two token tiles
  int arow[4];
  if (kMode == 0) {
    arow[0] = wm * 64;
    arow[1] = wm * 64 + 32;
    arow[2] = 128 + wm * 64;
    arow[3] = 128 + wm * 64 + 32;
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) arow[t] = wm * 128 + 32 * t;
  }
  const int brow0 = wn * 64;

  f32x16 acc[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t][0] = acc[t][1] = f32x16{};

  gload(0);
  sstore();
  __syncthreads();
  const int l32 = lane & 31, lhi = lane >> 5;
  for (int k0 = 0; k0 < K; k0 += kBK) {
    const bool more = k0 + kBK < K;
    if (more) gload(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = kk * 2 + lhi;
      bf16x8 af[4], bf[2];
#pragma unroll
      for (int t = 0; t < 4; ++t) af[t] = *(const bf16x8*)(smem + swz(arow[t] + l32, chunk));
#pragma unroll
      for (int t = 0; t < 2; ++t)
        bf[t] = *(const bf16x8*)(smem + kBMW * 128 + swz(brow0 + 32 * t + l32, chunk));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[t][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t], bf[0], acc[t][0], 0, 0, 0);
        acc[t][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t], bf[1], acc[t][1], 0, 0, 0);
      }
    }
    __syncthreads();
    if (more) sstore();
    __syncthreads();
  }

  // ---- epilogue.  Lane holds token column l32 and channels
  // (r/4)*8 + lhi*4 + r%4 of each 32-row weight tile.
#pragma unroll
  for (int tj = 0; tj < 2; ++tj) {
    const int row = it.row_begin + brow0 + 32 * tj + l32;
    if (row >= it.row_end) continue;
    if (kMode == 0) {
      uint16_t* h = (uint16_t*)a.out + (int64_t)row * N;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = it.ntile * kGemmGateUpChannels + wm * 64 + i * 32 + q * 8 + lhi * 4;
          if (ch >= N) continue;
          uint16_t v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float g = acc[i][tj][q * 4 + c];
            const float u = acc[2 + i][tj][q * 4 + c];
            v[c] = f32_to_bf16_bits(silu(g) * u);
          }
          i32x2 pk = {(int)(v[0] | ((uint32_t)v[1] << 16)), (int)(v[2] | ((uint32_t)v[3] << 16))};
          *(i32x2*)(h + ch) = pk;
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = it.ntile * kGemmDownChannels + wm * 128 + t * 32 + q * 8 + lhi * 4;
          if (ch >= N) continue;
          if (kOutF32) {
            f32x4 v = {acc[t][tj][q * 4 + 0], acc[t][tj][q * 4 + 1], acc[t][tj][q * 4 + 2],
                       acc[t][tj][q * 4 + 3]};
            *(f32x4*)((float*)a.out + (int64_t)row * N + ch) = v;
          } else {
            uint16_t v[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = f32_to_bf16_bits(acc[t][tj][q * 4 + c]);
            i32x2 pk = {(int)(v[0] | ((uint32_t)v[1] << 16)), (int)(v[2] | ((uint32_t)v[3] << 16))};
            *(i32x2*)((uint16_t*)a.out + (int64_t)row * N + ch) = pk;
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gate_up_bf16(const GemmArgs& a, int grid, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<0, false>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_down_bf16(const GemmArgs& a, int grid, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  if (a.out_f32)
    hipLaunchKernelGGL((gemm_bf16_kernel<1, true>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<1, false>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
