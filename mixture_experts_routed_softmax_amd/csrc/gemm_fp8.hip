// OCP-fp8 (e4m3) grouped GEMMs of the expert MLPs with 128 x 128 weight block
// scales and dynamic per-row activation scales.
//
// "Experts backends": FP8 experts carry float32 or UE8M0 block scales
// (paragraph under the backend table; note in "FP8 and FP4 quantized
// experts"), and the activations use dynamic per-row scales, never static
// per-tensor ones (same section).  With x^ = codes_x * s_x (per row, per 128
// channels) and W = codes_w * s_w (per 128 x 128 block):
//   g[r, j] = sum_kb s_w(j, kb) * s_x(r, kb) * sum_{k in kb} cx[r, k] * cw[j, k]
// i.e. one v_mfma_scale_f32_32x32x64_f8f6f4 pair per 128-deep chunk into a
// temporary, promoted into the fp32 accumulator with the product of the two
// scales.  gate/up then applies SwiGLU and quantizes h per row per 128
// channels (the tile covers exactly one 128-channel group) with
// s = amax / 448, codes = RNE_e4m3(h / s); down writes bf16 or fp32 rows.
//
// Tile geometry is the one of the bf16 kernels (256 weight rows x 128 token
// rows, 4 waves of 128 x 64), with a K step of 128 codes (128 B per row).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBMW = 256;
constexpr int kBNT = 128;
constexpr int kBK = 128;   // fp8 codes per K step = one scale block

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ float wscale(const void* s, int ue8m0, int64_t idx) {
  return ue8m0 ? e8m0_to_f32(((const uint8_t*)s)[idx]) : ((const float*)s)[idx];
}

template <int kMode, bool kOutF32>
__global__ __launch_bounds__(256, 1) void gemm_fp8_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[(kBMW + kBNT) * 128];
  __shared__ float s_amax[2][kBNT];
  const int w = xcd_work_index(a.sched->total);
  if (w < 0) return;
  const WorkItem it = ((const WorkItem*)(a.sched + 1))[w];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int K = a.K, N = a.N;
  const int KB = K / 128;
  const int e = it.expert;

  const int col = tid & 7;
  const int r0 = tid >> 3;
  const uint8_t* aptr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r0 + 32 * i;
    const uint8_t* src;
    int ch;
    if (kMode == 0) {
      ch = it.ntile * kGemmGateUpChannelsFp8 + (row & 127);
      src = (const uint8_t*)(row < 128 ? a.w0 : a.w1);
    } else {
      ch = it.ntile * kGemmDownChannelsFp8 + row;
      src = (const uint8_t*)a.w0;
    }
    ch = ch < N ? ch : N - 1;
    aptr[i] = src + ((int64_t)e * N + ch) * K + col * 16;
  }
  const uint8_t* bptr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = it.row_begin + r0 + 32 * i;
    r = r < it.row_end ? r : it.row_end - 1;
    const int64_t src_row = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
    bptr[i] = (const uint8_t*)a.act + src_row * K + col * 16;
  }
  // activation-scale rows of this lane's two token columns
  const float* sa_row[2];
#pragma unroll
  for (int tj = 0; tj < 2; ++tj) {
    int r = it.row_begin + wn * 64 + 32 * tj + (lane & 31);
    r = r < it.row_end ? r : it.row_end - 1;
    const int64_t src_row = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
    sa_row[tj] = a.act_scales + src_row * KB;
  }
  // weight-scale rows: gate/up tiles use block row ntile of s_gate / s_up; the
  // down tiles of wave wm use block row 2*ntile + wm.
  const int NB = (N + 127) / 128;
  int64_t sw_base0, sw_base1;
  if (kMode == 0) {
    sw_base0 = ((int64_t)e * NB + it.ntile) * KB;
    sw_base1 = sw_base0;
  } else {
    int br = it.ntile * 2 + wm;
    br = br < NB ? br : NB - 1;
    sw_base0 = ((int64_t)e * NB + br) * KB;
    sw_base1 = sw_base0;
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
  for (int kb = 0; kb < KB; ++kb) {
    const bool more = kb + 1 < KB;
    if (more) gload((kb + 1) * kBK);
    // scales of this K block
    float sw[4];
    if (kMode == 0) {
      const float sg = wscale(a.s0, a.scale_ue8m0, sw_base0 + kb);
      const float su = wscale(a.s1, a.scale_ue8m0, sw_base1 + kb);
      sw[0] = sw[1] = sg;
      sw[2] = sw[3] = su;
    } else {
      const float sd = wscale(a.s0, a.scale_ue8m0, sw_base0 + kb);
      sw[0] = sw[1] = sw[2] = sw[3] = sd;
    }
    const float sx0 = sa_row[0][kb], sx1 = sa_row[1][kb];

    i32x8 af[4][2], bf[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c0 = kk * 4 + lhi * 2;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        i32x4 lo = *(const i32x4*)(smem + swz(arow[t] + l32, c0));
        i32x4 hi = *(const i32x4*)(smem + swz(arow[t] + l32, c0 + 1));
        af[t][kk] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        i32x4 lo = *(const i32x4*)(smem + kBMW * 128 + swz(brow0 + 32 * t + l32, c0));
        i32x4 hi = *(const i32x4*)(smem + kBMW * 128 + swz(brow0 + 32 * t + l32, c0 + 1));
        bf[t][kk] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
    }
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
      const float sx = tj ? sx1 : sx0;
#pragma unroll
      for (int tp = 0; tp < 4; tp += 2) {
        f32x16 p0 = {}, p1 = {};
        p0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[tp][0], bf[tj][0], p0, 0, 0, 0, 127, 0, 127);
        p1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[tp + 1][0], bf[tj][0], p1, 0, 0, 0, 127, 0, 127);
        p0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[tp][1], bf[tj][1], p0, 0, 0, 0, 127, 0, 127);
        p1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[tp + 1][1], bf[tj][1], p1, 0, 0, 0, 127, 0, 127);
        const float m0 = sw[tp] * sx, m1 = sw[tp + 1] * sx;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[tp][tj][r] = __builtin_fmaf(p0[r], m0, acc[tp][tj][r]);
          acc[tp + 1][tj][r] = __builtin_fmaf(p1[r], m1, acc[tp + 1][tj][r]);
        }
      }
    }
    __syncthreads();
    if (more) sstore();
    __syncthreads();
  }

  if (kMode == 0) {
    // SwiGLU, then per-row quantization over the tile's 128 channels
    float hv[2][2][16];
    with_gate_act(a.gate_act, [&](auto k) {
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
#pragma unroll
        for (int i = 0; i < 2; ++i) gated16<decltype(k)::value>(acc[i][tj], acc[2 + i][tj], hv[tj][i]);
    });
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(hv[tj][i][r]));
      m = fmaxf(m, __shfl_xor(m, 32));
      if (lhi == 0) s_amax[wm][brow0 + 32 * tj + l32] = m;
    }
    __syncthreads();
    const int NG = N / 128;
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
      const int row = it.row_begin + brow0 + 32 * tj + l32;
      if (row >= it.row_end) continue;
      const float amax = fmaxf(s_amax[0][brow0 + 32 * tj + l32], s_amax[1][brow0 + 32 * tj + l32]);
      const float s = amax > 0.f ? amax / 448.0f : 1.0f;
      uint8_t* h = (uint8_t*)a.out + (int64_t)row * N;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = it.ntile * kGemmGateUpChannelsFp8 + wm * 64 + i * 32 + q * 8 + lhi * 4;
          const uint32_t pk = pack_fp8x4(hv[tj][i][q * 4 + 0] / s, hv[tj][i][q * 4 + 1] / s,
                                         hv[tj][i][q * 4 + 2] / s, hv[tj][i][q * 4 + 3] / s);
          *(uint32_t*)(h + ch) = pk;
        }
      if (wm == 0 && lhi == 0) a.out_scales[(int64_t)row * NG + it.ntile] = s;
    }
  } else {
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
      const int row = it.row_begin + brow0 + 32 * tj + l32;
      if (row >= it.row_end) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = it.ntile * kGemmDownChannelsFp8 + wm * 128 + t * 32 + q * 8 + lhi * 4;
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

}  // namespace

hipError_t launch_gate_up_fp8(const GemmArgs& a, int grid, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_fp8_kernel<0, false>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_down_fp8(const GemmArgs& a, int grid, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  if (a.out_f32)
    hipLaunchKernelGGL((gemm_fp8_kernel<1, true>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_fp8_kernel<1, false>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
