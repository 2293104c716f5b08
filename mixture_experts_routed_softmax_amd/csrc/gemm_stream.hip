// Weight-streaming expert GEMMs for decode-sized batches (T <= 64, so every
// expert owns at most 64 token rows), on tile-packed weights, bf16 or fp8.
//
// "Experts backends", section "Decode-stage switching": small token counts
// call for a different execution scheme than the grouped GEMM of large
// batches.  At T <= 64 the layer is bound by reading the touched experts'
// weights from HBM; this kernel reads every weight byte exactly once, spread
// over all compute units, and multiplies it against the (L2-resident) token
// rows of its expert:
//   gate/up : h[r, j] = silu(x_r . w_gate[e, j]) * (x_r . w_up[e, j])
//   down    : y[r, o] = h_r . w_down[e, o]
//
// One workgroup per (touched expert, packed 256-row tile); 4 waves, each
// owning 64 weight rows (gate/up: the gate and up rows of 32 channels) for all
// of the expert's tokens (one or two 32-token MFMA tiles).  Weights go from
// the contiguous packed chunks straight into registers in MFMA layout through
// a register ring of 4 (bf16) or 3 (fp8) K steps (no LDS, no barriers); token fragments are loaded
// from global memory (they stay in L2).  FP8: the partial sum of every
// 64-deep step is promoted with the s_w * s_x of its 128-deep scale block; the
// gate/up epilogue quantizes h per row over the block's 128 channels
// (s = amax / 448).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kRowB = 64;       // packed bytes per row per K step
constexpr int kChunk = 256 * kRowB;
template <bool kFp8>
constexpr int kRing = kFp8 ? 3 : 4;   // K steps in flight per wave

__device__ __forceinline__ int pswz(int row, int chunk) {
  return row * kRowB + ((chunk ^ ((row >> 2) & 3)) << 4);
}

__device__ __forceinline__ float wscale(const void* s, int ue8m0, int64_t idx) {
  return ue8m0 ? e8m0_to_f32(((const uint8_t*)s)[idx]) : ((const float*)s)[idx];
}

template <bool kFp8, int NT>
struct Step {
  i32x4 a[2][2];    // [weight tile][16-byte piece]
  i32x4 b[NT][2];   // [token tile][16-byte piece]
};

template <bool kFp8, int kMode, bool kOutF32, int NT>
__device__ __forceinline__ void stream_tile(const GemmArgs& a, const WorkItem& it) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int e = it.expert;
  const int K = a.K, N = a.N;
  const int elt = kFp8 ? 1 : 2;
  const int KT = K * elt / kRowB;

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
  // bf16: logical chunks 2*kk + hl (kk = 0, 1); fp8: 2*hl and 2*hl + 1
  int aoff[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int q = 0; q < 2; ++q) aoff[t][q] = pswz(arow[t], kFp8 ? hl * 2 + q : q * 2 + hl);
  // token rows of this lane
  const uint8_t* brow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int r = it.row_begin + j * 32 + l32;
    r = r < it.row_end ? r : it.row_end - 1;
    const int64_t src_row = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
    brow[j] = (const uint8_t*)a.act + src_row * (int64_t)K * elt;
  }
  // byte offsets (within a K step) of the token pieces, same K mapping as A
  int boff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) boff[q] = (kFp8 ? hl * 2 + q : q * 2 + hl) * 16;

  typedef Step<kFp8, NT> S;
  auto load = [&](S& st, int kt) {
    const uint8_t* ck = abase + (int64_t)kt * kChunk;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q) st.a[t][q] = *(const i32x4*)(ck + aoff[t][q]);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q) st.b[j][q] = *(const i32x4*)(brow[j] + (int64_t)kt * kRowB + boff[q]);
  };

  f32x16 acc[2][NT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[t][j] = f32x16{};

  // fp8 scale bookkeeping
  const int KB = K / 128;
  int64_t sw0 = 0, sw1 = 0;
  const float* sa[NT] = {};
  if constexpr (kFp8) {
    const int NBr = (N + 127) / 128;
    if (kMode == 0) {
      sw0 = ((int64_t)e * NBr + it.ntile) * KB;
      sw1 = sw0;
    } else {
      int br = it.ntile * 2 + (wave >> 1);
      br = br < NBr ? br : NBr - 1;
      sw0 = ((int64_t)e * NBr + br) * KB;
      sw1 = sw0;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      int r = it.row_begin + j * 32 + l32;
      r = r < it.row_end ? r : it.row_end - 1;
      const int64_t src_row = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
      sa[j] = a.act_scales + src_row * KB;
    }
  }

  auto consume = [&](const S& st, int kt) {
    if constexpr (kFp8) {
      // both 64-deep halves of a 128-deep scale block carry the same scales,
      // so each step's partial sum is promoted on its own
      const int kb = kt >> 1;
      const float s0 = wscale(a.s0, a.scale_ue8m0, sw0 + kb);
      const float s1 = wscale(kMode == 0 ? a.s1 : a.s0, a.scale_ue8m0, sw1 + kb);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const i32x8 bv = {st.b[j][0].x, st.b[j][0].y, st.b[j][0].z, st.b[j][0].w,
                          st.b[j][1].x, st.b[j][1].y, st.b[j][1].z, st.b[j][1].w};
        const float sx = sa[j][kb];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const i32x8 av = {st.a[t][0].x, st.a[t][0].y, st.a[t][0].z, st.a[t][0].w,
                            st.a[t][1].x, st.a[t][1].y, st.a[t][1].z, st.a[t][1].w};
          const f32x16 p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, f32x16{}, 0, 0, 0, 127, 0, 127);
          const float m = (t == 0 ? s0 : s1) * sx;
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
  constexpr int R = kRing<kFp8>;
  S ring[R];
#pragma unroll
  for (int d = 0; d < R; ++d)
    if (d < KT) load(ring[d], d);
  for (int kt0 = 0; kt0 < KT; kt0 += R) {
#pragma unroll
    for (int d = 0; d < R; ++d) {
      const int kt = kt0 + d;
      if (kt < KT) {
        consume(ring[d], kt);
        if (kt + R < KT) load(ring[d], kt + R);
      }
    }
  }

  // ---- epilogue
  if (kMode == 0) {
    const int ch0 = it.ntile * 128 + wave * 32;
    if constexpr (kFp8) {
      __shared__ float s_amax[4][64];
      float hv[NT][16];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        float m = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          hv[j][r] = silu(acc[0][j][r]) * acc[1][j][r];
          m = fmaxf(m, fabsf(hv[j][r]));
        }
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
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int row = it.row_begin + j * 32 + l32;
        if (row >= it.row_end) continue;
        uint16_t* h = (uint16_t*)a.out + (int64_t)row * N;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = ch0 + q * 8 + hl * 4;
          if (ch >= N) continue;
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = silu(acc[0][j][q * 4 + c]) * acc[1][j][q * 4 + c];
          *(i32x2*)(h + ch) = i32x2{(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
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

template <bool kFp8, int kMode, bool kOutF32>
__global__ __launch_bounds__(256, 2) void gemm_stream_kernel(GemmArgs a) {
  const int w = xcd_work_index(a.sched->total);
  if (w < 0) return;
  const WorkItem it = ((const WorkItem*)(a.sched + 1))[w];
  if (it.row_end - it.row_begin > 32)
    stream_tile<kFp8, kMode, kOutF32, 2>(a, it);
  else
    stream_tile<kFp8, kMode, kOutF32, 1>(a, it);
}

}  // namespace

hipError_t launch_gemm_stream(const GemmArgs& a, int fp8, int mode, int grid, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  dim3 g(grid), b(256);
  if (fp8) {
    if (mode == 0) hipLaunchKernelGGL((gemm_stream_kernel<true, 0, false>), g, b, 0, stream, a);
    else if (a.out_f32) hipLaunchKernelGGL((gemm_stream_kernel<true, 1, true>), g, b, 0, stream, a);
    else hipLaunchKernelGGL((gemm_stream_kernel<true, 1, false>), g, b, 0, stream, a);
  } else {
    if (mode == 0) hipLaunchKernelGGL((gemm_stream_kernel<false, 0, false>), g, b, 0, stream, a);
    else if (a.out_f32) hipLaunchKernelGGL((gemm_stream_kernel<false, 1, true>), g, b, 0, stream, a);
    else hipLaunchKernelGGL((gemm_stream_kernel<false, 1, false>), g, b, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace moe
