// Router: logits, key = logit + bias, top-k selection and routing weights.
//
// "Experts backends", opening paragraph: for each token a router selects k
// experts and the expert outputs are aggregated with routing weights.  The
// page gives no router formula; this kernel implements
//   key[t,e] = sum_h x[t,h] * w_router[e,h] + bias[e]        (fp32 accumulate)
//   ids[t,:] = the k largest keys, descending, ties -> lowest expert index
//   score    = softmax over all E keys, or sigmoid(key)
//   w[t,i]   = score(ids[t,i]) [ / sum_i score ] * routed_scale
//
// One workgroup (4 waves) owns 32 tokens and all E <= 256 experts.  bf16
// logits come from v_mfma_f32_32x32x16_bf16 with the router rows as the A
// operand (32 experts per tile) and the token rows as B (32 tokens): each wave
// owns the expert tiles w and w+4 over the whole hidden dimension, so no
// cross-wave reduction is needed.  The logits of the 32 tokens land in LDS,
// then each wave selects the top k for 8 tokens with 64-lane argmax
// reductions (4 keys per lane).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kTokPerBlock = 32;

struct KeyIdx {
  float key;
  int idx;
};

__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

template <bool kBf16>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const void* __restrict__ xv, const void* __restrict__ wrv, const float* __restrict__ bias,
    int64_t T, int H, int E, int k, int score, int renorm, float routed_scale,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  __shared__ float s_key[kTokPerBlock][kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kTokPerBlock;

  if constexpr (kBf16) {
    const uint16_t* x = (const uint16_t*)xv;
    const uint16_t* wr = (const uint16_t*)wrv;
    const int ntiles = (E + 31) / 32;
    const int krow = (lane >> 5) * 8;   // K offset of this lane inside a 16-deep step
    const int64_t tok = t0 + (lane & 31);
    const int64_t tok_c = tok < T ? tok : T - 1;  // clamp: results of padded rows are unused
    const uint16_t* xrow = x + tok_c * H + krow;
    for (int nt = wave; nt < ntiles; nt += 4) {
      const int e = nt * 32 + (lane & 31);
      const bool e_ok = e < E;
      const uint16_t* wrow = wr + (int64_t)(e_ok ? e : 0) * H + krow;
      f32x16 acc = {};
      int kk = 0;
      for (; kk + 64 <= H; kk += 64) {
        bf16x8 a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a[u] = *(const bf16x8*)(wrow + kk + 16 * u);
          b[u] = *(const bf16x8*)(xrow + kk + 16 * u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (!e_ok) a[u] = bf16x8{};
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u], acc, 0, 0, 0);
        }
      }
      for (; kk < H; kk += 16) {
        bf16x8 a = *(const bf16x8*)(wrow + kk);
        bf16x8 b = *(const bf16x8*)(xrow + kk);
        if (!e_ok) a = bf16x8{};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
      // C[i][j]: i = expert within tile, j = token; lane holds j = lane%32 and
      // i = (r/4)*8 + (lane/32)*4 + r%4.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int ei = nt * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (ei < E) s_key[lane & 31][ei] = acc[r];
      }
    }
  } else {
    const float* x = (const float*)xv;
    const float* wr = (const float*)wrv;
    for (int idx = tid; idx < kTokPerBlock * E; idx += 256) {
      int tl = idx / E, e = idx % E;
      int64_t tok = t0 + tl;
      if (tok >= T) continue;
      const float* xr = x + tok * H;
      const float* wrow = wr + (int64_t)e * H;
      float z = 0.f;
      for (int h = 0; h < H; ++h) z = __builtin_fmaf(xr[h], wrow[h], z);
      s_key[tl][e] = z;
    }
  }
  __syncthreads();

  // ---- selection: each wave handles 8 tokens
  for (int tl = wave; tl < kTokPerBlock; tl += 4) {
    const int64_t tok = t0 + tl;
    if (tok >= T) break;
    float key[4];
    bool taken[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int e = lane + 64 * q;
      taken[q] = !(e < E);
      key[q] = e < E ? s_key[tl][e] + (bias ? bias[e] : 0.f) : -INFINITY;
    }
    float my_key = 0.f;   // lane i < k keeps slot i
    int my_idx = 0;
    float kmax = 0.f;
    for (int i = 0; i < k; ++i) {
      float bk = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (!taken[q] && better(key[q], lane + 64 * q, bk, bi)) { bk = key[q]; bi = lane + 64 * q; }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        float ok = __shfl_xor(bk, off);
        int oi = __shfl_xor(bi, off);
        if (better(ok, oi, bk, bi)) { bk = ok; bi = oi; }
      }
      if ((bi & 63) == lane) taken[bi >> 6] = true;
      if (lane == i) { my_key = bk; my_idx = bi; }
      if (i == 0) kmax = bk;
    }
    float s;
    if (score == 0) {  // softmax over all experts
      float part = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q < E) part += expf(key[q] - kmax);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
      s = expf(my_key - kmax) / part;
    } else {
      s = 1.0f / (1.0f + expf(-my_key));
    }
    if (renorm) {
      float sum = lane < k ? s : 0.f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
      s = s / sum;
    }
    if (lane < k) {
      ids_out[tok * k + lane] = my_idx;
      w_out[tok * k + lane] = s * routed_scale;
    }
  }
}

}  // namespace

hipError_t launch_route_topk(const void* x, const void* w_router, const float* bias, int64_t T,
                             int H, int E, int k, int act_bf16, int score, int renorm,
                             float routed_scale, int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((T + kTokPerBlock - 1) / kTokPerBlock));
  if (act_bf16)
    hipLaunchKernelGGL(route_topk_kernel<true>, grid, dim3(256), 0, stream, x, w_router, bias, T, H,
                       E, k, score, renorm, routed_scale, ids, w);
  else
    hipLaunchKernelGGL(route_topk_kernel<false>, grid, dim3(256), 0, stream, x, w_router, bias, T,
                       H, E, k, score, renorm, routed_scale, ids, w);
  return hipGetLastError();
}

}  // namespace moe
