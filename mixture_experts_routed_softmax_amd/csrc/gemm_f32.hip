// fp32 expert MLPs (small fp32 layers): one thread per (sorted row, output
// channel), fp32 FMA over the reduction.  Same arithmetic as the grouped
// GEMMs ("Experts backends", backend table, row deepgemm_megamoe: up
// projection with the gated activation, down projection), without tiling: these layers
// are tiny and exist for exact-precision parity.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// expert of sorted row r: largest e with offsets[e] <= r (and a non-empty segment)
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void gate_up_f32_kernel(GemmArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.P * a.N) return;
  const int r = (int)(idx / a.N);
  const int j = (int)(idx % a.N);
  const int e = expert_of_row(a.offsets, a.E, r);
  const int64_t src_row = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
  const float* x = (const float*)a.act + src_row * a.K;
  const float* wg = (const float*)a.w0 + ((int64_t)e * a.N + j) * a.K;
  const float* wu = (const float*)a.w1 + ((int64_t)e * a.N + j) * a.K;
  float g = 0.f, u = 0.f;
  for (int h = 0; h < a.K; ++h) {
    g = __builtin_fmaf(x[h], wg[h], g);
    u = __builtin_fmaf(x[h], wu[h], u);
  }
  float act;
  if (a.gate_act == 1) act = 0.5f * g * (1.0f + erff(g * 0.70710678118654752f));   // exact gelu
  else if (a.gate_act == 2) act = fmaxf(g, 0.0f);                                   // relu
  else act = g / (1.0f + expf(-g));                                                 // silu
  ((float*)a.out)[(int64_t)r * a.N + j] = act * u;
}

__global__ __launch_bounds__(256) void down_f32_kernel(GemmArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.P * a.N) return;
  const int r = (int)(idx / a.N);
  const int o = (int)(idx % a.N);
  const int e = expert_of_row(a.offsets, a.E, r);
  const float* h = (const float*)a.act + (int64_t)r * a.K;
  const float* wd = (const float*)a.w0 + ((int64_t)e * a.N + o) * a.K;
  float y = 0.f;
  for (int c = 0; c < a.K; ++c) y = __builtin_fmaf(h[c], wd[c], y);
  if (a.out_f32)
    ((float*)a.out)[(int64_t)r * a.N + o] = y;
  else
    ((uint16_t*)a.out)[(int64_t)r * a.N + o] = f32_to_bf16_bits(y);
}

}  // namespace

hipError_t launch_gate_up_f32(const GemmArgs& a, hipStream_t stream) {
  const int64_t n = a.P * a.N;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gate_up_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_down_f32(const GemmArgs& a, hipStream_t stream) {
  const int64_t n = a.P * a.N;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(down_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
