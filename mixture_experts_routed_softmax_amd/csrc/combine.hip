// Weighted combine back to token order ("Experts backends", opening
// paragraph: the expert outputs are aggregated with the routing weights):
//   out[t, :] = sum_{i<k} w[t, i] * y_sorted[inv[t*k + i], :]
// fp32 sums in slot order, one rounding to the output type, no atomics.
// One workgroup per (token, 2048 channels), 8 channels (one 16-byte bf16
// load per slot) per thread; the loads of up to 8 slots are issued together.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

template <bool kYF32, bool kOutF32>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int k, int H,
                                                      void* __restrict__ out) {
  __shared__ int s_row[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    // a pair without a row of y (inv outside [0, T*k): an out-of-range id)
    // contributes nothing
    const int64_t row = inv[t * k + threadIdx.x];
    s_row[threadIdx.x] = row >= 0 && row < (int64_t)gridDim.x * k ? (int)row : -1;
    s_w[threadIdx.x] = w[t * k + threadIdx.x];
  }
  __syncthreads();
  const int c = blockIdx.y * 256 + threadIdx.x;   // group of 8 channels
  if (c < H / 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < k; i0 += 8) {
      // the loads of 8 slots first, then the slot-ordered accumulation
      f32x4 v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v0[u] = f32x4{};
        v1[u] = f32x4{};
        if (i0 + u < k && s_row[i0 + u] >= 0) {
          const int64_t base = (int64_t)s_row[i0 + u] * H + c * 8;
          if (kYF32) {
            v0[u] = *(const f32x4*)((const float*)y + base);
            v1[u] = *(const f32x4*)((const float*)y + base + 4);
          } else {
            v0[u] = __builtin_bit_cast(f32x4, *(const i32x4*)((const uint16_t*)y + base));
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (i0 + u >= k) break;
        if (s_row[i0 + u] < 0) continue;
        const float wi = s_w[i0 + u];
        if (kYF32) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[q] = __builtin_fmaf(wi, v0[u][q], acc[q]);
            acc[4 + q] = __builtin_fmaf(wi, v1[u][q], acc[4 + q]);
          }
        } else {
          const i32x4 v = __builtin_bit_cast(i32x4, v0[u]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t two = (uint32_t)v[q];
            acc[2 * q] = __builtin_fmaf(wi, bf16_bits_to_f32((uint16_t)(two & 0xffff)), acc[2 * q]);
            acc[2 * q + 1] = __builtin_fmaf(wi, bf16_bits_to_f32((uint16_t)(two >> 16)), acc[2 * q + 1]);
          }
        }
      }
    }
    const int64_t o = t * H + c * 8;
    if (kOutF32) {
      *(f32x4*)((float*)out + o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *(f32x4*)((float*)out + o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      i32x4 pk;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pk[q] = (int)pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      *(i32x4*)((uint16_t*)out + o) = pk;
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_f32, const int32_t* inv, const float* w, int64_t T,
                          int k, int H, void* out, int out_f32, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)T, (unsigned)((H / 8 + 255) / 256)), block(256);
  if (y_f32 && out_f32)
    hipLaunchKernelGGL((combine_kernel<true, true>), grid, block, 0, stream, y, inv, w, k, H, out);
  else if (y_f32)
    hipLaunchKernelGGL((combine_kernel<true, false>), grid, block, 0, stream, y, inv, w, k, H, out);
  else if (out_f32)
    hipLaunchKernelGGL((combine_kernel<false, true>), grid, block, 0, stream, y, inv, w, k, H, out);
  else
    hipLaunchKernelGGL((combine_kernel<false, false>), grid, block, 0, stream, y, inv, w, k, H, out);
  return hipGetLastError();
}

}  // namespace moe
