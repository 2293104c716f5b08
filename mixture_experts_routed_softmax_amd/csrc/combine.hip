// Weighted combine back to token order ("Experts backends", opening
// paragraph: a token's output adds up its experts' results, each scaled by
// its routing weight):
//   out[t, :] = sum_{i<k} w[t, i] * y_sorted[inv[t*k + i], :]
// fp32 sums in slot order, one rounding to the output type, no atomics.
// One workgroup per (token, 2048 channels), 8 channels (one 16-byte bf16
// load per slot) per thread; the loads of up to 8 slots are issued together.
// y is read once and out written once: streaming (non-temporal) accesses
// (dsv3_bf16: 213 -> 200 us; workgroups of 128 threads instead of 256
// measured 220 us).
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
            v0[u] = __builtin_nontemporal_load((const f32x4*)((const float*)y + base));
            v1[u] = __builtin_nontemporal_load((const f32x4*)((const float*)y + base + 4));
          } else {
            v0[u] = __builtin_bit_cast(f32x4, __builtin_nontemporal_load((const i32x4*)((const uint16_t*)y + base)));
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
      __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, (f32x4*)((float*)out + o));
      __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, (f32x4*)((float*)out + o + 4));
    } else {
      i32x4 pk;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pk[q] = (int)pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      __builtin_nontemporal_store(pk, (i32x4*)((uint16_t*)out + o));
    }
  }
}

// The combine after a streaming down launch without its reduction launch.
// When that launch was split (S > 1, the same function of its item count as
// the launch's), y row r of channel tile nt is the sum, in split order, of
// the partial rows of the units (item, 0 .. S-1), item = rowinfo[r] / 64 + nt,
// at row rowinfo[r] % 64 of each partial tile, rounded to y's type; else the
// launch wrote y.  Then out[t, :] as in combine_kernel.
template <bool kYF32, bool kOutF32>
__global__ __launch_bounds__(256) void combine_split_kernel(const void* __restrict__ y,
                                                            const float* __restrict__ partial,
                                                            const int32_t* __restrict__ rowinfo,
                                                            const Schedule* __restrict__ sched, int ksteps,
                                                            int slots, const int32_t* __restrict__ inv,
                                                            const float* __restrict__ w, int k, int H,
                                                            void* __restrict__ out) {
  __shared__ int s_row[kMaxTopK];
  __shared__ int s_info[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int64_t t = blockIdx.x;
  const int S = stream_splits(sched->total, ksteps, slots);
  if (threadIdx.x < k) {
    const int64_t row = inv[t * k + threadIdx.x];
    const bool ok = row >= 0 && row < (int64_t)gridDim.x * k;
    s_row[threadIdx.x] = ok ? (int)row : -1;
    s_info[threadIdx.x] = ok && S > 1 ? rowinfo[row] : 0;
    s_w[threadIdx.x] = w[t * k + threadIdx.x];
  }
  __syncthreads();
  const int c = blockIdx.y * 256 + threadIdx.x;   // group of 8 channels
  if (c >= H / 8) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int nt = c / 32, cc = (c % 32) * 8;   // channel tile, channel within it
  for (int i = 0; i < k; ++i) {
    if (s_row[i] < 0) continue;
    float v[8];
    if (S == 1) {
      const int64_t base = (int64_t)s_row[i] * H + c * 8;
      if (kYF32) {
        const f32x4 v0 = *(const f32x4*)((const float*)y + base);
        const f32x4 v1 = *(const f32x4*)((const float*)y + base + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = v0[q];
          v[4 + q] = v1[q];
        }
      } else {
        const i32x4 b = *(const i32x4*)((const uint16_t*)y + base);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] = bf16_bits_to_f32((uint16_t)((uint32_t)b[q] & 0xffff));
          v[2 * q + 1] = bf16_bits_to_f32((uint16_t)((uint32_t)b[q] >> 16));
        }
      }
    } else {
      const int info = s_info[i];
      const int64_t u0 = (int64_t)(info / 64 + nt) * S;
      const float* p0 = partial + u0 * kStreamPartFloats + (info % 64) * 256 + cc;
      // the loads of all (at most kStreamMaxSplit) splits first, then the
      // split-ordered sum
      f32x4 a0[kStreamMaxSplit], a1[kStreamMaxSplit];
#pragma unroll
      for (int sp = 0; sp < kStreamMaxSplit; ++sp) {
        const int64_t o = (int64_t)(sp < S ? sp : S - 1) * kStreamPartFloats;   // (unconditional loads)
        a0[sp] = *(const f32x4*)(p0 + o);
        a1[sp] = *(const f32x4*)(p0 + o + 4);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = 0.f;
#pragma unroll
      for (int sp = 0; sp < kStreamMaxSplit; ++sp) {
        if (sp >= S) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] += a0[sp][q];
          v[4 + q] += a1[sp][q];
        }
      }
      if (!kYF32) {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = bf16_bits_to_f32(f32_to_bf16_bits(v[q]));
      }
    }
    const float wi = s_w[i];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(wi, v[q], acc[q]);
  }
  const int64_t o = t * H + c * 8;
  if (kOutF32) {
    *(f32x4*)((float*)out + o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)((float*)out + o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    i32x4 pk;
#pragma unroll
    for (int q = 0; q < 4; ++q) pk[q] = (int)pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    *(i32x4*)((uint16_t*)out + o) = pk;
  }
}

// The same combine for small batches, where a split down launch leaves up to
// k * 16 partial rows per token: one workgroup per (token, 32 channels), so
// that the partial reads spread over many CUs.  Thread (q, g) loads the 8
// channels g of (slot, split) pair q = slot * S + split into LDS, a chunk of
// slots at a time; thread c < 32 then sums channel c of each slot over its
// splits in split order, rounds to y's type and accumulates the slots in slot
// order, exactly as combine_split_kernel does.
constexpr int kFineChannels = 32;
constexpr int kFinePairs = 128;   // (slot, split) pairs staged in LDS at once

template <bool kYF32, bool kOutF32>
__global__ __launch_bounds__(256) void combine_split_fine_kernel(const void* __restrict__ y,
                                                                 const float* __restrict__ partial,
                                                                 const int32_t* __restrict__ rowinfo,
                                                                 const Schedule* __restrict__ sched, int ksteps,
                                                                 int slots, const int32_t* __restrict__ inv,
                                                                 const float* __restrict__ w, int k, int H,
                                                                 void* __restrict__ out) {
  __shared__ int s_row[kMaxTopK];
  __shared__ int s_info[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  __shared__ float s_v[kFinePairs][kFineChannels];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int S = stream_splits(sched->total, ksteps, slots);
  if (tid < k) {
    const int64_t row = inv[t * k + tid];
    const bool ok = row >= 0 && row < (int64_t)gridDim.x * k;
    s_row[tid] = ok ? (int)row : -1;
    s_info[tid] = ok && S > 1 ? rowinfo[row] : 0;
    s_w[tid] = w[t * k + tid];
  }
  __syncthreads();
  const int ch0 = blockIdx.y * kFineChannels;         // first channel of this workgroup
  const int g = tid & 3;                              // 8-channel group of this thread
  const int c8 = ch0 / 8 + g;                         // global group of 8 channels
  const int nt = c8 / 32, cc = (c8 % 32) * 8;         // channel tile, channel within it
  const int kc = kFinePairs / S < k ? kFinePairs / S : k;   // slots per chunk (S <= 16)
  float acc = 0.f;
  for (int i0 = 0; i0 < k; i0 += kc) {
    const int npairs = (k - i0 < kc ? k - i0 : kc) * S;
    for (int q = tid >> 2; q < npairs; q += 64) {
      const int i = i0 + q / S, sp = q % S;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (s_row[i] >= 0) {
        if (S == 1) {
          const int64_t base = (int64_t)s_row[i] * H + c8 * 8;
          if (kYF32) {
            const f32x4 v0 = *(const f32x4*)((const float*)y + base);
            const f32x4 v1 = *(const f32x4*)((const float*)y + base + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              v[j] = v0[j];
              v[4 + j] = v1[j];
            }
          } else {
            const i32x4 b = *(const i32x4*)((const uint16_t*)y + base);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              v[2 * j] = bf16_bits_to_f32((uint16_t)((uint32_t)b[j] & 0xffff));
              v[2 * j + 1] = bf16_bits_to_f32((uint16_t)((uint32_t)b[j] >> 16));
            }
          }
        } else {
          const int info = s_info[i];
          const float* p = partial + ((int64_t)(info / 64 + nt) * S + sp) * kStreamPartFloats + (info % 64) * 256 + cc;
          const f32x4 v0 = *(const f32x4*)p;
          const f32x4 v1 = *(const f32x4*)(p + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] = v0[j];
            v[4 + j] = v1[j];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) s_v[q][g * 8 + j] = v[j];
    }
    __syncthreads();
    if (tid < kFineChannels) {
      for (int ii = 0; ii < npairs / S; ++ii) {
        const int i = i0 + ii;
        if (s_row[i] < 0) continue;
        float v = 0.f;
        for (int sp = 0; sp < S; ++sp) v += s_v[ii * S + sp][tid];
        if (!kYF32 && S > 1) v = bf16_bits_to_f32(f32_to_bf16_bits(v));
        acc = __builtin_fmaf(s_w[i], v, acc);
      }
    }
    __syncthreads();
  }
  if (tid < kFineChannels) {
    const int64_t o = t * H + ch0 + tid;
    if (kOutF32) ((float*)out)[o] = acc;
    else ((uint16_t*)out)[o] = f32_to_bf16_bits(acc);
  }
}

}  // namespace

hipError_t launch_combine_stream(const void* y, int y_f32, const float* partial, const int32_t* rowinfo,
                                 const Schedule* sched, int ksteps, int slots, const int32_t* inv, const float* w,
                                 int64_t T, int k, int H, void* out, int out_f32, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (H % 8 != 0 || k > kMaxTopK) return hipErrorInvalidValue;
  const bool fine = T <= kCombineFineMaxT && H % kFineChannels == 0;
  dim3 grid((unsigned)T, (unsigned)(fine ? H / kFineChannels : (H / 8 + 255) / 256)), block(256);
#define MOE_COMBINE_SPLIT(YF, OF)                                                                          \
  do {                                                                                                     \
    if (fine)                                                                                              \
      hipLaunchKernelGGL((combine_split_fine_kernel<YF, OF>), grid, block, 0, stream, y, partial, rowinfo, \
                         sched, ksteps, slots, inv, w, k, H, out);                                        \
    else                                                                                                   \
      hipLaunchKernelGGL((combine_split_kernel<YF, OF>), grid, block, 0, stream, y, partial, rowinfo,      \
                         sched, ksteps, slots, inv, w, k, H, out);                                        \
  } while (0)
  if (y_f32 && out_f32) MOE_COMBINE_SPLIT(true, true);
  else if (y_f32) MOE_COMBINE_SPLIT(true, false);
  else if (out_f32) MOE_COMBINE_SPLIT(false, true);
  else MOE_COMBINE_SPLIT(false, false);
#undef MOE_COMBINE_SPLIT
  return hipGetLastError();
}

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
