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
// bf16 logits come from v_mfma_f32_32x32x16_bf16 (router rows as the A
// operand, 32 experts per tile; token rows as B, 32 tokens per tile) in a grid
// of (token tile, expert tile, K slice) workgroups sized to fill the chip at
// any batch size; the slices' partial logits are added in a fixed order by
// the selection kernel.  Selection: one wave per token, 4 keys per lane, k
// rounds of a 64-lane argmax reduction.
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

// Top-k of one token's keys held by a wave (lane l owns experts l, l+64,
// l+128, l+192): k rounds of a 64-lane argmax (larger key wins, ties to the
// lower index), then the scores and routing weights; lane i < k writes slot i.
__device__ __forceinline__ void select_topk(float (&key)[4], bool (&taken)[4], int lane, int E, int k, int score,
                                            int renorm, float routed_scale, int32_t* ids_out, float* w_out) {
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
    ids_out[lane] = my_idx;
    w_out[lane] = s * routed_scale;
  }
}

// fp32 router (small fp32 layers): one workgroup owns 32 tokens and all
// experts, logits by fp32 FMA into LDS, then the wave-level selection.
__global__ __launch_bounds__(256) void route_topk_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    int64_t T, int H, int E, int k, int score, int renorm, float routed_scale,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  __shared__ float s_key[kTokPerBlock][kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kTokPerBlock;
  {
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
    select_topk(key, taken, lane, E, k, score, renorm, routed_scale, ids_out + tok * k, w_out + tok * k);
  }
}

// ---------------------------------------------------------------- split router
// bf16 logits as a grid of (32-token tile, 32-expert tile, K slice) workgroups
// so that the chip is filled at any batch size.  Each of the 4 waves of a
// workgroup takes every 4th 16-deep K step of the slice; the four partial
// tiles are added in LDS in wave order and the slice's partial logits written
// to part[slice][t][e].  topk_kernel adds the slices in slice order (a fixed
// order: deterministic; exact whenever the inputs' partial sums are exact in
// fp32) and selects.

__global__ __launch_bounds__(256) void logits_kernel(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ wr, int64_t T, int H,
                                                     int E, int steps_per_slice,
                                                     float* __restrict__ part) {
  __shared__ float s_p[4][32][33];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int e0 = blockIdx.y * 32;
  const int slice = blockIdx.z;
  const int nsteps = H / 16;
  const int s_begin = slice * steps_per_slice;
  const int s_end = min(nsteps, s_begin + steps_per_slice);
  int64_t tok = t0 + l32;
  tok = tok < T ? tok : T - 1;
  const int e = e0 + l32;
  const bool e_ok = e < E;
  const uint16_t* xrow = x + tok * H + hl * 8;
  const uint16_t* wrow = wr + (int64_t)(e_ok ? e : 0) * H + hl * 8;
  f32x16 acc = {};
  int st = s_begin + wave;
  for (; st + 12 < s_end; st += 16) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = *(const bf16x8*)(wrow + (st + 4 * u) * 16);
      b[u] = *(const bf16x8*)(xrow + (st + 4 * u) * 16);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!e_ok) a[u] = bf16x8{};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u], acc, 0, 0, 0);
    }
  }
  for (; st < s_end; st += 4) {
    bf16x8 a = *(const bf16x8*)(wrow + st * 16);
    bf16x8 b = *(const bf16x8*)(xrow + st * 16);
    if (!e_ok) a = bf16x8{};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
  // C[i][j]: i = expert in tile, j = token in tile
#pragma unroll
  for (int r = 0; r < 16; ++r) s_p[wave][(r >> 2) * 8 + hl * 4 + (r & 3)][l32] = acc[r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 32 * 32; idx += 256) {
    const int j = idx >> 5, i = idx & 31;   // token j, expert i: consecutive threads -> consecutive experts
    const int64_t t = t0 + j;
    if (t < T && e0 + i < E) {
      const float v = ((s_p[0][i][j] + s_p[1][i][j]) + s_p[2][i][j]) + s_p[3][i][j];
      part[((int64_t)slice * T + t) * E + e0 + i] = v;
    }
  }
}

// one wave per token: key = sum over slices + bias, then the top-k selection
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ part, int slices, int64_t T,
                                                   int E, const float* __restrict__ bias, int k, int score,
                                                   int renorm, float routed_scale, int32_t* __restrict__ ids_out,
                                                   float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= T) return;
  float key[4];
  bool taken[4];
  // Slices are added in ascending order; the loads of 8 slices are issued
  // together so that their latencies overlap.
  float z[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sl0 = 0; sl0 < slices; sl0 += 8) {
    float v[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[q][u] = (e < E && sl0 + u < slices) ? part[((int64_t)(sl0 + u) * T + tok) * E + e] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < 8; ++u) z[q] += v[q][u];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    taken[q] = !(e < E);
    key[q] = e < E ? z[q] + (bias ? bias[e] : 0.f) : -INFINITY;
  }
  select_topk(key, taken, lane, E, k, score, renorm, routed_scale, ids_out + tok * k, w_out + tok * k);
}

}  // namespace

int route_slices(int64_t T, int H, int E) {
  const int64_t tiles = ((T + 31) / 32) * ((E + 31) / 32);
  const int max_slices = (H / 16) / 4;   // at least one 16-deep step per wave
  int64_t sl = (512 + tiles - 1) / tiles;
  if (sl > max_slices) sl = max_slices;
  return (int)(sl < 1 ? 1 : sl);
}

size_t route_workspace_bytes(int64_t T, int H, int E, int act_bf16) {
  if (!act_bf16 || T == 0) return 0;
  return (size_t)route_slices(T, H, E) * T * E * sizeof(float);
}

hipError_t launch_route_topk(const void* x, const void* w_router, const float* bias, int64_t T,
                             int H, int E, int k, int act_bf16, int score, int renorm,
                             float routed_scale, int32_t* ids, float* w, float* part, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (act_bf16) {
    const int slices = route_slices(T, H, E);
    const int nsteps = H / 16;
    const int per = (nsteps + slices - 1) / slices;
    dim3 grid((unsigned)((T + 31) / 32), (unsigned)((E + 31) / 32), (unsigned)slices);
    hipLaunchKernelGGL(logits_kernel, grid, dim3(256), 0, stream, (const uint16_t*)x, (const uint16_t*)w_router,
                       T, H, E, per, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, part, slices, T, E, bias,
                       k, score, renorm, routed_scale, ids, w);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((T + kTokPerBlock - 1) / kTokPerBlock));
  hipLaunchKernelGGL(route_topk_f32_kernel, grid, dim3(256), 0, stream, (const float*)x, (const float*)w_router,
                     bias, T, H, E, k, score, renorm, routed_scale, ids, w);
  return hipGetLastError();
}

}  // namespace moe
