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
#include "topk_select.h"

namespace moe {

namespace {

constexpr int kTokPerBlock = 32;

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
      key[q] = e < E ? nan_to_neg_inf(s_key[tl][e] + (bias ? bias[e] : 0.f)) : -INFINITY;
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

// ------------------------------------------------- LDS-staged router (large T)
// For large batches: a workgroup owns 64 tokens (128 for kEP = 256) and all
// experts (padded to kEP = 64, 128 or 256 rows) over a K slice.  The token and router rows of a
// 64-deep K chunk are brought into LDS by global_load_lds (one 1 KB
// instruction = 8 rows x 128 B, rows swizzled chunk ^ (row & 7)), 3 chunks in
// flight, so each row is read once per workgroup in whole cache lines.
// 8 waves; kWT = 8 / (kEP / 32) waves share a 32-expert tile: one wave takes
// every token tile, two waves one token tile each, four waves one token tile
// and every other 16-deep slice (their partial tiles are added in a fixed
// order).  The slice's logits go to part[slice][t][e] as in logits_kernel.
// tokens per workgroup: 128 when the experts pad to 256 rows (the router
// rows, re-read by every workgroup, then carry twice the tokens), else 64
__host__ __device__ constexpr int big_tok(int ep) { return ep > 128 ? 128 : 64; }
constexpr int kRouteStages = 3;
typedef __attribute__((address_space(3))) void* lds_ptr;

// 16 bytes per lane from global memory straight into LDS (wave base + lane * 16)
__device__ __forceinline__ void route_lds_load16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds_wave_base, 16, 0, 0);
}

__device__ __forceinline__ int rswz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int kEP>
__global__ __launch_bounds__(512) void logits_lds_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wr, int64_t T, int H,
                                                         int E, int chunks_per_slice, float* __restrict__ part) {
  constexpr int kBigTok = big_tok(kEP);
  constexpr int kXB = kBigTok * 128;                  // token bytes per stage
  constexpr int kStage = kXB + kEP * 128;
  constexpr int kXI = kBigTok / 64;                   // token DMA instructions per wave per chunk
  constexpr int kWI = kEP / 64;                       // router DMA instructions per wave per chunk
  constexpr int kLoads = kXI + kWI;
  constexpr int kET = kEP / 32, kWT = 8 / kET;       // expert tiles, waves per expert tile
  constexpr int kNJ = kWT == 1 ? kBigTok / 32 : 1;    // token tiles per wave
  constexpr int kUStep = kWT == 4 ? 2 : 1;            // 16-deep slices: every kUStep-th
  static_assert(kWT == 1 || kBigTok == 64, "two or four waves per expert tile split 64 tokens");
  static_assert((kEP + 1) * kBigTok * 4 <= kRouteStages * kStage, "logit tile fits the ring");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRouteStages * kStage];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31, hl = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * kBigTok;
  const int nchunks = H / 64;
  const int c0 = blockIdx.y * chunks_per_slice;
  const int c1 = min(nchunks, c0 + chunks_per_slice);
  // DMA sources: token rows (i*8 + wave)*8 + lane/8, router rows likewise
  const int slot = lane & 7;
  const uint16_t* xsrc[kXI];
#pragma unroll
  for (int i = 0; i < kXI; ++i) {
    const int r = (i * 8 + wv) * 8 + (lane >> 3);
    int64_t t = t0 + r;
    t = t < T ? t : T - 1;
    xsrc[i] = x + t * H + ((slot ^ (r & 7)) * 8);
  }
  const uint16_t* wsrc[kWI];
#pragma unroll
  for (int i = 0; i < kWI; ++i) {
    const int r = (i * 8 + wv) * 8 + (lane >> 3);
    const int e = r < E ? r : E - 1;
    wsrc[i] = wr + (int64_t)e * H + ((slot ^ (r & 7)) * 8);
  }
  auto issue = [&](int stage, int c) {
    uint8_t* sb = smem + stage * kStage;
#pragma unroll
    for (int i = 0; i < kXI; ++i) route_lds_load16(xsrc[i] + c * 64, sb + (i * 8 + wv) * 1024);
#pragma unroll
    for (int i = 0; i < kWI; ++i) route_lds_load16(wsrc[i] + c * 64, sb + kXB + (i * 8 + wv) * 1024);
  };
  const int et = wave / kWT, sub = wave % kWT;
  const int j0 = kWT == 1 ? 0 : (sub & 1);
  const int u0 = kWT == 4 ? (sub >> 1) : 0;
  f32x16 acc[kNJ] = {};
  if (c0 < c1) issue(0, c0);
  if (c0 + 1 < c1) issue(1, c0 + 1);
  for (int c = c0; c < c1; ++c) {
    if (c + 1 < c1) __builtin_amdgcn_s_waitcnt((kLoads & 15) | ((kLoads >> 4) << 14) | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
    __syncthreads();   // chunk c landed for all; chunk c-1's stage is free
    if (c + 2 < c1) issue((c + 2 - c0) % kRouteStages, c + 2);
    const uint8_t* sb = smem + ((c - c0) % kRouteStages) * kStage;
#pragma unroll
    for (int u = u0; u < 4; u += kUStep) {
      const int q = 2 * u + hl;
      const bf16x8 a = *(const bf16x8*)(sb + kXB + rswz(et * 32 + l32, q));
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj) {
        const bf16x8 b = *(const bf16x8*)(sb + rswz((j0 + jj) * 32 + l32, q));
        acc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[jj], 0, 0, 0);
      }
    }
  }
  __syncthreads();   // the ring is free: reuse it for the logit tile s_l[token][expert]
  float* s_l = (float*)smem;   // rows of kEP + 1 floats: the tile's lanes hit distinct banks
  // C[i][n] of a tile: i = expert (r/4)*8 + hl*4 + r%4, n = token l32
  auto put = [&](bool add) {
#pragma unroll
    for (int jj = 0; jj < kNJ; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = (j0 + jj) * 32 + l32, i = et * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
        float* d = s_l + n * (kEP + 1) + i;
        *d = add ? *d + acc[jj][r] : acc[jj][r];
      }
  };
  if (u0 == 0) put(false);
  __syncthreads();
  if (u0 != 0) put(true);   // the other half of the 16-deep slices, added second
  __syncthreads();
  for (int idx = threadIdx.x; idx < kBigTok * kEP; idx += 512) {
    const int n = idx / kEP, i = idx - n * kEP;
    const int64_t t = t0 + n;
    if (t < T && i < E) part[((int64_t)blockIdx.y * T + t) * E + i] = s_l[n * (kEP + 1) + i];
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
  token_keys(part, slices, T, tok, E, bias, lane, key, taken);
  select_topk(key, taken, lane, E, k, score, renorm, routed_scale, ids_out + tok * k, w_out + tok * k);
}

}  // namespace

// large batches take the LDS-staged router
bool route_big(int64_t T, int H) { return T >= 256 && H % 64 == 0; }

int route_slices(int64_t T, int H, int E) {
  if (route_big(T, H)) {
    const int tok = big_tok(E > 128 ? 256 : (E > 64 ? 128 : 64));
    const int64_t tiles = (T + tok - 1) / tok;
    const int nchunks = H / 64;
    int64_t sl = (256 + tiles - 1) / tiles;
    const int max_sl = nchunks / 4 > 0 ? nchunks / 4 : 1;   // at least 4 chunks per slice
    if (sl > max_sl) sl = max_sl;
    return (int)(sl < 1 ? 1 : sl);
  }
  const int64_t tiles = ((T + 31) / 32) * ((E + 31) / 32);
  // at least one 16-deep step per wave, and at most 8 slices: more would
  // shorten the logits launch less than they lengthen the top-k sums
  const int max_slices = (H / 16) / 4 < 8 ? (H / 16) / 4 : 8;
  int64_t sl = (512 + tiles - 1) / tiles;
  if (sl > max_slices) sl = max_slices;
  return (int)(sl < 1 ? 1 : sl);
}

size_t route_workspace_bytes(int64_t T, int H, int E, int act_bf16) {
  if (!act_bf16 || T == 0) return 0;
  return (size_t)route_slices(T, H, E) * T * E * sizeof(float);
}

hipError_t launch_route_logits(const void* x, const void* w_router, int64_t T, int H, int E, float* part,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (route_big(T, H)) return hipErrorInvalidValue;
  const int slices = route_slices(T, H, E);
  const int nsteps = H / 16;
  const int per = (nsteps + slices - 1) / slices;
  dim3 grid((unsigned)((T + 31) / 32), (unsigned)((E + 31) / 32), (unsigned)slices);
  hipLaunchKernelGGL(logits_kernel, grid, dim3(256), 0, stream, (const uint16_t*)x, (const uint16_t*)w_router, T, H,
                     E, per, part);
  return hipGetLastError();
}

hipError_t launch_route_topk(const void* x, const void* w_router, const float* bias, int64_t T,
                             int H, int E, int k, int act_bf16, int score, int renorm,
                             float routed_scale, int32_t* ids, float* w, float* part, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (act_bf16 && route_big(T, H)) {
    const int slices = route_slices(T, H, E);
    const int nchunks = H / 64;
    const int per = (nchunks + slices - 1) / slices;
    const int ep = E > 128 ? 256 : (E > 64 ? 128 : 64);
    const int tok = big_tok(ep);
    dim3 grid((unsigned)((T + tok - 1) / tok), (unsigned)slices);
    const uint16_t* xb = (const uint16_t*)x;
    const uint16_t* wb = (const uint16_t*)w_router;
    if (ep == 64) hipLaunchKernelGGL(logits_lds_kernel<64>, grid, dim3(512), 0, stream, xb, wb, T, H, E, per, part);
    else if (ep == 128) hipLaunchKernelGGL(logits_lds_kernel<128>, grid, dim3(512), 0, stream, xb, wb, T, H, E, per, part);
    else hipLaunchKernelGGL(logits_lds_kernel<256>, grid, dim3(512), 0, stream, xb, wb, T, H, E, per, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, part, slices, T, E, bias,
                       k, score, renorm, routed_scale, ids, w);
    return hipGetLastError();
  }
  if (act_bf16) {
    hipError_t e = launch_route_logits(x, w_router, T, H, E, part, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, part,
                       route_slices(T, H, E), T, E, bias, k, score, renorm, routed_scale, ids, w);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((T + kTokPerBlock - 1) / kTokPerBlock));
  hipLaunchKernelGGL(route_topk_f32_kernel, grid, dim3(256), 0, stream, (const float*)x, (const float*)w_router,
                     bias, T, H, E, k, score, renorm, routed_scale, ids, w);
  return hipGetLastError();
}

}  // namespace moe
