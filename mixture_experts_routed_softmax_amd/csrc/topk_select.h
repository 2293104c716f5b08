// Top-k selection of one token by one wave, shared by the router's selection
// launch and the small-batch selection + permutation launch.
//
// "Experts backends", opening paragraph: for each token a router selects k
// experts and the expert outputs are aggregated with routing weights:
//   ids[t,:] = the k largest keys, descending, ties -> lowest expert index
//   score    = softmax over all E keys, or sigmoid(key)
//   w[t,i]   = score(ids[t,i]) [ / sum_i score ] * routed_scale
#pragma once
#include "common.h"

namespace moe {

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
                                            int renorm, float routed_scale, int32_t* ids_out, float* w_out,
                                            int* ids_lds = nullptr) {
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
    if (ids_lds) ids_lds[lane] = my_idx;
  }
}

// Keys of token `tok` for a wave (lane l: experts l, l+64, l+128, l+192):
// the slices' partial logits part[slice][T][E] added in ascending slice
// order (the loads of 8 slices are issued together so that their latencies
// overlap), plus the bias; experts past E are taken already and NaN keys
// rank as -inf.
__device__ __forceinline__ void token_keys(const float* __restrict__ part, int slices, int64_t T, int64_t tok, int E,
                                           const float* __restrict__ bias, int lane, float (&key)[4],
                                           bool (&taken)[4]) {
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
    key[q] = e < E ? nan_to_neg_inf(z[q] + (bias ? bias[e] : 0.f)) : -INFINITY;
  }
}

}  // namespace moe


