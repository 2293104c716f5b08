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

// Wave reductions with DPP lane moves instead of LDS-routed shuffles: xor 1
// and xor 2 inside quads, mirrors inside half rows and rows (each lane then
// holds its row's result), the row broadcasts of lanes 15 and 31 (row 3 then
// holds the wave's), and a read of lane 63, so every lane gets the same value.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ void argmax_step(float& bk, int& bi) {
  const float ok = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(bk), __float_as_int(bk), kCtrl,
                                                              kRowMask, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(bi, bi, kCtrl, kRowMask, 0xf, false);
  if (better(ok, oi, bk, bi)) {
    bk = ok;
    bi = oi;
  }
}

// (key, index) of the wave's best lane: larger key, ties to the lower index
__device__ __forceinline__ void wave_argmax(float& bk, int& bi) {
  argmax_step<0xb1, 0xf>(bk, bi);    // quad_perm [1,0,3,2]
  argmax_step<0x4e, 0xf>(bk, bi);    // quad_perm [2,3,0,1]
  argmax_step<0x141, 0xf>(bk, bi);   // row_half_mirror
  argmax_step<0x140, 0xf>(bk, bi);   // row_mirror
  argmax_step<0x142, 0xa>(bk, bi);   // row_bcast:15 into rows 1 and 3
  argmax_step<0x143, 0xc>(bk, bi);   // row_bcast:31 into rows 2 and 3
  bk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bk), 63));
  bi = __builtin_amdgcn_readlane(bi, 63);
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float sum_step(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xf, false));
}

// sum over the wave (a fixed order: the same value in every lane)
__device__ __forceinline__ float wave_sum(float v) {
  v = sum_step<0xb1, 0xf>(v);
  v = sum_step<0x4e, 0xf>(v);
  v = sum_step<0x141, 0xf>(v);
  v = sum_step<0x140, 0xf>(v);
  v = sum_step<0x142, 0xa>(v);
  v = sum_step<0x143, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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
    wave_argmax(bk, bi);
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
    s = expf(my_key - kmax) / wave_sum(part);
  } else {
    s = 1.0f / (1.0f + expf(-my_key));
  }
  if (renorm) {
    s = s / wave_sum(lane < k ? s : 0.f);
  }
  if (lane < k) {
    ids_out[lane] = my_idx;
    w_out[lane] = s * routed_scale;
    if (ids_lds) ids_lds[lane] = my_idx;
  }
}

// Keys of token `tok` for a wave (lane l: experts l, l+64, l+128, l+192):
// the slices' partial logits part[slice][T][E] added in ascending slice
// order, plus the bias; experts past E are taken already and NaN keys rank
// as -inf.  The loads of 8 slices and the bias are issued together, without
// branches (indices clamped into range, the extra values then ignored), so
// that their latencies overlap.
__device__ __forceinline__ void token_keys(const float* __restrict__ part, int slices, int64_t T, int64_t tok, int E,
                                           const float* __restrict__ bias, int lane, float (&key)[4],
                                           bool (&taken)[4]) {
  float z[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
  if (bias != nullptr)
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = bias[min(lane + 64 * q, E - 1)];
  for (int sl0 = 0; sl0 < slices; sl0 += 8) {
    float v[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ec = min(lane + 64 * q, E - 1);
#pragma unroll
      for (int u = 0; u < 8; ++u) v[q][u] = part[((int64_t)min(sl0 + u, slices - 1) * T + tok) * E + ec];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (sl0 + u < slices) z[q] += v[q][u];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    taken[q] = !(e < E);
    key[q] = e < E ? nan_to_neg_inf(z[q] + b[q]) : -INFINITY;
  }
}

}  // namespace moe


