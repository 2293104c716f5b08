// Device-side helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

constexpr int kWave = 64;
constexpr int kNumXcd = 8;      // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 32;

// One unit of grouped-GEMM work: rows [row_begin, row_end) of the expert-sorted
// matrix, all owned by `expert`, times output-channel tile `ntile`.
struct WorkItem {
  int32_t row_begin;
  int32_t row_end;
  int32_t expert;
  int32_t ntile;
};

// Schedule header in the workspace, followed by WorkItem items[capacity].
struct Schedule {
  int32_t total;
  int32_t pad[3];
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// two fp32 -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, b2));
}

// silu(g) = g * sigmoid(g); v_rcp_f32 (1 ulp) instead of an IEEE division
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// gate activation of the gated MLP (moe_gate_act: 0 silu, 1 gelu, 2 relu);
// gelu is the exact form 0.5 g (1 + erf(g / sqrt 2)).
template <int kAct>
__device__ __forceinline__ float gate_act(float g) {
  if constexpr (kAct == 1) return 0.5f * g * (1.0f + erff(g * 0.70710678118654752f));
  else if constexpr (kAct == 2) return fmaxf(g, 0.0f);
  else return silu(g);
}
// the same with the activation chosen at run time (`act` is uniform)
__device__ __forceinline__ float gate_fn(float g, int act) {
  if (act == 1) return gate_act<1>(g);
  if (act == 2) return gate_act<2>(g);
  return gate_act<0>(g);
}
// Calls f(std::integral_constant<int, act>{}) for the uniform activation id,
// so that a loop of activations inside f is straight-line code.
template <class F>
__device__ __forceinline__ void with_gate_act(int act, F&& f) {
  if (act == 1) f(std::integral_constant<int, 1>{});
  else if (act == 2) f(std::integral_constant<int, 2>{});
  else f(std::integral_constant<int, 0>{});
}
// h = act(g) * u over the 16 values a lane holds of a 32 x 32 tile pair
template <int kAct>
__device__ __forceinline__ void gated16(const f32x16& g, const f32x16& u, float (&h)[16]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) h[r] = gate_act<kAct>(g[r]) * u[r];
}

// Router keys: a NaN key ranks as -inf, so it loses to every number and ties
// with -inf (lowest expert index first); every top-k round then takes a valid
// untaken expert.
__device__ __forceinline__ float nan_to_neg_inf(float v) { return v != v ? -INFINITY : v; }

// value of an E8M0 scale byte: 2^(b-127)
__device__ __forceinline__ float e8m0_to_f32(uint8_t b) { return __builtin_ldexpf(1.0f, (int)b - 127); }

// Packs two floats into OCP e4m3 codes (round to nearest even); inputs are
// within +-464 by construction, so no code overflows.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// XCD-aware work index of this workgroup.  Workgroups are dealt round-robin
// to the 8 XCDs; work items are dealt to XCDs in chunks of C consecutive
// items (consecutive items share an expert's weight tile or token rows, see
// build_schedule, so a chunk reuses them from one L2), and successive chunks
// go to successive XCDs so that a hot expert's items spread over all of them.
// Returns -1 for workgroups beyond the live work.  gridDim.x is a multiple of
// 8 * C covering every item index the schedule can hold.
constexpr int kXcdChunk = 8;
template <int C = kXcdChunk>
__device__ __forceinline__ int xcd_work_index(int total) {
  const int xcd = blockIdx.x % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int w = ((slot / C) * kNumXcd + xcd) * C + slot % C;
  return w < total ? w : -1;
}

}  // namespace moe
