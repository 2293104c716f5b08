// Backward of the routed expert layer ("Experts backends", section "SonicMoE":
// training of gated-MLP experts).  With the top-k selection held fixed, for the
// output gradient dout and sorted row r = (token t, slot i) of expert e:
//
//   e_r   = W_down[e]^T dout_t                      (grouped GEMM, ragged rows)
//   dw    = e_r . a_r,  a_r = act(g_r) * u_r        (routing-weight gradient)
//   dg    = w e_r * u_r * act'(g_r),  du = w e_r * act(g_r)
//   dx_r  = W_gate[e]^T dg + W_up[e]^T du          (grouped GEMM, ragged rows)
//   dW_down[e] = sum_r (dout_t) (w a_r)^T           (grouped GEMM, ragged K)
//   dW_gate[e] = sum_r dg x_t^T, dW_up[e] = sum_r du x_t^T
//
// One GEMM kernel serves all of them: C[n][m] = sum_k A[m][k] B[n][k], stored
// as out[n][m].  The A operand is always MN-major in memory (a K index is a
// row, M is contiguous): the weights for the data gradients, the sorted
// activations for the weight gradients.  B is K-major (token rows, ragged N)
// or MN-major (ragged K).  Both travel global -> LDS with global_load_lds in
// their memory layout; an MN-major operand is turned into MFMA fragments by
// ds_read_b64_tr_b16, which hands each lane four K-consecutive values of one
// column: lane i of a 16-lane group receives element i % 4 of the 8-byte
// pieces addressed by lanes 4j + i / 4 (j = 0..3), so lanes that address four
// consecutive K rows at four consecutive 4-column pieces produce the
// transposed 4 x 16 block.  Two such reads form the 8 K values a lane of
// v_mfma_f32_32x32x16_bf16 needs.  The reads of a K half are one inline
// assembly block that ends with its own lgkmcnt wait (see frags_mn2).
//
// Tile 256 (M) x 256 (N), K step 32, 8 waves of 64 x 128 (2 x 4 MFMA tiles),
// 4 LDS stages of 32 KB (one workgroup per CU).  MN-major stages hold 32 K
// rows of 512 B with 16-byte chunk c of row r at c ^ 4 (r & 3): the 16 lanes
// of a transposed read touch 16 distinct chunks (all 64 banks).  K-major
// stages hold 256 rows of 64 B with chunk c at c ^ ((r >> 2) & 3).  Columns
// past M or N read zeros and are not stored; MFMA tiles without live rows or
// columns are skipped.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBwdThreads = 512;
constexpr int kTile = kBwdTile;                // M and N extent of a tile
constexpr int kOpBytes = kTile * 64;           // one operand per stage: 32 K x 256 bf16
constexpr int kStageB = 2 * kOpBytes;
constexpr int kStagesB = 4;
constexpr int kLoadsB = 4;                     // DMA instructions per thread per stage

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_void;

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void)lds_wave_base, 16, 0, 0);
}

template <int n>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// byte offset of element `col` of K row r in an MN-major stage (512-byte rows)
__device__ __forceinline__ int mn_off(int r, int col) {
  return r * 512 + ((((col >> 3) ^ ((r & 3) << 2))) << 4) + (col & 7) * 2;
}
// byte offset of 16-byte chunk c of row r in a K-major stage (64-byte rows)
__device__ __forceinline__ int km_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS address of a lane's part of the MFMA fragment of columns m0 .. m0+31,
// K half h (16 rows) of an MN-major stage; the fragment is two transposed
// reads, at this address and 2048 bytes on (K rows r and r+4, same swizzle).
__device__ __forceinline__ uint32_t mn_addr(const uint8_t* st, int h, int m0, int lane) {
  const int G = lane >> 4, s = lane & 15;
  const int col = m0 + (G & 1) * 16 + 4 * (s & 3);
  const int r = h * 16 + (G >> 1) * 8 + (s >> 2);
  return (uint32_t)(uintptr_t)(lds_void)(st + mn_off(r, col));
}

__device__ __forceinline__ bf16x8 join(v4s lo, v4s hi) {
  return __builtin_bit_cast(bf16x8, v8s{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
}

// The transposed reads are inline assembly (the ds_read_tr builtin makes the
// compiler wait for every LDS DMA in flight before each read), and each block
// waits for its own reads (lgkmcnt(0)) before it ends, so its outputs are
// complete when the compiler first sees them: no register of a read in
// flight is ever reused or copied.  The memory clobber keeps the block in
// program order with the barrier and the DMA builtins.
// Two fragments (addresses p0, p1).
__device__ __forceinline__ void frags_mn2(uint32_t p0, uint32_t p1, bf16x8& f0, bf16x8& f1) {
  v4s a, b, c, d;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %5\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
      : "v"(p0), "v"(p1)
      : "memory");
  f0 = join(a, b);
  f1 = join(c, d);
}

// Six fragments (addresses p[0..5]).
__device__ __forceinline__ void frags_mn6(const uint32_t (&p)[6], bf16x8 (&f)[6]) {
  v4s r[12];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %12\n\t"
      "ds_read_b64_tr_b16 %1, %12 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %13\n\t"
      "ds_read_b64_tr_b16 %3, %13 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %14\n\t"
      "ds_read_b64_tr_b16 %5, %14 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %15\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:2048\n\t"
      "ds_read_b64_tr_b16 %8, %16\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %10, %17\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5])
      : "memory");
#pragma unroll
  for (int i = 0; i < 6; ++i) f[i] = join(r[2 * i], r[2 * i + 1]);
}

// kRK: ragged K (weight gradients) or ragged rows (data gradients).  kRouter
// only separates the router's launches from the experts' in profiles.
template <int kRK, bool kRouter>
__global__ __launch_bounds__(kBwdThreads, 1) void gemm_bwd_kernel(BwdGemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStagesB * kStageB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int wm = wave & 3, wn = wave >> 2;     // wave tile: M 64 (2 MFMA tiles) x N 128 (4 tiles)

  // ---- work item
  int e, mt, nt = 0, rb = 0, re = 0;
  int64_t kbase = 0;
  int nK;
  const int MT = (a.M + kTile - 1) / kTile;
  if (kRK) {
    const int NT = (a.n_total + kTile - 1) / kTile;
    const int item = blockIdx.x;
    e = item / (MT * NT);
    const int rem = item - e * MT * NT;
    mt = rem / NT;
    nt = rem - mt * NT;
    if (a.offsets) {
      kbase = a.offsets[e];
      nK = a.offsets[e + 1] - a.offsets[e];
    } else if (a.k_chunk > 0) {   // group e = K rows [e k_chunk, (e+1) k_chunk) of K
      kbase = (int64_t)e * a.k_chunk;
      nK = a.K - (int)kbase < a.k_chunk ? a.K - (int)kbase : a.k_chunk;
    } else {
      nK = a.K;
    }
  } else {
    if (a.sched) {
      const int w = xcd_work_index(a.sched->total);
      if (w < 0) return;
      const WorkItem it = ((const WorkItem*)(a.sched + 1))[w];
      e = it.expert;
      mt = it.ntile;
      rb = it.row_begin;
      re = it.row_end;
    } else {
      const int tile = blockIdx.x / MT;
      mt = blockIdx.x - tile * MT;
      e = 0;
      rb = tile * kTile;
      if (rb >= a.n_total) return;
      re = rb + kTile < a.n_total ? rb + kTile : a.n_total;
    }
    nK = a.K;
  }
  const int KT = (nK + 31) / 32;

  // ---- loaders.  MN-major operand: instruction i of wave w fills K rows
  // (i*8 + w)*2 .. +2 of the stage; lane -> row lane/32, chunk slot lane%32
  // holding global chunk slot ^ 4 (row & 3).  Chunks past the operand's
  // extent (M, or n_total) read zeros.
  const int mn_r = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int mcol[2], ncol[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = (i * 8 + wave) * 2 + mn_r;
    const int c = (lane & 31) ^ ((rr & 3) << 2);
    mcol[i] = mt * kTile + c * 8;
    ncol[i] = nt * kTile + c * 8;
  }
  // K-major B (ragged N): instruction i of wave w fills rows (i*8 + w)*16 .. +16
  const uint16_t* brow[2] = {nullptr, nullptr};
  if (!kRK) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rr = (i * 8 + wave) * 16 + (lane >> 2);
      int r = rb + rr;
      r = r < re ? r : re - 1;
      const int64_t src = a.b_gather ? (int64_t)(a.b_gather[r] / a.b_div) : (int64_t)r;
      const int c = (lane & 3) ^ ((rr >> 2) & 3);
      brow[i] = a.b + src * a.ldb + c * 8;
    }
  }
  auto a_src = [&](int kr, int i) -> const uint16_t* {   // K row kr (item-relative) of A, this lane's chunk
    if (kr >= nK || mcol[i] >= a.M) return a.zeros;
    if (kRK) return a.a + (kbase + kr) * a.lda + mcol[i];
    if (kr >= a.a_krows) return a.zeros;
    if (kr < a.a_split) return a.a + (int64_t)e * a.a_gs + (int64_t)kr * a.lda + mcol[i];
    return a.a2 + (int64_t)e * a.a_gs + (int64_t)(kr - a.a_split) * a.lda + mcol[i];
  };
  auto issue = [&](int stage, int kt) {
    uint8_t* st = smem + stage * kStageB;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kr = kt * 32 + (i * 8 + wv) * 2 + mn_r;
      dma16(a_src(kr, i), st + (i * 8 + wv) * 1024);
    }
    if (kRK) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int kr = kt * 32 + (i * 8 + wv) * 2 + mn_r;
        const uint16_t* src = kr < nK && ncol[i] < a.n_total ? a.b + (kbase + kr) * a.ldb + ncol[i] : a.zeros;
        dma16(src, st + kOpBytes + (i * 8 + wv) * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(brow[i] + kt * 32, st + kOpBytes + (i * 8 + wv) * 1024);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  // live MFMA tiles of this wave: M columns inside M, N rows inside the item
  const int nvalid = kRK ? a.n_total - nt * kTile : re - rb;
  int my_nt = (nvalid - wn * 128 + 31) / 32;
  my_nt = my_nt < 0 ? 0 : (my_nt > 4 ? 4 : my_nt);
  int my_mt = (a.M - mt * kTile - wm * 64 + 31) / 32;
  my_mt = my_mt < 0 ? 0 : (my_mt > 2 ? 2 : my_mt);

#pragma unroll
  for (int p = 0; p < kStagesB - 1; ++p)
    if (p < KT) issue(p, p);
  for (int s = 0; s < KT; ++s) {
    const int ahead = KT - 1 - s;   // steps issued after step s
    if (ahead >= 2) wait_vm<2 * kLoadsB>();
    else if (ahead == 1) wait_vm<kLoadsB>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (s + kStagesB - 1 < KT) issue((s + kStagesB - 1) % kStagesB, s + kStagesB - 1);
    const uint8_t* st = smem + (s % kStagesB) * kStageB;
    if (my_mt > 0 && my_nt > 0) {
      // per K half: the fragments (read and waited for), then their MFMAs;
      // the other wave of the SIMD keeps the matrix pipe busy meanwhile
      bf16x8 fa[2][2], fb[2][4];
      auto read_half = [&](int h) {
        if constexpr (kRK) {
          const uint32_t p[6] = {mn_addr(st, h, wm * 64, lane), mn_addr(st, h, wm * 64 + 32, lane),
                                 mn_addr(st + kOpBytes, h, wn * 128, lane),
                                 mn_addr(st + kOpBytes, h, wn * 128 + 32, lane),
                                 mn_addr(st + kOpBytes, h, wn * 128 + 64, lane),
                                 mn_addr(st + kOpBytes, h, wn * 128 + 96, lane)};
          bf16x8 f[6];
          frags_mn6(p, f);
          fa[h][0] = f[0];
          fa[h][1] = f[1];
#pragma unroll
          for (int j = 0; j < 4; ++j) fb[h][j] = f[2 + j];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            fb[h][j] = *(const bf16x8*)(st + kOpBytes + km_off(wn * 128 + j * 32 + l32, h * 2 + hl));
          frags_mn2(mn_addr(st, h, wm * 64, lane), mn_addr(st, h, wm * 64 + 32, lane), fa[h][0], fa[h][1]);
        }
      };
      auto mfma_half = [&](int h) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            if (j < my_nt && t < my_mt) acc[t][j] = mfma_bf16(fa[h][t], fb[h][j], acc[t][j]);
      };
      read_half(0);
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(0);
      __builtin_amdgcn_sched_barrier(0);
      read_half(1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(1);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue: lane holds C[m][n] for n = l32 of each B tile and
  // m = (r/4)*8 + hl*4 + r%4 of each A tile; out[n][m].
  if (kRK && !a.out_f32) {
    // bf16 weight gradients go through LDS (the ring is free now): each wave
    // writes its values in out[n][m] order, 16-byte chunk c of tile row r at
    // chunk c ^ (r & 31), then the workgroup stores whole rows, 16 contiguous
    // bytes per lane, instead of 8-byte pieces of 32 rows per store.
    static_assert(kTile * kTile * 2 <= kStagesB * kStageB, "the bf16 tile fits the ring");
    __syncthreads();   // every wave is done with the ring
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const int r = wn * 128 + tj * 32 + l32;
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ml = wm * 64 + ti * 32 + q * 8 + hl * 4;
          const f32x16& c = acc[ti][tj];
          *(i32x2*)(smem + r * (kTile * 2) + (((ml >> 3) ^ (r & 31)) << 4) + ((ml >> 2) & 1) * 8) =
              i32x2{(int)pack_bf16x2(c[q * 4 + 0], c[q * 4 + 1]), (int)pack_bf16x2(c[q * 4 + 2], c[q * 4 + 3])};
        }
    }
    __syncthreads();
    for (int idx = tid; idx < kTile * (kTile / 8); idx += kBwdThreads) {
      const int r = idx / (kTile / 8), c = idx % (kTile / 8);
      const int n = nt * kTile + r, m = mt * kTile + c * 8;
      if (n >= a.n_valid || m >= a.M) continue;
      const bool second = a.out2 && n >= a.n_split;
      const int nn = second ? n - a.n_split : n;
      uint8_t* base = (uint8_t*)(second ? a.out2 : a.out);
      *(i32x4*)(base + ((int64_t)e * a.o_gs + (int64_t)nn * a.ldo + m) * 2) =
          *(const i32x4*)(smem + r * (kTile * 2) + ((c ^ (r & 31)) << 4));
    }
    return;
  }
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) {
    const int rr = wn * 128 + tj * 32 + l32;
    uint8_t* orow;
    if (kRK) {
      const int n = nt * kTile + rr;
      if (n >= a.n_valid) continue;
      const bool second = a.out2 && n >= a.n_split;
      const int nn = second ? n - a.n_split : n;
      uint8_t* base = (uint8_t*)(second ? a.out2 : a.out);
      orow = base + ((int64_t)e * a.o_gs + (int64_t)nn * a.ldo) * (a.out_f32 ? 4 : 2);
    } else {
      if (rr >= nvalid) continue;
      orow = (uint8_t*)a.out + (int64_t)(rb + rr) * a.ldo * (a.out_f32 ? 4 : 2);
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = mt * kTile + wm * 64 + ti * 32 + q * 8 + hl * 4;
        if (m >= a.M) continue;
        const f32x16& c = acc[ti][tj];
        if (a.out_f32) {
          *(f32x4*)(orow + (int64_t)m * 4) = f32x4{c[q * 4 + 0], c[q * 4 + 1], c[q * 4 + 2], c[q * 4 + 3]};
        } else {
          *(i32x2*)(orow + (int64_t)m * 2) =
              i32x2{(int)pack_bf16x2(c[q * 4 + 0], c[q * 4 + 1]), (int)pack_bf16x2(c[q * 4 + 2], c[q * 4 + 3])};
        }
      }
  }
}

// derivative of the gate activation (moe_gate_act: 0 silu, 1 exact gelu, 2 relu)
__device__ __forceinline__ float gate_deriv(float g, int act) {
  if (act == 1) {
    const float Phi = 0.5f * (1.0f + erff(g * 0.70710678118654752f));
    const float phi = 0.39894228040143268f * __expf(-0.5f * g * g);
    return Phi + g * phi;
  }
  if (act == 2) return g > 0.0f ? 1.0f : 0.0f;
  const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
  return sg * (1.0f + g * (1.0f - sg));
}

// One workgroup per sorted row r (pair p = perm[r]):
//   dw[p] = sum_j e_j a_j  (a = act(g) u, in channel order per thread, then a
//   fixed-order workgroup sum), ap = w a, dgu = [w e u act'(g) | w e act(g)]
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ ev, const float* __restrict__ gu,
                                                         const int32_t* __restrict__ perm, const float* __restrict__ w,
                                                         int I, int act, float* __restrict__ dw,
                                                         uint16_t* __restrict__ ap, uint16_t* __restrict__ dgu) {
  __shared__ float s_red[4];
  const int64_t r = blockIdx.x;
  const int p = perm[r];
  const float wp = w[p];
  const float* er = ev + r * I;
  const float* gr = gu + r * 2 * I;
  float part = 0.f;
  for (int j = threadIdx.x * 4; j < I; j += 256 * 4) {
    const f32x4 e4 = *(const f32x4*)(er + j);
    const f32x4 g4 = *(const f32x4*)(gr + j);
    const f32x4 u4 = *(const f32x4*)(gr + I + j);
    float a4[4], dg4[4], du4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float g = g4[c], u = u4[c];
      const float fg = gate_fn(g, act);
      a4[c] = fg * u;
      part = __builtin_fmaf(e4[c], a4[c], part);
      const float we = wp * e4[c];
      dg4[c] = we * u * gate_deriv(g, act);
      du4[c] = we * fg;
    }
    *(i32x2*)(ap + r * I + j) = i32x2{(int)pack_bf16x2(wp * a4[0], wp * a4[1]), (int)pack_bf16x2(wp * a4[2], wp * a4[3])};
    *(i32x2*)(dgu + r * 2 * I + j) = i32x2{(int)pack_bf16x2(dg4[0], dg4[1]), (int)pack_bf16x2(dg4[2], dg4[3])};
    *(i32x2*)(dgu + r * 2 * I + I + j) = i32x2{(int)pack_bf16x2(du4[0], du4[1]), (int)pack_bf16x2(du4[2], du4[3])};
  }
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = part;
  __syncthreads();
  if (threadIdx.x == 0) dw[p] = ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
}

// One wave per token: router keys from the partial logits (slices added in
// order, as the forward's selection does), scores, and the key gradient
//   ds_i  = c (dw_i / S - sum_j dw_j s_j / S^2)  (renormalised) or c dw_i
//   dkey  = s (ds - sum s ds)  (softmax over all E)  or  ds s (1 - s)  (sigmoid)
// written as fp32 [T,E] and as bf16 [T,Epad] (zero past E).
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ part, int slices, int64_t T, int E,
                                                         int Epad, const float* __restrict__ bias,
                                                         const int32_t* __restrict__ ids, const float* __restrict__ dw,
                                                         int k, int score, int renorm, float routed_scale,
                                                         float* __restrict__ dkey, uint16_t* __restrict__ dkey_b) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float key[4], s[4], ds[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    float z = 0.f;
    if (e < E)
      for (int sl = 0; sl < slices; ++sl) z += part[((int64_t)sl * T + t) * E + e];
    key[q] = e < E ? nan_to_neg_inf(z + (bias ? bias[e] : 0.f)) : -INFINITY;
    ds[q] = 0.f;
  }
  if (score == 0) {
    float m = fmaxf(fmaxf(key[0], key[1]), fmaxf(key[2], key[3]));
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float den = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s[q] = lane + 64 * q < E ? __expf(key[q] - m) : 0.f;
      den += s[q];
    }
    for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] = s[q] / den;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] = lane + 64 * q < E ? 1.0f / (1.0f + __expf(-key[q])) : 0.f;
  }
  // selected scores: S and sum dw s (every lane computes them, in slot order)
  float S = 0.f, dws = 0.f;
  for (int i = 0; i < k; ++i) {
    const int e = ids[t * k + i];
    const int q = e >> 6;
    const float sq = q == 0 ? s[0] : (q == 1 ? s[1] : (q == 2 ? s[2] : s[3]));
    const float se = __shfl(sq, e & 63);
    S += se;
    dws += dw[t * k + i] * se;
  }
  for (int i = 0; i < k; ++i) {
    const int e = ids[t * k + i];
    if ((e & 63) == lane) {
      const float d = renorm ? routed_scale * (dw[t * k + i] / S - dws / (S * S)) : routed_scale * dw[t * k + i];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if ((e >> 6) == q) ds[q] = d;
    }
  }
  float dk[4];
  if (score == 0) {
    float sds = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) sds += s[q] * ds[q];
    for (int off = 32; off > 0; off >>= 1) sds += __shfl_xor(sds, off);
#pragma unroll
    for (int q = 0; q < 4; ++q) dk[q] = s[q] * (ds[q] - sds);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) dk[q] = ds[q] * s[q] * (1.0f - s[q]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    if (e < E) dkey[t * E + e] = dk[q];
    if (e < Epad) dkey_b[t * Epad + e] = f32_to_bf16_bits(e < E ? dk[q] : 0.f);
  }
}

// dbias[e] = sum_t dkey[t, e]: one workgroup per expert, per-thread sums in
// token order, then a fixed-order workgroup sum
__global__ __launch_bounds__(256) void bias_grad_kernel(const float* __restrict__ dkey, int64_t T, int E,
                                                        float* __restrict__ dbias) {
  __shared__ float s_red[4];
  const int e = blockIdx.x;
  float v = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += 256) v += dkey[t * E + e];
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) dbias[e] = ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
}

// dx[t] = sum_i dxp[inv[t*k+i]] + dxr[t] (slot order, fp32), rounded to bf16.
// The token's rows are read from inv once into LDS, then the loads of up to 8
// slots are issued together (streaming: every row is read once): qwen-like
// backward 48 -> 31 us
__global__ __launch_bounds__(256) void dx_combine_kernel(const float* __restrict__ dxp, const float* __restrict__ dxr,
                                                         const int32_t* __restrict__ inv, int k, int H,
                                                         uint16_t* __restrict__ dx) {
  __shared__ int s_row[kMaxTopK];
  const int64_t t = blockIdx.x;
  const int64_t P = (int64_t)gridDim.x * k;
  if ((int)threadIdx.x < k) {
    const int64_t row = inv[t * k + threadIdx.x];
    s_row[threadIdx.x] = row >= 0 && row < P ? (int)row : -1;   // a pair without a row contributes nothing
  }
  __syncthreads();
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  f32x4 acc = __builtin_nontemporal_load((const f32x4*)(dxr + t * H + c));
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < k; i0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i0 + u < k && s_row[i0 + u] >= 0)
        v[u] = __builtin_nontemporal_load((const f32x4*)(dxp + (int64_t)s_row[i0 + u] * H + c));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (i0 + u >= k) break;
      if (s_row[i0 + u] < 0) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) sum[q] += v[u][q];
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = sum[q] + acc[q];
  *(i32x2*)(dx + t * H + c) = i32x2{(int)pack_bf16x2(acc[0], acc[1]), (int)pack_bf16x2(acc[2], acc[3])};
}

// out[i] = bf16(sum_c part[c][i]) over the K chunks in order
__global__ __launch_bounds__(256) void chunk_sum_kernel(const float* __restrict__ part, int chunks, int64_t n,
                                                       uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 acc = *(const f32x4*)(part + i);
  for (int c = 1; c < chunks; ++c) {
    const f32x4 v = *(const f32x4*)(part + (int64_t)c * n + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += v[q];
  }
  *(i32x2*)(out + i) = i32x2{(int)pack_bf16x2(acc[0], acc[1]), (int)pack_bf16x2(acc[2], acc[3])};
}

__global__ void fill_zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

hipError_t launch_gemm_bwd(const BwdGemmArgs& a, int ragged_k, int router, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  dim3 g(grid), b(kBwdThreads);
  if (ragged_k && router) hipLaunchKernelGGL((gemm_bwd_kernel<1, true>), g, b, 0, stream, a);
  else if (ragged_k) hipLaunchKernelGGL((gemm_bwd_kernel<1, false>), g, b, 0, stream, a);
  else if (router) hipLaunchKernelGGL((gemm_bwd_kernel<0, true>), g, b, 0, stream, a);
  else hipLaunchKernelGGL((gemm_bwd_kernel<0, false>), g, b, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* ev, const float* gu, const int32_t* perm, const float* w, int64_t P,
                             int I, int act, float* dw, uint16_t* ap, uint16_t* dgu, hipStream_t stream) {
  if (P == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)P), dim3(256), 0, stream, ev, gu, perm, w, I, act, dw, ap, dgu);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* part, int slices, int64_t T, int E, int Epad, const float* bias,
                             const int32_t* ids, const float* dw, int k, int score, int renorm, float routed_scale,
                             float* dkey, uint16_t* dkey_b, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(router_bwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, part, slices, T, E, Epad,
                     bias, ids, dw, k, score, renorm, routed_scale, dkey, dkey_b);
  return hipGetLastError();
}

hipError_t launch_bias_grad(const float* dkey, int64_t T, int E, float* dbias, hipStream_t stream) {
  hipLaunchKernelGGL(bias_grad_kernel, dim3((unsigned)E), dim3(256), 0, stream, dkey, T, E, dbias);
  return hipGetLastError();
}

hipError_t launch_dx_combine(const float* dxp, const float* dxr, const int32_t* inv, int64_t T, int k, int H,
                             uint16_t* dx, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(dx_combine_kernel, dim3((unsigned)T, (unsigned)((H / 4 + 255) / 256)), dim3(256), 0, stream, dxp,
                     dxr, inv, k, H, dx);
  return hipGetLastError();
}

hipError_t launch_chunk_sum(const float* part, int chunks, int64_t n, uint16_t* out, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(chunk_sum_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, stream, part, chunks, n,
                     out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t stream) {
  const int64_t n = bytes / 4;
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t*)p, n);
  return hipGetLastError();
}

}  // namespace moe
