// Grouped gate/up and down GEMMs of FP8 expert MLPs on tile-packed e4m3
// weights with 128 x 128 block scales, one wave per SIMD.
//
// "Experts backends", section "FP8 and FP4 quantized experts": the experts'
// weights are e4m3 with one scale per 128 x 128 block (float32 or UE8M0) and
// the activations are quantized per row and 128 channels; each expert is a
// gated MLP run as one grouped GEMM over the expert-sorted token rows (backend
// table, rows grouped_mm / deepgemm):
//
//   gate/up : h[r, j] = act(x_r . w_gate[e, j]) * (x_r . w_up[e, j]),
//             then h quantized per row over the tile's 128 channels
//   down    : y[r, o] = h_r . w_down[e, o]
//
// with x . w = sum over 128-deep blocks kb of s_x(r, kb) s_w(kb) (q_x . q_w).
//
// Tile = 256 weight rows x 128 token rows.  4 waves, one per SIMD; wave w owns
// 64 weight rows (gate/up: gate rows and up rows of the same 32 channels, so
// the gated activation and h's quantization happen in registers) for all 128
// tokens, as 2 x 4 tiles of v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales).
// A 128-deep scale block is two MFMAs deep: each tile's two MFMAs add into a
// partial tile, which is folded into the fp32 accumulators with
// s_w(block) s_x(row, block) (the promotion), tile by tile in a pipeline, so
// that the vector unit's promotions run beside the matrix core's MFMAs.
//
// Weight rows are private to a wave and go from the packed chunks straight
// into registers in MFMA operand order, two blocks ahead.  Token rows are
// shared by the four waves: they are gathered through the expert permutation
// into an LDS ring by buffer_load ... lds (the DMA path), 128 bytes (one
// cache line, one scale block) per row and block.  One barrier per block.
// The scales of the whole K range (the tile's rows' activation scales and
// the weight blocks' scales) are staged in LDS once per tile.
//
// FP4 experts (same section: e2m1 weights, two per byte, one UE8M0 scale per
// row and 32 consecutive K) run on the same kernel (kFp4): a 128-deep block is
// then 64 packed bytes per weight row, one 16 KB chunk, and the MFMA takes
// the e2m1 weights as its A operand (a lane half holds 32 consecutive K, the
// matching e4m3 token bytes are the same pieces as for fp8 weights) with the
// lane's weight scale byte as its scale operand, so the promotion multiplies
// by s_x(row, block) alone.  The scale dword of a weight row (the block's four
// 32-K scales) rides with the block's weight loads.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kThreads = 256;            // 4 waves, one per SIMD
constexpr int kTok = 128;                // token rows per tile
constexpr int kBlkB = 128;               // bytes of a token row per K block (128 e4m3: one scale block)
constexpr int kStage = kTok * kBlkB;     // 16 KB of tokens per LDS stage
constexpr int kStages = 6;               // LDS stages of tokens (96 KB)
constexpr int kTokAhead = kStages - 1;   // blocks the token DMA runs ahead
constexpr int kWSlots = 3;               // register slots of weights (blocks)
constexpr int kWAhead = kWSlots - 1;     // blocks the weight loads run ahead
constexpr int kChunk = 256 * 64;         // packed weight chunk: 256 rows x 64 bytes (64 K)
// weight loads per wave and block: fp8 8 x 16 bytes; fp4 4 x 16 bytes and
// the two weight tiles' scale dwords
template <bool kFp4>
constexpr int kWLoads = kFp4 ? 6 : 8;
constexpr int kMaxKB = kStreamMaxScaleBlocks;   // K / 128 at most (K <= 8192)
static_assert(kThreads == 2 * kTok, "two threads stage each token row's scales");
// word 3 of a gfx9 buffer resource: 32-bit data format, raw (untyped) access
constexpr int kBufferConfig = 0x00020000;

typedef __attribute__((address_space(3))) void* lds_ptr;

// token row r's 16-byte chunk c (of 8) sits at position c ^ ((r >> 1) & 7)
__device__ __forceinline__ int tswz(int r, int c) { return r * kBlkB + ((c ^ ((r >> 1) & 7)) << 4); }
// packed weights: row r's 16-byte piece c (of 4) of a 64-byte K step at c ^ ((r >> 2) & 3)
__device__ __forceinline__ int wswz(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

__device__ __forceinline__ float wscale(const void* s, int ue8m0, int64_t idx) {
  return ue8m0 ? e8m0_to_f32(((const uint8_t*)s)[idx]) : ((const float*)s)[idx];
}

template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(n) for a wave-uniform n known only at run time
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n < 0 ? 0 : (n > 63 ? 63 : n)) {
#define MOE_W(i) case i: wait_vmcnt<i>(); break;
    MOE_W(0) MOE_W(1) MOE_W(2) MOE_W(3) MOE_W(4) MOE_W(5) MOE_W(6) MOE_W(7) MOE_W(8) MOE_W(9) MOE_W(10)
    MOE_W(11) MOE_W(12) MOE_W(13) MOE_W(14) MOE_W(15) MOE_W(16) MOE_W(17) MOE_W(18) MOE_W(19) MOE_W(20)
    MOE_W(21) MOE_W(22) MOE_W(23) MOE_W(24) MOE_W(25) MOE_W(26) MOE_W(27) MOE_W(28) MOE_W(29) MOE_W(30)
    MOE_W(31) MOE_W(32) MOE_W(33) MOE_W(34) MOE_W(35) MOE_W(36) MOE_W(37) MOE_W(38) MOE_W(39) MOE_W(40)
    MOE_W(41) MOE_W(42) MOE_W(43) MOE_W(44) MOE_W(45) MOE_W(46) MOE_W(47) MOE_W(48) MOE_W(49) MOE_W(50)
    MOE_W(51) MOE_W(52) MOE_W(53) MOE_W(54) MOE_W(55) MOE_W(56) MOE_W(57) MOE_W(58) MOE_W(59) MOE_W(60)
    MOE_W(61) MOE_W(62) MOE_W(63)
#undef MOE_W
  }
}

// weights of one block for one wave: [weight tile][64-deep half][16-byte
// piece] (fp4: one piece per half, and the tiles' scale dwords)
template <bool kFp4>
struct WBlk {
  i32x4 a[2][2][kFp4 ? 1 : 2];
  uint32_t s[kFp4 ? 2 : 1];
};

__device__ __forceinline__ i32x8 join8(const i32x4& lo, const i32x4& hi) {
  return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

template <int kMode, bool kFp4>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_grouped_fp8_kernel(
    GemmArgs a) {
  constexpr int kWL = kWLoads<kFp4>;
  constexpr int kBlkW = kFp4 ? kChunk : 2 * kChunk;   // packed weight bytes of a 128-deep block
  // one LDS object: the token ring, then the activation scales of the tile's
  // rows [kb][row], the weight block scales (gate/up: gate, up; down: row
  // halves) and the gate/up epilogue's per-wave row maxima of |h|
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage + (kMaxKB * kTok + 2 * kMaxKB + 4 * kTok) * 4];
  float* s_sx = (float*)(smem + kStages * kStage);
  float (*s_sw)[kMaxKB] = (float (*)[kMaxKB])(s_sx + kMaxKB * kTok);
  float (*s_amax)[kTok] = (float (*)[kTok])(s_sx + kMaxKB * kTok + 2 * kMaxKB);
  const int w = xcd_work_index<kGroupedXcdChunk>(a.sched->total);
  if (w < 0) return;
  const WorkItem it = ((const WorkItem*)(a.sched + 1))[w];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int K = a.K, N = a.N;
  const int KB = K / 128;                  // scale blocks = K blocks of the pipeline
  const int valid = it.row_end - it.row_begin;
  const int ntok = (valid + 31) >> 5;      // live 32-token tiles, 1..4
  const int e = it.expert;

  // ---- weights: a buffer resource over the tile's packed chunks; the lane's
  // pieces at fixed offsets, the K step as scalar offset
  const uint8_t* wbase = (const uint8_t*)a.w0 + ((int64_t)e * a.wtiles + it.ntile) * KB * (int64_t)kBlkW;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)wbase, 0, KB * kBlkW, kBufferConfig);
  int arow[2];
  if (kMode == 0) {
    arow[0] = wave * 32 + l32;          // gate rows of channels wave*32 .. +31
    arow[1] = 128 + wave * 32 + l32;    // up rows of the same channels
  } else {
    arow[0] = wave * 64 + l32;
    arow[1] = wave * 64 + 32 + l32;
  }
  // An e4m3 operand of lane half hl holds 32 of the MFMA's 64 K.  Which 32 is
  // free as long as the weights and the tokens agree (the MFMA sums over all
  // 64): lane half hl takes the 16-byte pieces hl and hl + 2 of a 64-byte K
  // step, so that the two lane halves' token reads hit different LDS banks.
  // (fp4: the e2m1 operand of lane half hl in 64-deep half q is the 16-byte
  // piece 2q + hl, i.e. 32 consecutive K, of the block's 64-byte row; paired
  // with the same token pieces as for fp8 weights, as the MFMA lays the two
  // formats out)
  int aoff[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int q = 0; q < 2; ++q) aoff[t][q] = wswz(arow[t], 2 * q + hl);
  // fp4 weight scales: K / 32 UE8M0 bytes per weight row (gate/up: gate rows
  // in s0, up rows in s1), the block's four in one dword; rows past N take
  // the last row's scales (their packed weights are zero)
  __amdgpu_buffer_rsrc_t sres[2];
  int soff[2];
  if constexpr (kFp4) {
    const int KS = K / 32;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      int ch = kMode == 0 ? it.ntile * 128 + (arow[t] & 127) : it.ntile * 256 + arow[t];
      ch = ch < N ? ch : N - 1;
      const uint8_t* sb = (const uint8_t*)(kMode == 0 && t == 1 ? a.s1 : a.s0) + (int64_t)e * N * KS;
      sres[t] = __builtin_amdgcn_make_buffer_rsrc((void*)sb, 0, N * KS, kBufferConfig);
      soff[t] = ch * KS;
    }
  }
  auto load_w = [&](WBlk<kFp4>& wb, int kb) {
    if constexpr (kFp4) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          wb.a[t][h][0] =
              __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, aoff[t][h], kb * kBlkW, 0));
#pragma unroll
      for (int t = 0; t < 2; ++t) wb.s[t] = __builtin_amdgcn_raw_buffer_load_b32(sres[t], soff[t], kb * 4, 0);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int q = 0; q < 2; ++q)
            wb.a[t][h][q] = __builtin_bit_cast(
                i32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, aoff[t][q], (2 * kb + h) * kChunk, 0));
    }
  };
  // one MFMA of weight tile t, 64-deep half h (unit scales for fp8; fp4: the
  // lane's 32-K weight scale byte 2h + hl of the tile row's dword)
  auto mfma = [&](const WBlk<kFp4>& wb, int t, int h, const i32x8& b, const f32x16& c) {
    if constexpr (kFp4) {
      const i32x4 v = wb.a[t][h][0];
      const int sc = (int)__builtin_amdgcn_ubfe(wb.s[t], 16 * h + 8 * hl, 8);
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0}, b, c, 4, 0,
                                                             0, sc, 0, 127);
    } else {
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(join8(wb.a[t][h][0], wb.a[t][h][1]), b, c, 0, 0, 0,
                                                             127, 0, 127);
    }
  };

  // ---- tokens: DMA instruction i of wave w fills LDS rows 32i + 8w .. +8 of
  // the stage (token tile i); lane l writes position l & 7 of row 32i + 8w + l/8
  const __amdgpu_buffer_rsrc_t tres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.act), 0, (int)(uint32_t)(a.act_rows * (int64_t)K), kBufferConfig);
  int toff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * i + 8 * wave + (lane >> 3);
    int r = it.row_begin + row;
    r = r < it.row_end ? r : it.row_end - 1;
    const uint32_t src_row = a.gather ? (uint32_t)(a.gather[r] / a.gather_div) : (uint32_t)r;
    const uint32_t c = (uint32_t)((lane & 7) ^ ((row >> 1) & 7));
    toff[i] = (int)(src_row * (uint32_t)K + c * 16);
  }

  // ---- scales of the whole K range into LDS: the activation scales of the
  // tile's rows as s_sx[kb][row] (two threads per row, every load issued
  // before the first store) and the fp8 weight blocks' scales
  {
    const int row = tid >> 1, half = tid & 1;
    int r = it.row_begin + row;
    r = r < it.row_end ? r : it.row_end - 1;
    const int64_t src = a.gather ? (int64_t)(a.gather[r] / a.gather_div) : (int64_t)r;
    const float* sp = a.act_scales + src * KB;
    float v[kMaxKB / 2];
#pragma unroll
    for (int u = 0; u < kMaxKB / 2; ++u) {
      const int kb = half + 2 * u;
      v[u] = sp[kb < KB ? kb : KB - 1];
    }
#pragma unroll
    for (int u = 0; u < kMaxKB / 2; ++u) {
      const int kb = half + 2 * u;
      if (kb < KB) s_sx[kb * kTok + row] = v[u];
    }
    const int NBr = (N + 127) / 128;
    for (int i = tid; i < (kFp4 ? 0 : 2 * KB); i += kThreads) {
      const int h = i / KB, kb = i - h * KB;
      if (kMode == 0) {
        s_sw[h][kb] = wscale(h == 0 ? a.s0 : a.s1, a.scale_ue8m0, ((int64_t)e * NBr + it.ntile) * KB + kb);
      } else {
        int br = it.ntile * 2 + h;
        br = br < NBr ? br : NBr - 1;
        s_sw[h][kb] = wscale(a.s0, a.scale_ue8m0, ((int64_t)e * NBr + br) * KB + kb);
      }
    }
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = f32x16{};

  auto mainloop = [&](auto nt_const) {
    constexpr int NT = decltype(nt_const)::value;
    // tokens of block kb into LDS stage `stage`
    auto issue_t = [&](int stage, int kb) {
      uint8_t* sb = smem + stage * kStage + wave * 1024;
#pragma unroll
      for (int i = 0; i < NT; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(tres, (lds_ptr)(sb + i * 4096), 16, toff[i], kb * kBlkB, 0, 0);
    };
    // memory instructions issued after the token DMA of block j once the tops
    // up to `upto` issued (tops: t < 0 the prologue; top t issues the tokens
    // of block t + kTokAhead, then the weights of block t + kWAhead)
    auto ops_after = [&](int j, int upto) {
      const int t0 = j - kTokAhead;
      int n = (t0 + kWAhead >= 0 && t0 + kWAhead < KB) ? kWL : 0;
      for (int t = t0 + 1; t <= upto; ++t) {
        if (t + kTokAhead >= 0 && t + kTokAhead < KB) n += NT;
        if (t + kWAhead >= 0 && t + kWAhead < KB) n += kWL;
      }
      return n;
    };
    WBlk<kFp4> ring[kWSlots];
    // prologue: the tops t < 0
#pragma unroll
    for (int t = -kTokAhead; t < 0; ++t) {
      if (t + kTokAhead < KB) issue_t(t + kTokAhead, t + kTokAhead);
      if (t + kWAhead >= 0 && t + kWAhead < KB) load_w(ring[(t + kWAhead + kWSlots) % kWSlots], t + kWAhead);
    }
    // token fragments of tile j, half h of the block in stage `stage`: row
    // j*32 + l32, pieces 4h + hl and 4h + 2 + hl.  (Typed 16-byte loads, as
    // in the bf16 kernel: the compiler then leaves their ordering against the
    // token DMA to the explicit waits and barriers instead of waiting for
    // every DMA in flight.)
    auto frag = [&](int stage, int j, int h) {
      const uint8_t* sb = smem + stage * kStage;
      const bf16x8 lo = *(const bf16x8*)(sb + tswz(j * 32 + l32, 4 * h + hl));
      const bf16x8 hi = *(const bf16x8*)(sb + tswz(j * 32 + l32, 4 * h + 2 + hl));
      return join8(__builtin_bit_cast(i32x4, lo), __builtin_bit_cast(i32x4, hi));
    };
    // token fragments of two blocks: [parity][half][token tile]
    i32x8 fb[2][2][NT];
    // One block kb.  At its top this wave's DMA of block kb+1 has landed; the
    // barrier then certifies every wave's, and that the stage of block kb-1
    // (read during block kb-2) is free for the DMA of block kb + kTokAhead.
    // The fragments of block kb were read during block kb-1; those of block
    // kb+1 are read in the middle of this block's pipeline.  In the steady
    // state (every earlier top issued in full, kb + kTokAhead < KB) the wait
    // is a compile-time count and the loads are issued without conditions,
    // so that the compiler's own waits for the weight registers stay exact.
    constexpr int kSteadyWait = kWL + (kTokAhead - 2) * (NT + kWL);
    static_assert(kSteadyWait < 64, "vmcnt range");
    auto block = [&](int kb, auto d_const, auto p_const, auto steady_const) {
      constexpr int d = decltype(d_const)::value;
      constexpr int p = decltype(p_const)::value;
      constexpr bool kSteady = decltype(steady_const)::value;
      constexpr int df = (d + kWAhead) % kWSlots;
      if (kSteady) wait_vmcnt<kSteadyWait>();
      else if (kb + 1 < KB) wait_vmcnt_le(ops_after(kb + 1, kb - 1));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (kSteady || kb + kTokAhead < KB) issue_t((kb + kTokAhead) % kStages, kb + kTokAhead);
      if (kSteady || kb + kWAhead < KB) load_w(ring[df], kb + kWAhead);
      // gate/up: gate and up tiles; down: both tiles lie in row half wave >> 1
      // (fp4: the MFMA applied the weight scales)
      const float sw0 = kFp4 ? 1.f : s_sw[kMode == 0 ? 0 : (wave >> 1)][kb];
      const float sw1 = kFp4 ? 1.f : s_sw[kMode == 0 ? 1 : (wave >> 1)][kb];
      float m[2][NT];   // s_w(kb) * s_x(row, kb); lane holds token l32 of each token tile
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float sx = s_sx[kb * kTok + j * 32 + l32];
        m[0][j] = sw0 * sx;
        m[1][j] = sw1 * sx;
      }
      // Instruction order pinned, a three-stage pipeline over the 2*NT tiles
      // k = 2j + t: slot s issues the first MFMA of tile s, the second MFMA
      // of tile s-1 and the promotion of tile s-2 (split around the second
      // MFMA), so that each MFMA's input was finished two MFMAs earlier, the
      // vector unit promotes while the matrix core runs, and only three
      // tiles' partial sums are live (they fit the vector registers the
      // promotion reads).  The next block's fragments are read at slot NT.
      constexpr int NK = 2 * NT;
      const int stn = (kb + 1) % kStages;
      const bool next = kSteady || kb + 1 < KB;
      f32x16 part[NK];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sl = 0; sl < NK + 2; ++sl) {
        if (sl < NK) {
          const int j = sl >> 1, t = sl & 1;
          part[sl] = mfma(ring[d], t, 0, fb[p][0][j], f32x16{});
        }
        __builtin_amdgcn_sched_barrier(0);
        if (sl >= 2) {
          const int k = sl - 2, j = k >> 1, t = k & 1;
#pragma unroll
          for (int r = 0; r < 8; ++r) acc[t][j][r] = __builtin_fmaf(part[k][r], m[t][j], acc[t][j][r]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (sl >= 1 && sl - 1 < NK) {
          const int k = sl - 1, j = k >> 1, t = k & 1;
          part[k] = mfma(ring[d], t, 1, fb[p][1][j], part[k]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (sl >= 2) {
          const int k = sl - 2, j = k >> 1, t = k & 1;
#pragma unroll
          for (int r = 8; r < 16; ++r) acc[t][j][r] = __builtin_fmaf(part[k][r], m[t][j], acc[t][j][r]);
        }
        if (sl == NT && next) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < NT; ++j) fb[p ^ 1][h][j] = frag(stn, j, h);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    constexpr std::integral_constant<int, 0> i0{};
    constexpr std::integral_constant<int, 1> i1{};
    constexpr std::integral_constant<int, 2> i2{};
    constexpr std::true_type steady{};
    constexpr std::false_type guarded{};
    static_assert(kWSlots == 3 && kTokAhead - kWAhead == 3, "head of three blocks, loops unrolled by six");
    // block 0's fragments, once its DMA landed for every wave
    wait_vmcnt_le(ops_after(0, -1));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < NT; ++j) fb[0][h][j] = frag(0, j, h);
    // head: blocks 0-2 (the prologue's tops issued no weights before block
    // 0); weight slot kb % 3 and fragment parity kb % 2 stay compile-time
    block(0, i0, i0, guarded);
    if (1 < KB) block(1, i1, i1, guarded);
    if (2 < KB) block(2, i2, i0, guarded);
    int kb = 3;
    for (; kb + 5 + kTokAhead < KB; kb += 6) {
      block(kb, i0, i1, steady);
      block(kb + 1, i1, i0, steady);
      block(kb + 2, i2, i1, steady);
      block(kb + 3, i0, i0, steady);
      block(kb + 4, i1, i1, steady);
      block(kb + 5, i2, i0, steady);
    }
    for (; kb < KB; kb += 6) {
      block(kb, i0, i1, guarded);
      if (kb + 1 < KB) block(kb + 1, i1, i0, guarded);
      if (kb + 2 < KB) block(kb + 2, i2, i1, guarded);
      if (kb + 3 < KB) block(kb + 3, i0, i0, guarded);
      if (kb + 4 < KB) block(kb + 4, i1, i1, guarded);
      if (kb + 5 < KB) block(kb + 5, i2, i0, guarded);
    }
  };
  switch (ntok) {
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 3: mainloop(std::integral_constant<int, 3>{}); break;
    default: mainloop(std::integral_constant<int, 4>{}); break;
  }

  // ---- epilogue.  Lane holds token l32 of each token tile and channels
  // (r/4)*8 + hl*4 + r%4 of each 32-row weight tile.  The outputs go through
  // LDS (the token ring is free now): each wave writes its values in row-major
  // order, 16-byte chunk c of row r at chunk c ^ (r & (CH-1)) (CH chunks per
  // row), then the workgroup stores whole rows, 16 contiguous bytes per lane.
  constexpr int RB = kMode == 0 ? 128 : 512;   // bytes per output row of the tile (fp8 h; bf16 y)
  constexpr int CH = RB / 16;
  static_assert(kTok * RB <= kStages * kStage, "the output tile fits the token ring");
  if (kMode == 0) {
    // h = act(g) * u, quantized per row over the tile's 128 channels
    // (s = amax / 448; 4 waves x 32 channels)
    float hv[4][16];
    with_gate_act(a.gate_act, [&](auto k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) gated16<decltype(k)::value>(acc[0][j], acc[1][j], hv[j]);
    });
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(hv[j][r]));
      m = fmaxf(m, __shfl_xor(m, 32));
      if (hl == 0) s_amax[wave][j * 32 + l32] = m;
    }
    __syncthreads();   // (also: every wave is done with the token ring)
    const int NG = N / 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = j * 32 + l32;
      if (j >= ntok || r >= valid) continue;
      const float amax = fmaxf(fmaxf(s_amax[0][r], s_amax[1][r]), fmaxf(s_amax[2][r], s_amax[3][r]));
      const float s = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = wave * 32 + q * 8 + hl * 4;
        *(uint32_t*)(smem + r * RB + (((ch >> 4) ^ (r & (CH - 1))) << 4) + (ch & 15)) =
            pack_fp8x4(hv[j][q * 4 + 0] / s, hv[j][q * 4 + 1] / s, hv[j][q * 4 + 2] / s, hv[j][q * 4 + 3] / s);
      }
      if (wave == 0 && hl == 0) a.out_scales[(int64_t)(it.row_begin + r) * NG + it.ntile] = s;
    }
  } else {
    __syncthreads();   // every wave is done with the token ring
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = j * 32 + l32;
      if (j >= ntok || r >= valid) continue;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& y = acc[t][j];
          const int ch = wave * 64 + t * 32 + q * 8 + hl * 4;
          *(i32x2*)(smem + r * RB + (((ch >> 3) ^ (r & (CH - 1))) << 4) + ((ch >> 2) & 1) * 8) =
              i32x2{(int)pack_bf16x2(y[q * 4 + 0], y[q * 4 + 1]), (int)pack_bf16x2(y[q * 4 + 2], y[q * 4 + 3])};
        }
    }
  }
  __syncthreads();
  const int elt = kMode == 0 ? 1 : 2;               // output bytes per channel
  const int64_t col0 = (int64_t)it.ntile * (RB / elt);
  for (int idx = tid; idx < valid * CH; idx += kThreads) {
    const int r = idx / CH, c = idx % CH;
    const int64_t ch = col0 + c * (16 / elt);
    if (ch < N)
      *(i32x4*)((uint8_t*)a.out + ((int64_t)(it.row_begin + r) * N + ch) * elt) =
          *(const i32x4*)(smem + r * RB + ((c ^ (r & (CH - 1))) << 4));
  }
}

}  // namespace

bool gemm_grouped_fp8_fits(int64_t act_rows, int K) {
  return K % 128 == 0 && K / 128 <= kMaxKB && act_rows * (int64_t)K <= (int64_t)UINT32_MAX;
}

hipError_t launch_gemm_grouped_fp8(const GemmArgs& a, int64_t act_rows, int mode, bool fp4, int grid,
                                   hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  if (!gemm_grouped_fp8_fits(act_rows, a.K)) return hipErrorInvalidValue;
  GemmArgs c = a;
  c.act_rows = act_rows;
  if (mode != 0 && c.out_f32) return hipErrorInvalidValue;   // down writes bf16 y
  if (fp4 && !c.scale_ue8m0) return hipErrorInvalidValue;   // fp4 weights carry UE8M0 scales
  dim3 g(grid), b(kThreads);
  if (fp4) {
    if (mode == 0) hipLaunchKernelGGL((gemm_grouped_fp8_kernel<0, true>), g, b, 0, stream, c);
    else hipLaunchKernelGGL((gemm_grouped_fp8_kernel<1, true>), g, b, 0, stream, c);
  } else {
    if (mode == 0) hipLaunchKernelGGL((gemm_grouped_fp8_kernel<0, false>), g, b, 0, stream, c);
    else hipLaunchKernelGGL((gemm_grouped_fp8_kernel<1, false>), g, b, 0, stream, c);
  }
  return hipGetLastError();
}

}  // namespace moe
