// Grouped GEMMs of bf16 expert MLPs on tile-packed weights, one wave per SIMD.
//
// "Experts backends": each expert is a gated MLP (backend table, row
// deepgemm_megamoe: up projection, gated activation, down projection; section
// "SonicMoE": silu, gelu or relu gates) and all experts run as one grouped
// GEMM over the expert-sorted token rows (rows grouped_mm / deepgemm):
//
//   gate/up : h[r, j] = act(x_r . w_gate[e, j]) * (x_r . w_up[e, j])
//   down    : y[r, o] = h_r . w_down[e, o]
//
// Tile = 256 weight rows x 256 token rows.  4 waves, one per SIMD (512
// registers each: the 256 fp32 accumulators live in the accumulation
// registers); wave w owns 64 weight rows (gate/up: gate rows and up rows of
// the same 32 channels, so the gated activation is applied in registers) for
// all 256 tokens, as 2 x 8 tiles of v_mfma_f32_32x32x16_bf16.
//
// The two operands travel differently.  Weight rows are private to a wave:
// they go from the packed chunks (pack.hip) straight into registers in MFMA
// operand order, several K steps ahead, and never touch LDS.  Token rows are
// shared by all four waves: they are gathered through the expert permutation
// into an LDS ring by global_load_lds (the DMA path), 128 bytes (64 bf16, one
// cache line) per row and K step, so every gathered row is read from memory
// in whole lines.  One barrier per 64-deep K step; the LDS traffic per step is
// 32 KB of DMA writes and 64 KB of fragment reads (each token fragment feeds
// two MFMAs, each weight fragment eight).
//
// Pipeline (4 slots, unrolled by 4): at the top of step s the weights and
// tokens of step s+1 have landed; the barrier frees the LDS stage of step
// s-1, which receives the tokens of step s+3, and the register slot of step
// s-1 receives its weights.  The token fragments of each 16-deep K slice are
// read from LDS while the MFMAs of the previous slice run.  Token tiles past
// the item's last row skip their DMA, their LDS reads and their MFMAs.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kThreads = 256;            // 4 waves, one per SIMD
constexpr int kTok = 256;                // token rows per tile
constexpr int kStepB = 128;              // bytes of a token row per K step (64 bf16)
constexpr int kStage = kTok * kStepB;    // 32 KB of tokens per LDS stage
constexpr int kStages = 5;               // LDS stages of tokens (160 KB)
constexpr int kTokAhead = kStages - 1;   // steps the token DMA runs ahead
// register slots of weights: loaded two steps ahead, so at most 48 memory
// instructions separate a weight load from its use (the 6-bit vmcnt counter
// and the compiler's waits for the registers stay exact)
constexpr int kWSlots = 3;
constexpr int kWAhead = kWSlots - 1;     // steps the weight loads run ahead
constexpr int kChunk = 256 * 64;         // packed weight chunk: 256 rows x 64 bytes (32 K)
constexpr int kWLoads = 8;               // weight loads per wave and K step
// word 3 of a gfx9 buffer resource: 32-bit data format, raw (untyped) access
constexpr int kBufferConfig = 0x00020000;

typedef __attribute__((address_space(3))) void* lds_ptr;

// token row r's 16-byte chunk c (of 8) sits at position c ^ ((r >> 1) & 7):
// the 16 lanes of a fragment read (16 consecutive rows, one chunk) then touch
// 16 distinct 16-byte bank groups
__device__ __forceinline__ int tswz(int r, int c) { return r * kStepB + ((c ^ ((r >> 1) & 7)) << 4); }
// packed weights: row r's 16-byte piece c (of 4) of a 64-byte K step at c ^ ((r >> 2) & 3)
__device__ __forceinline__ int wswz(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

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

// weights of one K step for one wave: [weight tile][16-deep K slice]
struct WStep {
  bf16x8 a[2][4];
};

template <int kMode, bool kOutF32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_grouped_bf16_kernel(
    GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage];
  const int w = xcd_work_index<kGroupedXcdChunk>(a.sched->total);
  if (w < 0) return;
  const WorkItem it = ((const WorkItem*)(a.sched + 1))[w];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int K = a.K, N = a.N;
  const int KT = K / 64;                   // K steps (K is a multiple of 64)
  const int valid = it.row_end - it.row_begin;
  const int ntok = (valid + 31) >> 5;      // live 32-token tiles, 1..8

  // ---- weights: packed chunks of (expert, tile), two 64-byte chunks per step.
  // Loads go through a buffer resource over the tile: a fixed 32-bit lane
  // offset plus a scalar offset per K step, so no per-lane address math.
  const uint8_t* wbase = (const uint8_t*)a.w0 + ((int64_t)it.expert * a.wtiles + it.ntile) * (2 * KT) * (int64_t)kChunk;
  const __amdgpu_buffer_rsrc_t wres =
      __builtin_amdgcn_make_buffer_rsrc((void*)wbase, 0, 2 * KT * kChunk, kBufferConfig);
  int arow[2];
  if (kMode == 0) {
    arow[0] = wave * 32 + l32;          // gate rows of channels wave*32 .. +31
    arow[1] = 128 + wave * 32 + l32;    // up rows of the same channels
  } else {
    arow[0] = wave * 64 + l32;
    arow[1] = wave * 64 + 32 + l32;
  }
  // K slice q of a step lives in chunk q >> 1, pieces (q & 1) * 2 + hl
  int aoff[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int p = 0; p < 2; ++p) aoff[t][p] = wswz(arow[t], p * 2 + hl);
  // half h of the weights of step kt: K slices 2h, 2h+1 (chunk h)
  auto load_w_part = [&](WStep& ws, int kt, int h) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        ws.a[t][2 * h + qq] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(wres, aoff[t][qq], (2 * kt + h) * kChunk, 0));
  };
  auto load_w = [&](WStep& ws, int kt) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        ws.a[t][q] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(wres, aoff[t][q & 1], (2 * kt + (q >> 1)) * kChunk, 0));
  };

  // ---- tokens: DMA instruction i of wave w fills LDS rows 32i + 8w .. +8,
  // i.e. token tile i; lane l writes position l & 7 of row 32i + 8w + l/8.
  // A buffer resource over the activation rows (at most 4 GiB, checked by the
  // launcher); lane offsets fixed, the K step's 128 bytes as scalar offset.
  const __amdgpu_buffer_rsrc_t tres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.act), 0, (int)(uint32_t)(a.act_rows * (int64_t)K * 2), kBufferConfig);

  int toff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 32 * i + 8 * wave + (lane >> 3);
    int r = it.row_begin + row;
    r = r < it.row_end ? r : it.row_end - 1;
    const uint32_t src_row = a.gather ? (uint32_t)(a.gather[r] / a.gather_div) : (uint32_t)r;
    const uint32_t c = (uint32_t)((lane & 7) ^ ((row >> 1) & 7));
    toff[i] = (int)(src_row * (uint32_t)(K * 2) + c * 16);
  }

  f32x16 acc[2][8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = f32x16{};

  auto mainloop = [&](auto nt_const) {
    constexpr int NT = decltype(nt_const)::value;
    // tokens of step kt into LDS stage `stage`
    auto issue_t = [&](int stage, int kt) {
      uint8_t* sb = smem + stage * kStage + wave * 1024;
#pragma unroll
      for (int i = 0; i < NT; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(tres, (lds_ptr)(sb + i * 4096), 16, toff[i], kt * kStepB, 0, 0);
    };
    // half h of the token DMA of step kt: tiles [h * 4, h * 4 + 4) of the live ones
    auto issue_t_part = [&](int stage, int kt, int h) {
      uint8_t* sb = smem + stage * kStage + wave * 1024;
#pragma unroll
      for (int i = 0; i < NT; ++i)
        if (i / 4 == h)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(tres, (lds_ptr)(sb + i * 4096), 16, toff[i], kt * kStepB, 0, 0);
    };
    // token fragments of K slice q of the stage at sb (row j*32 + l32, chunk 2q + hl)
    auto read_b = [&](bf16x8 (&fb)[8], const uint8_t* sb, int q) {
#pragma unroll
      for (int j = 0; j < NT; ++j) fb[j] = *(const bf16x8*)(sb + tswz(j * 32 + l32, 2 * q + hl));
    };
    auto mfma_slice = [&](const WStep& ws, const bf16x8 (&fb)[8], int q) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ws.a[t][q], fb[j], acc[t][j], 0, 0, 0);
    };
    // The issue order is that of a sequence of step tops t = -kTokAhead,
    // -kTokAhead+1, ...: top t issues the tokens of step t+kTokAhead, then
    // the weights of step t+kWAhead (each if that step exists; the tops
    // t < 0 form the prologue).  ops_after(j, upto): memory instructions
    // issued after the tokens of step j once the tops up to `upto` issued.
    auto ops_after = [&](int j, int upto) {
      const int t0 = j - kTokAhead;
      int n = (t0 + kWAhead >= 0 && t0 + kWAhead < KT) ? kWLoads : 0;
      for (int t = t0 + 1; t <= upto; ++t) {
        if (t + kTokAhead >= 0 && t + kTokAhead < KT) n += NT;
        if (t + kWAhead >= 0 && t + kWAhead < KT) n += kWLoads;
      }
      return n;
    };
    constexpr int kSteadyWait = kWLoads + (kTokAhead - 2) * (NT + kWLoads);
    static_assert(kSteadyWait < 64, "vmcnt range");

    WStep ring[kWSlots];
    bf16x8 fb[2][8];
    // prologue: the tops t < 0, then step 0's tokens landed
#pragma unroll
    for (int t = -kTokAhead; t < 0; ++t) {
      if (t + kTokAhead < KT) issue_t(t + kTokAhead, t + kTokAhead);
      if (t + kWAhead >= 0 && t + kWAhead < KT) load_w(ring[(t + kWAhead + kWSlots) % kWSlots], t + kWAhead);
    }
    // (a compile-time count whenever every prologue top issued in full, so
    // that the compiler's own waits for the weight registers stay exact)
    if (KT >= kTokAhead) wait_vmcnt<(kTokAhead - 1) * NT + (kWAhead - 0) * kWLoads>();
    else wait_vmcnt<0>();
    // ... and the top of step 0 needs step 1's tokens
    if (KT >= kTokAhead) wait_vmcnt<(kTokAhead - 2) * NT + (kWAhead - 0) * kWLoads>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    read_b(fb[0], smem, 0);

    // One K step s: weights in register slot d = s % kWSlots, tokens in LDS
    // stage `st` = s % kStages.  At its top: this wave's tokens of step s+1
    // landed (and, by issue order, every earlier load), then the barrier
    // (every wave's tokens of s+1 landed; stage s-1 is no longer read), then
    // the tokens of step s+kTokAhead into stage (s-1) % kStages and the
    // weights of step s+kWAhead into slot (s-1) % kWSlots.  The weights'
    // own waits are the compiler's.
    auto step = [&](int s, int st, auto d_const, auto tail_const) {
      constexpr int d = decltype(d_const)::value;
      constexpr bool kTail = decltype(tail_const)::value;
      constexpr int df = (d + kWAhead) % kWSlots;
      const int st_next = st + 1 == kStages ? 0 : st + 1;
      const int st_fill = st == 0 ? kStages - 1 : st - 1;
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const bool do_t = !kTail || s + kTokAhead < KT;
      const bool do_w = !kTail || s + kWAhead < KT;
      const bool do_next = !kTail || s + 1 < KT;
      const uint8_t* sb = smem + st * kStage;
      const uint8_t* sbn = smem + st_next * kStage;
      uint8_t* sfill = smem + st_fill * kStage + wave * 1024;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // Slice q in eight micro-steps pinned in program order: the two MFMAs
        // of token tile k, the read of tile k of the next slice (slice 0 of
        // step s+1 after slice 3), and after every second micro-step one of
        // the step's 16 memory instructions (token DMA in slices 0-1, weights
        // in slices 2-3, the order the waits count), so that the matrix pipe
        // and the address unit both see a steady stream.
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (k < NT) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
              acc[t][k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[d].a[t][q], fb[q & 1][k], acc[t][k], 0, 0, 0);
            if (q < 3) fb[(q + 1) & 1][k] = *(const bf16x8*)(sb + tswz(k * 32 + l32, 2 * q + 2 + hl));
            else if (do_next) fb[0][k] = *(const bf16x8*)(sbn + tswz(k * 32 + l32, hl));
          }
          if (k & 1) {
            const int m = q * 4 + (k >> 1);   // memory instruction m of the step
            if (m < 8) {
              if (do_t && m < NT)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(tres, (lds_ptr)(sfill + m * 4096), 16, toff[m],
                                                         (s + kTokAhead) * kStepB, 0, 0);
            } else if (do_w) {
              const int wq = m - 8, t = wq & 1, sl = wq >> 1;   // weight tile t, K slice sl
              ring[df].a[t][sl] = __builtin_bit_cast(
                  bf16x8, __builtin_amdgcn_raw_buffer_load_b128(wres, aoff[t][sl & 1],
                                                                (2 * (s + kWAhead) + (sl >> 1)) * kChunk, 0));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the next step's top waits until this wave's tokens of step s+2
      // landed (issued right here, at the end of this step: nothing is
      // issued in between)
      if (!kTail) wait_vmcnt<kSteadyWait>();
      else if (s + 1 < KT) wait_vmcnt_le(ops_after(s + 2, s));
    };
    constexpr std::integral_constant<int, 0> d0{};
    constexpr std::integral_constant<int, 1> d1{};
    constexpr std::integral_constant<int, 2> d2{};
    constexpr std::false_type steady{};
    constexpr std::true_type tail{};
    static_assert(kWSlots == 3, "the step loop is unrolled by the weight slots");
    int s = 0, st = 0;
    auto adv = [&](int& x) { x = x + 1 == kStages ? 0 : x + 1; };
    // steady state: steps s .. s+5 issue both operands and read ahead (two
    // rounds of the weight slots per iteration: the compiler's waits for the
    // weights of the first step after the loop back-edge are stricter than
    // needed, so the back-edge comes once every six steps)
    for (; s + 5 + kTokAhead < KT; s += 6) {
      step(s, st, d0, steady);
      adv(st);
      step(s + 1, st, d1, steady);
      adv(st);
      step(s + 2, st, d2, steady);
      adv(st);
      step(s + 3, st, d0, steady);
      adv(st);
      step(s + 4, st, d1, steady);
      adv(st);
      step(s + 5, st, d2, steady);
      adv(st);
    }
    for (; s < KT; s += 3) {
      step(s, st, d0, tail);
      adv(st);
      if (s + 1 < KT) step(s + 1, st, d1, tail);
      adv(st);
      if (s + 2 < KT) step(s + 2, st, d2, tail);
      adv(st);
    }
  };
  switch (ntok) {
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    case 2: mainloop(std::integral_constant<int, 2>{}); break;
    case 3: mainloop(std::integral_constant<int, 3>{}); break;
    case 4: mainloop(std::integral_constant<int, 4>{}); break;
    case 5: mainloop(std::integral_constant<int, 5>{}); break;
    case 6: mainloop(std::integral_constant<int, 6>{}); break;
    case 7: mainloop(std::integral_constant<int, 7>{}); break;
    default: mainloop(std::integral_constant<int, 8>{}); break;
  }

  // ---- epilogue.  Lane holds token l32 of each token tile and channels
  // (r/4)*8 + hl*4 + r%4 of each 32-row weight tile.  bf16 outputs go through
  // LDS (the token ring is free now): each wave writes its values in row-major
  // order, 16-byte chunk c of row r at chunk c ^ (r & (CH-1)) (CH chunks per
  // row), then the workgroup stores whole rows, 16 contiguous bytes per lane,
  // instead of 8-byte pieces of 32 different rows per store instruction.
  if constexpr (!kOutF32) {
    constexpr int CW = kMode == 0 ? 128 : 256;   // output channels of the tile
    constexpr int CH = CW / 8;                   // 16-byte chunks per row
    __syncthreads();   // every wave is done with the token ring
    // Every lane converts its values without conditions (rows past the item
    // land in LDS rows that are never stored; only whole dead token tiles,
    // a uniform condition, are skipped), with the gate activation fixed at
    // compile time, so that the conversion is straight-line code.
    auto stage = [&](auto act_const) {
      constexpr int kAct = decltype(act_const)::value;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j >= ntok) break;
        const int r = j * 32 + l32;
#pragma unroll
        for (int t = 0; t < (kMode == 0 ? 1 : 2); ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
              v[c] = kMode == 0 ? gate_act<kAct>(acc[0][j][q * 4 + c]) * acc[1][j][q * 4 + c]
                                : acc[t][j][q * 4 + c];
            const int ch = (kMode == 0 ? wave * 32 : wave * 64 + t * 32) + q * 8 + hl * 4;
            *(i32x2*)(smem + r * (CW * 2) + (((ch >> 3) ^ (r & (CH - 1))) << 4) + ((ch >> 2) & 1) * 8) =
                i32x2{(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
          }
      }
    };
    if (kMode != 0 || a.gate_act == 0) stage(std::integral_constant<int, 0>{});
    else if (a.gate_act == 1) stage(std::integral_constant<int, 1>{});
    else stage(std::integral_constant<int, 2>{});
    __syncthreads();
    const int ch_tile = it.ntile * CW;
    for (int idx = tid; idx < valid * CH; idx += kThreads) {
      const int r = idx / CH, c = idx % CH;
      const int ch = ch_tile + c * 8;
      if (ch < N) {
        const i32x4 v = *(const i32x4*)(smem + r * (CW * 2) + ((c ^ (r & (CH - 1))) << 4));
        i32x4* dst = (i32x4*)((uint16_t*)a.out + (int64_t)(it.row_begin + r) * N + ch);
        // y goes straight to memory (streaming stores; the combine reads it
        // once, after the launch): dsv3_bf16 down 2.49 -> 2.46 ms, combine
        // 200 -> 205 us.  h stays cached for the down launch.
        if constexpr (kMode == 1) __builtin_nontemporal_store(v, dst);
        else *dst = v;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = it.row_begin + j * 32 + l32;
      if (j >= ntok || row >= it.row_end) continue;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = it.ntile * 256 + wave * 64 + t * 32 + q * 8 + hl * 4;
          if (ch >= N) continue;
          const f32x16& y = acc[t][j];
          *(f32x4*)((float*)a.out + (int64_t)row * N + ch) =
              f32x4{y[q * 4 + 0], y[q * 4 + 1], y[q * 4 + 2], y[q * 4 + 3]};
        }
    }
  }
}

}  // namespace

bool gemm_grouped_bf16_fits(int64_t act_rows, int K) {
  return K % 64 == 0 && act_rows * (int64_t)K * 2 <= (int64_t)UINT32_MAX;
}

hipError_t launch_gemm_grouped_bf16(const GemmArgs& a, int64_t act_rows, int mode, int grid, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  if (!gemm_grouped_bf16_fits(act_rows, a.K)) return hipErrorInvalidValue;
  GemmArgs c = a;
  c.act_rows = act_rows;
  dim3 g(grid), b(kThreads);
  if (mode == 0) hipLaunchKernelGGL((gemm_grouped_bf16_kernel<0, false>), g, b, 0, stream, c);
  else if (c.out_f32) hipLaunchKernelGGL((gemm_grouped_bf16_kernel<1, true>), g, b, 0, stream, c);
  else hipLaunchKernelGGL((gemm_grouped_bf16_kernel<1, false>), g, b, 0, stream, c);
  return hipGetLastError();
}

}  // namespace moe
