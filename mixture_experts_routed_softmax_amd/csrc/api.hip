// libmoe host side: argument validation, workspace layout, launch sequences
// and stage timing.  The C ABI is declared in include/moe.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <algorithm>
#include <mutex>
#include <vector>

#include "moe.h"
#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define MOE_TRY_HIP(expr, what)                      \
  do {                                               \
    hipError_t e_ = (expr);                          \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int64_t pairs(const moe_desc* d) { return d->T * (int64_t)d->k; }

size_t elt_bytes(int dt) { return dt == MOE_DT_F32 ? 4 : dt == MOE_DT_BF16 ? 2 : 1; }
// bytes of one weight row of K values (fp4: two codes per byte)
int64_t w_row_bytes(int dt, int64_t K) { return dt == MOE_DT_FP4_E2M1 ? K / 2 : K * (int64_t)elt_bytes(dt); }

// quantized experts (fp8 or fp4 weights): activations and h are e4m3 codes
// with per-row per-128 fp32 scales
bool is_fp8(const moe_desc* d) { return d->w_dtype == MOE_DT_FP8_E4M3 || d->w_dtype == MOE_DT_FP4_E2M1; }
// weight format code of the streaming / packed kernels: 0 bf16, 1 fp8, 2 fp4
int wfmt(const moe_desc* d) {
  return d->w_dtype == MOE_DT_FP4_E2M1 ? 2 : (d->w_dtype == MOE_DT_FP8_E4M3 ? 1 : 0);
}

moe_status validate(const moe_desc* d) {
  if (!d) return fail(MOE_EINVAL, "desc is NULL");
  if (d->T < 0) return fail(MOE_EINVAL, "T = %lld < 0", (long long)d->T);
  if (d->H <= 0 || d->I <= 0) return fail(MOE_EINVAL, "H = %d, I = %d must be positive", d->H, d->I);
  if (d->E < 1 || d->E > kMaxExperts) return fail(MOE_EINVAL, "E = %d outside 1..%d", d->E, kMaxExperts);
  if (d->k < 1 || d->k > d->E) return fail(MOE_EINVAL, "k = %d outside 1..E (E = %d)", d->k, d->E);
  if (d->k > kMaxTopK) return fail(MOE_EUNSUPPORTED, "k = %d above %d", d->k, kMaxTopK);
  if (d->score != MOE_SCORE_SOFTMAX && d->score != MOE_SCORE_SIGMOID)
    return fail(MOE_EINVAL, "score = %d", d->score);
  if (d->renormalize != 0 && d->renormalize != 1)
    return fail(MOE_EINVAL, "renormalize = %d", d->renormalize);
  if (!std::isfinite(d->routed_scale)) return fail(MOE_EINVAL, "routed_scale is not finite");
  if (d->act_dtype != MOE_DT_F32 && d->act_dtype != MOE_DT_BF16)
    return fail(MOE_EINVAL, "act_dtype = %d", d->act_dtype);
  if (d->w_dtype != MOE_DT_F32 && d->w_dtype != MOE_DT_BF16 && d->w_dtype != MOE_DT_FP8_E4M3 &&
      d->w_dtype != MOE_DT_FP4_E2M1)
    return fail(MOE_EINVAL, "w_dtype = %d", d->w_dtype);
  if (d->y_dtype != MOE_DT_F32 && d->y_dtype != MOE_DT_BF16)
    return fail(MOE_EINVAL, "y_dtype = %d", d->y_dtype);
  if (d->path < MOE_PATH_AUTO || d->path > MOE_PATH_STREAM) return fail(MOE_EINVAL, "path = %d", d->path);
  for (int r : d->reserved)
    if (r != 0) return fail(MOE_EINVAL, "reserved fields must be zero");
  if (d->gate_act < MOE_GATE_SILU || d->gate_act > MOE_GATE_RELU)
    return fail(MOE_EINVAL, "gate_act = %d is not a moe_gate_act", d->gate_act);
  if (d->w_layout != MOE_LAYOUT_ROWMAJOR && d->w_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_EINVAL, "w_layout = %d", d->w_layout);
  if (d->w_layout == MOE_LAYOUT_PACKED && d->w_dtype == MOE_DT_F32)
    return fail(MOE_EUNSUPPORTED, "packed weights are bf16 or fp8");
  if (d->T * (int64_t)d->k > (int64_t)INT32_MAX / 2)
    return fail(MOE_EUNSUPPORTED, "T*k = %lld too large", (long long)(d->T * d->k));
  if (d->w_scale_fmt < MOE_SCALE_NONE || d->w_scale_fmt > MOE_SCALE_UE8M0)
    return fail(MOE_EINVAL, "w_scale_fmt = %d", d->w_scale_fmt);
  if (d->act_scheme < MOE_ACT_NONE || d->act_scheme > MOE_ACT_STATIC)
    return fail(MOE_EINVAL, "act_scheme = %d", d->act_scheme);

  if (d->w_dtype == MOE_DT_FP4_E2M1) {
    if (d->w_scale_fmt != MOE_SCALE_UE8M0) return fail(MOE_EINVAL, "fp4 experts need UE8M0 block scales");
    if (d->w_layout != MOE_LAYOUT_PACKED)
      return fail(MOE_EUNSUPPORTED, "fp4 experts run on packed weights only (moe_pack_weights)");
  }
  if (is_fp8(d)) {
    if (d->act_dtype != MOE_DT_BF16)
      return fail(MOE_EUNSUPPORTED, "fp8 experts need bf16 activations");
    if (d->w_scale_fmt == MOE_SCALE_NONE)
      return fail(MOE_EINVAL, "fp8 experts need block scales (F32 or UE8M0)");
    if (d->block != 128) return fail(MOE_EUNSUPPORTED, "fp8 block = %d; only 128 is supported", d->block);
    if (d->act_scheme == MOE_ACT_STATIC)
      return fail(MOE_EUNSUPPORTED,
                  "static (per-tensor) activation quantization is rejected; use dynamic per-row scales");
    if (d->act_scheme != MOE_ACT_DYNAMIC)
      return fail(MOE_EINVAL, "fp8 experts need act_scheme = MOE_ACT_DYNAMIC");
    if (d->H % 128 || d->I % 128)
      return fail(MOE_EUNSUPPORTED, "fp8 experts need H and I multiples of 128 (H = %d, I = %d)", d->H, d->I);
  } else {
    if (d->w_scale_fmt != MOE_SCALE_NONE) return fail(MOE_EINVAL, "block scales given for unquantized experts");
    if (d->act_scheme != MOE_ACT_NONE) return fail(MOE_EINVAL, "act_scheme set for unquantized experts");
    if (d->act_dtype != d->w_dtype)
      return fail(MOE_EUNSUPPORTED, "activation and expert dtypes differ (%d vs %d)", d->act_dtype, d->w_dtype);
    if (d->w_dtype == MOE_DT_BF16 && (d->H % 64 || d->I % 64))
      return fail(MOE_EUNSUPPORTED, "bf16 experts need H and I multiples of 64 (H = %d, I = %d)", d->H, d->I);
    if (d->w_dtype == MOE_DT_F32 && (d->H % 8 || d->I % 8))
      return fail(MOE_EUNSUPPORTED, "fp32 experts need H and I multiples of 8");
  }
  if (d->path == MOE_PATH_STREAM && (d->w_layout != MOE_LAYOUT_PACKED || d->T > kStreamMaxTokens))
    return fail(MOE_EUNSUPPORTED, "the weight-streaming path needs packed weights and T <= %d", kStreamMaxTokens);
  if (d->path == MOE_PATH_STREAM && is_fp8(d) &&
      (d->H / 128 > kStreamMaxScaleBlocks || d->I / 128 > kStreamMaxScaleBlocks))
    return fail(MOE_EUNSUPPORTED, "the fp8 weight-streaming path needs H, I <= %d", 128 * kStreamMaxScaleBlocks);
  return MOE_OK;
}

// ---- workspace layout ----------------------------------------------------

struct Carve {
  uint8_t* base;
  size_t off = 0;
  template <class T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
};

bool packed(const moe_desc* d) { return d->w_layout == MOE_LAYOUT_PACKED; }

int gate_up_ntiles(const moe_desc* d) {
  const int c = packed(d) ? kPackedGateUpChannels
                          : (d->w_dtype == MOE_DT_FP8_E4M3 ? kGemmGateUpChannelsFp8 : kGemmGateUpChannelsBf16);
  return (d->I + c - 1) / c;
}
int down_ntiles(const moe_desc* d) {
  const int c = packed(d) ? kPackedDownChannels
                          : (d->w_dtype == MOE_DT_FP8_E4M3 ? kGemmDownChannelsFp8 : kGemmDownChannelsBf16);
  return (d->H + c - 1) / c;
}

size_t packed_bytes(const moe_desc* d, int which) {
  const int gate_up = which == MOE_PACK_GATE_UP;
  const int64_t N = gate_up ? d->I : d->H;
  const int64_t K = gate_up ? d->H : d->I;
  const int64_t tiles = packed_tiles(gate_up, (int)N);
  return (size_t)d->E * tiles * 256 * w_row_bytes(d->w_dtype, K);
}

// bf16 gate/up and down on packed weights take the one-wave-per-SIMD grouped
// kernel (kernel traces against gemm_packed_kernel: gate/up H = 7168 4.27 vs
// 4.70 ms, H = 2048 260-263 vs 281-287 us; down I = 2048 2.48 vs 2.71 ms,
// I = 1408 154-158 vs 158-162 us); fp8 and fp4 experts the e4m3 one (fp8
// gate/up 3.08 vs 4.17 ms, down 2.04 vs 2.20 ms; fp4 gate/up 2.80 vs
// 3.65 ms, down 1.90 vs 2.08 ms)

// prefill schedules: an expert's items in blocks of kSchedBlockM row tiles x
// kSchedBlockN channel tiles, one block per XCD chunk of the grouped GEMMs
constexpr int kSchedBlockM = 4;
constexpr int kSchedBlockN = 4;

// expert GEMMs stream the touched experts' weights (decode-sized batches)
bool use_stream(const moe_desc* d) {
  if (is_fp8(d) && (d->H / 128 > kStreamMaxScaleBlocks || d->I / 128 > kStreamMaxScaleBlocks))
    return false;
  return packed(d) && d->T <= kStreamMaxTokens && (d->path == MOE_PATH_STREAM || d->path == MOE_PATH_AUTO);
}

// token rows per grouped-GEMM tile
int rows_per_tile(const moe_desc* d) {
  if (use_stream(d)) return kStreamMaxTokens;
  if (packed(d)) return is_fp8(d) ? kPackedTokFp8 : kPackedTokBf16;
  return kGemmRowsPerTile;
}

int64_t sched_capacity(const moe_desc* d, int ntiles) {
  const int64_t P = pairs(d);
  const int bm = rows_per_tile(d);
  const int64_t tiles = (P + bm - 1) / bm + std::min<int64_t>(d->E, P);
  return tiles * ntiles;
}

// Weight streaming: work units (items x K splits) the launch must cover, and
// split-K partial tiles the workspace must hold.  A split happens only below
// kStreamTarget items, so split units stay below 3 * kStreamTarget.
int64_t stream_units_cap(int64_t items) { return 2 * items + kStreamTarget; }
int64_t stream_partial_units(const moe_desc* d) {
  if (!use_stream(d)) return 0;
  const int64_t items = std::max(sched_capacity(d, gate_up_ntiles(d)), sched_capacity(d, down_ntiles(d)));
  return std::min<int64_t>(items * kStreamMaxSplit, 3 * kStreamTarget);
}
size_t stream_partial_bytes(const moe_desc* d) { return (size_t)stream_partial_units(d) * kStreamPartFloats * 4; }

size_t sched_bytes(int64_t cap) { return sizeof(Schedule) + (size_t)cap * sizeof(WorkItem); }

// grid covering every item index up to cap under xcd_work_index's mapping
// with chunks of `chunk` items
int grid_for(int64_t cap, int chunk = kXcdChunk) {
  const int64_t per = (int64_t)kNumXcd * chunk;
  return (int)((cap + per - 1) / per * per);
}

struct PermuteWs {
  int32_t* block_counts;
  int32_t* block_base;
  int32_t* sched_tables;   // scan -> scatter: what the schedules' items are computed from
  uint8_t* xq;
  float* xs;
};

PermuteWs carve_permute(Carve& c, const moe_desc* d, bool with_quant) {
  const int64_t nb = perm_blocks(pairs(d));
  PermuteWs w{};
  w.block_counts = c.take<int32_t>((size_t)nb * d->E);
  w.block_base = c.take<int32_t>((size_t)nb * d->E);
  w.sched_tables = c.take<int32_t>(kSchedTablesInts);
  if (with_quant) {
    w.xq = c.take<uint8_t>((size_t)d->T * d->H);
    w.xs = c.take<float>((size_t)d->T * (d->H / 128));
  }
  return w;
}

struct ForwardWs {
  float* route_part;
  int32_t* ids;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  PermuteWs pw;
  int32_t* perm;
  int32_t* inv;
  int32_t* touched;
  Schedule* sched_gu;
  Schedule* sched_dn;
  void* h;
  float* hs;
  void* y;
  float* partial;
  int32_t* rowinfo;   // weight streaming: where the down launch left each row
};

ForwardWs carve_forward(Carve& c, const moe_desc* d) {
  const int64_t P = pairs(d);
  ForwardWs w{};
  w.route_part = (float*)c.take<uint8_t>(route_workspace_bytes(d->T, d->H, d->E, d->act_dtype == MOE_DT_BF16));
  w.ids = c.take<int32_t>(P);
  w.w = c.take<float>(P);
  w.counts = c.take<int32_t>(d->E);
  w.offsets = c.take<int32_t>(d->E + 1);
  w.pw = carve_permute(c, d, is_fp8(d));
  w.perm = c.take<int32_t>(P);
  w.inv = c.take<int32_t>(P);
  w.touched = c.take<int32_t>(d->E + 1);
  if (d->w_dtype != MOE_DT_F32) {
    w.sched_gu = (Schedule*)c.take<uint8_t>(sched_bytes(sched_capacity(d, gate_up_ntiles(d))));
    w.sched_dn = (Schedule*)c.take<uint8_t>(sched_bytes(sched_capacity(d, down_ntiles(d))));
  }
  w.h = c.take<uint8_t>((size_t)P * d->I * (is_fp8(d) ? 1 : elt_bytes(d->w_dtype)));
  if (is_fp8(d)) w.hs = c.take<float>((size_t)P * (d->I / 128));
  w.y = c.take<uint8_t>((size_t)P * d->H * elt_bytes(d->y_dtype));
  if (use_stream(d)) {
    w.partial = (float*)c.take<uint8_t>(stream_partial_bytes(d));
    w.rowinfo = c.take<int32_t>(P);
  }
  return w;
}

size_t backward_ws_size(const moe_desc* d);

size_t ws_size(const moe_desc* d, int op) {
  Carve c{nullptr};
  switch (op) {
    case MOE_OP_ROUTE: return align_up(route_workspace_bytes(d->T, d->H, d->E, d->act_dtype == MOE_DT_BF16));
    case MOE_OP_PERMUTE: carve_permute(c, d, is_fp8(d)); return c.off;
    case MOE_OP_GATE_UP:
      return d->w_dtype == MOE_DT_F32 ? 0
                                      : align_up(sched_bytes(sched_capacity(d, gate_up_ntiles(d)))) +
                                            align_up(stream_partial_bytes(d));
    case MOE_OP_DOWN:
      return d->w_dtype == MOE_DT_F32 ? 0
                                      : align_up(sched_bytes(sched_capacity(d, down_ntiles(d)))) +
                                            align_up(stream_partial_bytes(d));
    case MOE_OP_COMBINE: return 0;
    case MOE_OP_FORWARD: carve_forward(c, d); return c.off;
    case MOE_OP_BACKWARD: return backward_ws_size(d);
    default: return 0;
  }
}

moe_status check_ws(const moe_desc* d, int op, void* ws, size_t ws_bytes) {
  size_t need = ws_size(d, op);
  if (need == 0) return MOE_OK;
  if (!ws || ws_bytes < need)
    return fail(MOE_EWORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, ws_bytes,
                ws ? "" : " (NULL)");
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
  return MOE_OK;
}

// ---- stage timing ----------------------------------------------------------

struct TimedLaunch {
  int stage;
  hipEvent_t start, stop;
};
bool g_timing = false;
// set for the duration of a no-allocation call: no stage events are created
// or recorded (creating an event may allocate)
thread_local bool g_no_events = false;
std::vector<TimedLaunch> g_pending;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pool_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Within one library call the launches are timed back to back: a stage's
// start event is the previous stage's stop event on the same stream (one
// event per launch instead of two; nothing else is enqueued in between).
// Every entry point resets the chain, so work enqueued between calls is never
// attributed to a stage.  The gate/up and backward weight-gradient stages
// (the dominant GEMMs) keep a start event of their own, recorded right before
// their launch: a chained start also counts the dispatch gap before the
// launch (measured: qwen_prefill gate/up 292 instead of 285 us, against a
// 284.5 us kernel).
hipEvent_t g_chain = nullptr;
hipStream_t g_chain_stream = nullptr;

struct StageTimer {
  int stage;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  StageTimer(int st, hipStream_t stream) : stage(st), s(stream) {
    if (!g_timing || g_no_events) return;
    const bool own_start = st == MOE_STAGE_GATE_UP || st == MOE_STAGE_BWD_WEIGHT;
    if (g_chain && g_chain_stream == s && !own_start) {
      a = g_chain;
    } else {
      a = pool_event();
      if (a) hipEventRecord(a, s);
    }
    b = pool_event();
  }
  ~StageTimer() {
    if (!g_timing || g_no_events || !a || !b) return;
    hipEventRecord(b, s);
    g_pending.push_back({stage, a, b});
    g_chain = b;
    g_chain_stream = s;
  }
};

// ---- launch sequences --------------------------------------------------------

SchedRequest sched_req(Schedule* s, const moe_desc* d, int ntiles) {
  SchedRequest r{};
  r.sched = s;
  r.rows_per_tile = rows_per_tile(d);
  r.ntiles = ntiles;
  r.capacity = (int)sched_capacity(d, ntiles);
  if (!use_stream(d)) {
    r.block_m = kSchedBlockM;
    r.block_n = kSchedBlockN;
  }
  return r;
}

moe_status run_permute(const moe_desc* d, const int32_t* ids, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* inv, int32_t* touched, const PermuteWs& pw,
                       SchedRequest s0, SchedRequest s1, hipStream_t st) {
  const int64_t P = pairs(d);
  const int64_t nb = perm_blocks(P);
  if (nb == 1) {
    StageTimer tm(MOE_STAGE_SCAN, st);
    MOE_TRY_HIP(launch_permute_small(ids, P, d->E, counts, offsets, perm, inv, touched, s0, s1, st),
                "permute launch");
    return MOE_OK;
  }
  if (nb <= kFusedHistBlocks) {
    StageTimer tm(MOE_STAGE_SCAN, st);
    MOE_TRY_HIP(launch_hist_scan(ids, P, d->E, counts, offsets, pw.block_base, touched, s0, s1, pw.sched_tables, st),
                "histogram and scan launch");
  } else {
    {
      StageTimer tm(MOE_STAGE_HIST, st);
      MOE_TRY_HIP(launch_hist(ids, P, d->E, pw.block_counts, st), "histogram launch");
    }
    StageTimer tm(MOE_STAGE_SCAN, st);
    MOE_TRY_HIP(launch_scan(pw.block_counts, nb, d->E, counts, offsets, pw.block_base, touched, s0, s1,
                            pw.sched_tables, st),
                "scan launch");
  }
  {
    StageTimer tm(MOE_STAGE_SCATTER, st);
    MOE_TRY_HIP(launch_scatter(ids, P, d->E, pw.block_base, perm, inv, s0, s1, pw.sched_tables, st),
                "scatter launch");
  }
  return MOE_OK;
}

GemmArgs gemm_common(const moe_desc* d) {
  GemmArgs a{};
  a.E = d->E;
  a.P = pairs(d);
  a.scale_ue8m0 = d->w_scale_fmt == MOE_SCALE_UE8M0;
  a.gate_act = d->gate_act;
  return a;
}

// per_expert_items: the streaming schedule holds one entry per touched expert
// (SchedRequest::implicit_items)
moe_status run_gate_up(const moe_desc* d, const void* act, const float* act_scales, const int32_t* gather,
                       const int32_t* offsets, const void* wg, const void* wu, const void* sg,
                       const void* su, void* h, float* hs, const Schedule* sched, float* partial, hipStream_t st,
                       bool per_expert_items = false) {
  GemmArgs a = gemm_common(d);
  a.per_expert_items = per_expert_items;
  a.partial = partial;
  a.act = act;
  a.act_scales = act_scales;
  a.gather = gather;
  a.gather_div = d->k;
  a.w0 = wg;
  a.w1 = wu;
  a.s0 = sg;
  a.s1 = su;
  a.K = d->H;
  a.N = d->I;
  a.out = h;
  a.out_scales = hs;
  a.out_f32 = d->w_dtype == MOE_DT_F32;
  a.sched = sched;
  a.offsets = offsets;
  a.wtiles = (int)packed_tiles(1, d->I);
  StageTimer tm(MOE_STAGE_GATE_UP, st);
  hipError_t e;
  const int grid = grid_for(sched_capacity(d, gate_up_ntiles(d)), kGroupedXcdChunk);
  const int64_t act_rows = gather ? d->T : pairs(d);   // x (read through perm) or x_sorted
  if (use_stream(d))
    e = launch_gemm_stream(a, wfmt(d), 0, grid_for(stream_units_cap(sched_capacity(d, gate_up_ntiles(d)))),
                           (int)std::min<int64_t>(sched_capacity(d, gate_up_ntiles(d)), kStreamTarget), d->T <= 32, st);
  else if (packed(d) && d->w_dtype == MOE_DT_BF16 && gemm_grouped_bf16_fits(act_rows, d->H))
    e = launch_gemm_grouped_bf16(a, act_rows, 0, grid, st);
  else if (packed(d) && is_fp8(d) && gemm_grouped_fp8_fits(act_rows, d->H))
    e = launch_gemm_grouped_fp8(a, act_rows, 0, d->w_dtype == MOE_DT_FP4_E2M1, grid, st);
  else if (packed(d)) e = launch_gemm_packed(a, wfmt(d), 0, grid, st);
  else if (d->w_dtype == MOE_DT_F32) e = launch_gate_up_f32(a, st);
  else if (d->w_dtype == MOE_DT_BF16) e = launch_gate_up_bf16(a, grid, st);
  else e = launch_gate_up_fp8(a, grid, st);
  MOE_TRY_HIP(e, "gate/up launch");
  return MOE_OK;
}

// rowinfo (weight streaming only): skip the split-K reduction launch and
// leave a split launch's y in the partial tiles for launch_combine_stream
moe_status run_down(const moe_desc* d, const void* h, const float* hs, const int32_t* offsets,
                    const void* wd, const void* sd, void* y, const Schedule* sched, float* partial, hipStream_t st,
                    int32_t* rowinfo = nullptr, bool per_expert_items = false) {
  GemmArgs a = gemm_common(d);
  a.per_expert_items = per_expert_items;
  a.rowinfo = rowinfo;
  a.partial = partial;
  a.act = h;
  a.act_scales = hs;
  a.w0 = wd;
  a.s0 = sd;
  a.K = d->I;
  a.N = d->H;
  a.out = y;
  a.out_f32 = d->y_dtype == MOE_DT_F32;
  a.sched = sched;
  a.offsets = offsets;
  a.wtiles = (int)packed_tiles(0, d->H);
  StageTimer tm(MOE_STAGE_DOWN, st);
  hipError_t e;
  const int grid = grid_for(sched_capacity(d, down_ntiles(d)), kGroupedXcdChunk);
  if (use_stream(d))
    e = launch_gemm_stream(a, wfmt(d), 1, grid_for(stream_units_cap(sched_capacity(d, down_ntiles(d)))),
                           (int)std::min<int64_t>(sched_capacity(d, down_ntiles(d)), kStreamTarget), d->T <= 32, st,
                           rowinfo == nullptr);
  else if (packed(d) && d->w_dtype == MOE_DT_BF16 && gemm_grouped_bf16_fits(pairs(d), d->I))
    e = launch_gemm_grouped_bf16(a, pairs(d), 1, grid, st);
  else if (packed(d) && is_fp8(d) && d->y_dtype == MOE_DT_BF16 && gemm_grouped_fp8_fits(pairs(d), d->I))
    e = launch_gemm_grouped_fp8(a, pairs(d), 1, d->w_dtype == MOE_DT_FP4_E2M1, grid, st);
  else if (packed(d)) e = launch_gemm_packed(a, wfmt(d), 1, grid, st);
  else if (d->w_dtype == MOE_DT_F32) e = launch_down_f32(a, st);
  else if (d->w_dtype == MOE_DT_BF16) e = launch_down_bf16(a, grid, st);
  else e = launch_down_fp8(a, grid, st);
  MOE_TRY_HIP(e, "down launch");
  return MOE_OK;
}


// ---- backward ------------------------------------------------------------

moe_status validate_backward(const moe_desc* d) {
  moe_status s = validate(d);
  if (s != MOE_OK) return s;
  if (d->act_dtype != MOE_DT_BF16 || d->w_dtype != MOE_DT_BF16)
    return fail(MOE_EUNSUPPORTED, "the backward takes bf16 activations and bf16 experts");
  if (d->w_layout != MOE_LAYOUT_ROWMAJOR) return fail(MOE_EUNSUPPORTED, "the backward takes row-major weights");
  if (d->H % 128 || d->I % 128)
    return fail(MOE_EUNSUPPORTED, "the backward needs H and I multiples of 128 (H = %d, I = %d)", d->H, d->I);
  return MOE_OK;
}

// the description the backward's grouped GEMMs are planned with
moe_desc backward_desc(const moe_desc* d) {
  moe_desc b = *d;
  b.path = MOE_PATH_GROUPED;
  b.w_layout = MOE_LAYOUT_ROWMAJOR;
  return b;
}

int expert_pad(int E) { return (E + 127) / 128 * 128; }

// tiles of the backward GEMM along an extent n (kBwdTile rows or columns each)
int bwd_tiles(int64_t n) { return (int)((n + kBwdTile - 1) / kBwdTile); }

// ragged-row schedule of a backward GEMM: kBwdTile token rows per tile
SchedRequest bwd_sched_req(Schedule* s, const moe_desc* d, int ntiles) {
  SchedRequest r = sched_req(s, d, ntiles);
  r.rows_per_tile = kBwdTile;
  r.block_m = r.block_n = 1;
  return r;
}

// dW_r = dkey^T x reduces over all T tokens: the K range is split into chunks
// of k_chunk rows (a multiple of 32) so that about 512 workgroups run; the
// fp32 partial sums are added in chunk order afterwards
int router_chunks(const moe_desc* d, int* k_chunk) {
  const int64_t per_chunk = (int64_t)bwd_tiles(d->H) * bwd_tiles(expert_pad(d->E));
  int64_t chunks = (512 + per_chunk - 1) / per_chunk;
  const int64_t max_chunks = (d->T + 255) / 256;
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks < 1) chunks = 1;
  int64_t kc = (d->T + chunks - 1) / chunks;
  kc = (kc + 31) / 32 * 32;
  chunks = (d->T + kc - 1) / kc;
  *k_chunk = (int)kc;
  return (int)chunks;
}

struct BackwardWs {
  float* route_part;
  int32_t* ids;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  PermuteWs pw;
  int32_t* perm;
  int32_t* inv;
  int32_t* touched;
  Schedule* sched_gu;   // recompute of g, u
  Schedule* sched_e;    // e = W_down^T dout (channel tiles of I)
  Schedule* sched_dx;   // dx rows (channel tiles of H)
  uint16_t* x_sorted;
  uint16_t* dout_sorted;
  float* gu;
  float* ev;
  uint16_t* ap;
  uint16_t* dgu;
  float* dw;
  float* dxp;
  float* dkey;
  uint16_t* dkey_b;
  float* dxr;
  float* dwr_part;
  uint16_t* zeros;
};

BackwardWs carve_backward(Carve& c, const moe_desc* d0) {
  const moe_desc bd = backward_desc(d0);
  const moe_desc* d = &bd;
  const int64_t P = pairs(d);
  const int64_t H = d->H, I = d->I;
  BackwardWs w{};
  w.route_part = (float*)c.take<uint8_t>(route_workspace_bytes(d->T, d->H, d->E, 1));
  w.ids = c.take<int32_t>(P);
  w.w = c.take<float>(P);
  w.counts = c.take<int32_t>(d->E);
  w.offsets = c.take<int32_t>(d->E + 1);
  w.pw = carve_permute(c, d, false);
  w.perm = c.take<int32_t>(P);
  w.inv = c.take<int32_t>(P);
  w.touched = c.take<int32_t>(d->E + 1);
  w.sched_gu = (Schedule*)c.take<uint8_t>(sched_bytes(sched_capacity(d, gate_up_ntiles(d))));
  w.sched_e = (Schedule*)c.take<uint8_t>(sched_bytes(sched_capacity(d, bwd_tiles(d->I))));
  w.sched_dx = (Schedule*)c.take<uint8_t>(sched_bytes(sched_capacity(d, bwd_tiles(d->H))));
  w.x_sorted = c.take<uint16_t>((size_t)P * H);
  w.dout_sorted = c.take<uint16_t>((size_t)P * H);
  w.gu = c.take<float>((size_t)P * 2 * I);
  w.ev = c.take<float>((size_t)P * I);
  w.ap = c.take<uint16_t>((size_t)P * I);
  w.dgu = c.take<uint16_t>((size_t)P * 2 * I);
  w.dw = c.take<float>(P);
  w.dxp = c.take<float>((size_t)P * H);
  w.dkey = c.take<float>((size_t)d->T * d->E);
  w.dkey_b = c.take<uint16_t>((size_t)d->T * expert_pad(d->E));
  w.dxr = c.take<float>((size_t)d->T * H);
  int kc = 0;
  w.dwr_part = c.take<float>((size_t)router_chunks(d, &kc) * d->E * H);
  w.zeros = c.take<uint16_t>(128);
  return w;
}

size_t backward_ws_size(const moe_desc* d) {
  const std::string keep = g_err;
  const bool ok = validate_backward(d) == MOE_OK;
  g_err = keep;
  if (!ok || d->T == 0) return 0;
  Carve c{nullptr};
  carve_backward(c, d);
  return c.off;
}

}  // namespace

// ---- static scratch of the no-allocation forward ---------------------------
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops): moe_forward_static carves its workspace out of this
// file-scope array instead of a caller buffer.  Each device holds its own copy
// at its own address from module load until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: its device
// address is taken once per device with hipGetSymbolAddress (with that device
// current) and only that address is passed to kernels.
constexpr size_t kStaticScratchBytes = MOE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, which must be the
// stream's device.
moe_status static_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  MOE_TRY_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EINVAL, "device %d out of range", dev);
  if (stream != nullptr) {
    int sdev = -1;
    MOE_TRY_HIP(hipStreamGetDevice(stream, &sdev), "hipStreamGetDevice");
    if (sdev != dev) return fail(MOE_EINVAL, "the stream belongs to device %d, the current device is %d", sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    MOE_TRY_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (p == nullptr || ((uintptr_t)p & (kAlign - 1)) != 0) return fail(MOE_EHIP, "static scratch address unusable");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

// ============================================================================
extern "C" {

const char* moe_status_str(int s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: unsupported combination";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace missing or too small";
    case MOE_EHIP: return "MOE_EHIP: HIP runtime error";
    default: return "unknown moe_status";
  }
}

const char* moe_last_error(void) { return g_err.c_str(); }

size_t moe_workspace_bytes(const moe_desc* d, int op) {
  if (validate(d) != MOE_OK) return 0;
  return ws_size(d, op);
}

moe_status moe_route_topk(const moe_desc* d, const void* x, const void* w_router, const float* bias,
                          int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  g_chain = nullptr;
  moe_status s = validate(d);
  if (s != MOE_OK) return s;
  if (d->T == 0) return MOE_OK;
  if (!x || !w_router || !ids || !w) return fail(MOE_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(w_router)) return fail(MOE_EINVAL, "x and w_router must be 16-byte aligned");
  if ((s = check_ws(d, MOE_OP_ROUTE, ws, ws_bytes)) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  StageTimer tm(MOE_STAGE_ROUTE, st);
  MOE_TRY_HIP(launch_route_topk(x, w_router, bias, d->T, d->H, d->E, d->k, d->act_dtype == MOE_DT_BF16,
                                d->score, d->renormalize, d->routed_scale, ids, w, (float*)ws, st),
              "router launch");
  return MOE_OK;
}

moe_status moe_permute(const moe_desc* d, const int32_t* ids, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv, void* x_sorted,
                       float* x_sorted_scales, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  g_chain = nullptr;
  moe_status s = validate(d);
  if (s != MOE_OK) return s;
  if (!counts || !offsets) return fail(MOE_EINVAL, "counts and offsets are required");
  const int64_t P = pairs(d);
  if (P > 0 && (!ids || !perm || !inv)) return fail(MOE_EINVAL, "ids, perm and inv are required");
  if ((x == nullptr) != (x_sorted == nullptr)) return fail(MOE_EINVAL, "x and x_sorted go together");
  if (x_sorted && is_fp8(d) && !x_sorted_scales)
    return fail(MOE_EINVAL, "fp8 experts need x_sorted_scales with x_sorted");
  if (x && (!aligned16(x) || !aligned16(x_sorted))) return fail(MOE_EINVAL, "x, x_sorted must be 16-byte aligned");
  if ((s = check_ws(d, MOE_OP_PERMUTE, ws, ws_bytes)) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  Carve c{(uint8_t*)ws};
  PermuteWs pw = carve_permute(c, d, is_fp8(d));
  SchedRequest none{};
  if ((s = run_permute(d, ids, counts, offsets, perm, inv, nullptr, pw, none, none, st)) != MOE_OK) return s;
  if (x_sorted && P > 0) {
    if (is_fp8(d)) {
      {
        StageTimer tm(MOE_STAGE_QUANT_X, st);
        MOE_TRY_HIP(launch_quant_rows_fp8((const uint16_t*)x, d->T, d->H, pw.xq, pw.xs, st), "quantize launch");
      }
      MOE_TRY_HIP(launch_gather_rows(pw.xq, perm, d->k, P, d->H, x_sorted, st), "gather launch");
      MOE_TRY_HIP(launch_gather_scales(pw.xs, perm, d->k, P, d->H / 128, x_sorted_scales, st),
                  "gather launch");
    } else {
      MOE_TRY_HIP(launch_gather_rows(x, perm, d->k, P, (int64_t)d->H * elt_bytes(d->act_dtype), x_sorted, st),
                  "gather launch");
    }
  }
  return MOE_OK;
}

moe_status moe_expert_gate_up_swiglu(const moe_desc* d, const void* x_sorted, const float* x_scales,
                                     const int32_t* offsets, const void* w_gate, const void* w_up,
                                     const void* w_gate_scales, const void* w_up_scales, void* h,
                                     float* h_scales, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  g_chain = nullptr;
  moe_status s = validate(d);
  if (s != MOE_OK) return s;
  if (pairs(d) == 0) return MOE_OK;
  if (!x_sorted || !offsets || !w_gate || (!w_up && !packed(d)) || !h) return fail(MOE_EINVAL, "NULL tensor argument");
  if (is_fp8(d) && (!x_scales || !w_gate_scales || !w_up_scales || !h_scales))
    return fail(MOE_EINVAL, "fp8 experts need x_scales, weight scales and h_scales");
  if (!aligned16(x_sorted) || !aligned16(w_gate) || (!packed(d) && !aligned16(w_up)) || !aligned16(h))
    return fail(MOE_EINVAL, "tensors must be 16-byte aligned");
  if ((s = check_ws(d, MOE_OP_GATE_UP, ws, ws_bytes)) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  Schedule* sched = nullptr;
  if (d->w_dtype != MOE_DT_F32) {
    sched = (Schedule*)ws;
    MOE_TRY_HIP(launch_schedule(offsets, d->E, sched_req(sched, d, gate_up_ntiles(d)), st), "schedule launch");
  }
  float* partial = sched ? (float*)((uint8_t*)ws + align_up(sched_bytes(sched_capacity(d, gate_up_ntiles(d))))) : nullptr;
  return run_gate_up(d, x_sorted, x_scales, nullptr, offsets, w_gate, w_up, w_gate_scales, w_up_scales, h,
                     h_scales, sched, partial, st);
}

moe_status moe_expert_down(const moe_desc* d, const void* h, const float* h_scales, const int32_t* offsets,
                           const void* w_down, const void* w_down_scales, void* y_sorted, void* ws,
                           size_t ws_bytes, void* stream) {
  g_err.clear();
  g_chain = nullptr;
  moe_status s = validate(d);
  if (s != MOE_OK) return s;
  if (pairs(d) == 0) return MOE_OK;
  if (!h || !offsets || !w_down || !y_sorted) return fail(MOE_EINVAL, "NULL tensor argument");
  if (is_fp8(d) && (!h_scales || !w_down_scales)) return fail(MOE_EINVAL, "fp8 experts need h_scales and w_down_scales");
  if (!aligned16(h) || !aligned16(w_down) || !aligned16(y_sorted))
    return fail(MOE_EINVAL, "tensors must be 16-byte aligned");
  if ((s = check_ws(d, MOE_OP_DOWN, ws, ws_bytes)) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  Schedule* sched = nullptr;
  if (d->w_dtype != MOE_DT_F32) {
    sched = (Schedule*)ws;
    MOE_TRY_HIP(launch_schedule(offsets, d->E, sched_req(sched, d, down_ntiles(d)), st), "schedule launch");
  }
  float* partial = sched ? (float*)((uint8_t*)ws + align_up(sched_bytes(sched_capacity(d, down_ntiles(d))))) : nullptr;
  return run_down(d, h, h_scales, offsets, w_down, w_down_scales, y_sorted, sched, partial, st);
}

moe_status moe_unpermute_combine(const moe_desc* d, const void* y_sorted, const int32_t* inv,
                                 const float* topk_w, void* out, void* stream) {
  g_err.clear();
  g_chain = nullptr;
  moe_status s = validate(d);
  if (s != MOE_OK) return s;
  if (d->T == 0) return MOE_OK;
  if (!y_sorted || !inv || !topk_w || !out) return fail(MOE_EINVAL, "NULL tensor argument");
  if (!aligned16(y_sorted) || !aligned16(out)) return fail(MOE_EINVAL, "tensors must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  StageTimer tm(MOE_STAGE_COMBINE, st);
  MOE_TRY_HIP(launch_combine(y_sorted, d->y_dtype == MOE_DT_F32, inv, topk_w, d->T, d->k, d->H, out,
                             d->act_dtype == MOE_DT_F32, st),
              "combine launch");
  return MOE_OK;
}

// The fused forward on a workspace of at least ws_size(d, MOE_OP_FORWARD)
// bytes (moe_forward: the caller's; moe_forward_static: the static scratch).
static moe_status forward_impl(const moe_desc* d, const void* x, const void* w_router, const float* bias,
                        const void* w_gate, const void* w_up, const void* w_down, const void* sg,
                        const void* su, const void* sd, void* out, int32_t* ids_out, float* w_out,
                        int32_t* counts_out, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  g_chain = nullptr;
  moe_status s = validate(d);
  if (s != MOE_OK) return s;
  if ((s = check_ws(d, MOE_OP_FORWARD, ws, ws_bytes)) != MOE_OK) return s;
  if (d->T > 0) {
    if (!x || !w_router || !w_gate || (!w_up && !packed(d)) || !w_down || !out)
      return fail(MOE_EINVAL, "NULL tensor argument");
    if (is_fp8(d) && (!sg || !su || !sd)) return fail(MOE_EINVAL, "fp8 experts need all three block-scale tensors");
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || (!packed(d) && !aligned16(w_up)) ||
        !aligned16(w_down) || !aligned16(out))
      return fail(MOE_EINVAL, "tensors must be 16-byte aligned");
  }
  hipStream_t st = (hipStream_t)stream;
  Carve c{(uint8_t*)ws};
  ForwardWs fw = carve_forward(c, d);
  int32_t* ids = ids_out ? ids_out : fw.ids;
  float* w = w_out ? w_out : fw.w;
  int32_t* counts = counts_out ? counts_out : fw.counts;
  const int64_t P = pairs(d);

  SchedRequest sgu{}, sdn{};
  if (d->w_dtype != MOE_DT_F32) {
    sgu = sched_req(fw.sched_gu, d, gate_up_ntiles(d));
    sdn = sched_req(fw.sched_dn, d, down_ntiles(d));
  }
  // weight streaming: the schedules hold one entry per touched expert and
  // the GEMMs derive their items from them (the one-workgroup permutation
  // launch wrote every item before: dsv3_fp8 T=64, 4884 items, 14.1 -> 9.9 us)
  const bool per_expert = use_stream(d);
  if (per_expert) sgu.implicit_items = sdn.implicit_items = true;
  // small bf16 batches: the top-k selection runs in the one-workgroup
  // permutation launch, right after the logits
  const bool select_in_permute = d->act_dtype == MOE_DT_BF16 && d->T > 0 && d->T <= kSelectPermuteMaxT &&
                                 !route_big(d->T, d->H) && P <= kPermChunk;
  if (select_in_permute) {
    {
      StageTimer tm(MOE_STAGE_ROUTE, st);
      MOE_TRY_HIP(launch_route_logits(x, w_router, d->T, d->H, d->E, fw.route_part, st), "router launch");
    }
    StageTimer tm(MOE_STAGE_SCAN, st);
    MOE_TRY_HIP(launch_select_permute_small(fw.route_part, route_slices(d->T, d->H, d->E), d->T, d->E, bias, d->k,
                                            d->score, d->renormalize, d->routed_scale, ids, w, counts, fw.offsets,
                                            fw.perm, fw.inv, fw.touched, sgu, sdn, st),
                "selection and permute launch");
  } else {
    if (d->T > 0) {
      StageTimer tm(MOE_STAGE_ROUTE, st);
      MOE_TRY_HIP(launch_route_topk(x, w_router, bias, d->T, d->H, d->E, d->k, d->act_dtype == MOE_DT_BF16,
                                    d->score, d->renormalize, d->routed_scale, ids, w, fw.route_part, st),
                  "router launch");
    }
    if ((s = run_permute(d, ids, counts, fw.offsets, fw.perm, fw.inv, fw.touched, fw.pw, sgu, sdn, st)) != MOE_OK)
      return s;
  }
  if (P == 0) return MOE_OK;
  const void* act = x;
  const float* act_scales = nullptr;
  if (is_fp8(d)) {
    StageTimer tm(MOE_STAGE_QUANT_X, st);
    MOE_TRY_HIP(launch_quant_rows_fp8((const uint16_t*)x, d->T, d->H, fw.pw.xq, fw.pw.xs, st), "quantize launch");
    act = fw.pw.xq;
    act_scales = fw.pw.xs;
  }
  if ((s = run_gate_up(d, act, act_scales, fw.perm, fw.offsets, w_gate, w_up, sg, su, fw.h, fw.hs, fw.sched_gu, fw.partial,
                       st, per_expert)) != MOE_OK)
    return s;
  // Weight streaming: the down launch's reduction launch is left out and the
  // combine reads y, or sums the partial tiles of a split launch, when
  //  - the batch is small enough for the combine's fine decomposition (one
  //    workgroup per token and 32 channels reads the partials in parallel), or
  //  - even the most items the batch can touch leave the down launch unsplit
  //    (then a split is rare, and a combine workgroup per token and 2048
  //    channels sums the partials).
  const int64_t dn_items_max = std::min<int64_t>(d->E, P) * down_ntiles(d);
  if (use_stream(d) &&
      ((d->T <= kCombineFineMaxT && d->H % 32 == 0) ||
       stream_splits((int)std::min<int64_t>(dn_items_max, 1 << 30), stream_ksteps(wfmt(d), d->I),
                     stream_slots(wfmt(d), d->T <= 32)) == 1)) {
    if ((s = run_down(d, fw.h, fw.hs, fw.offsets, w_down, sd, fw.y, fw.sched_dn, fw.partial, st, fw.rowinfo,
                      per_expert)) != MOE_OK)
      return s;
    StageTimer tm(MOE_STAGE_COMBINE, st);
    MOE_TRY_HIP(launch_combine_stream(fw.y, d->y_dtype == MOE_DT_F32, fw.partial, fw.rowinfo, fw.sched_dn,
                                      stream_ksteps(wfmt(d), d->I), stream_slots(wfmt(d), d->T <= 32), fw.inv, w,
                                      d->T, d->k, d->H, out, d->act_dtype == MOE_DT_F32, st),
                "combine launch");
    return MOE_OK;
  }
  if ((s = run_down(d, fw.h, fw.hs, fw.offsets, w_down, sd, fw.y, fw.sched_dn, fw.partial, st, nullptr,
                    per_expert)) != MOE_OK)
    return s;
  {
    StageTimer tm(MOE_STAGE_COMBINE, st);
    MOE_TRY_HIP(launch_combine(fw.y, d->y_dtype == MOE_DT_F32, fw.inv, w, d->T, d->k, d->H, out,
                               d->act_dtype == MOE_DT_F32, st),
                "combine launch");
  }
  return MOE_OK;
}

moe_status moe_forward(const moe_desc* d, const void* x, const void* w_router, const float* bias,
                       const void* w_gate, const void* w_up, const void* w_down, const void* sg,
                       const void* su, const void* sd, void* out, int32_t* ids_out, float* w_out,
                       int32_t* counts_out, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(d, x, w_router, bias, w_gate, w_up, w_down, sg, su, sd, out, ids_out, w_out, counts_out, ws,
                      ws_bytes, stream);
}

moe_status moe_forward_static(const moe_desc* d, const void* x, const void* w_router, const float* bias,
                              const void* w_gate, const void* w_up, const void* w_down, const void* sg,
                              const void* su, const void* sd, void* out, int32_t* ids_out, float* w_out,
                              int32_t* counts_out, void* stream) {
  g_err.clear();
  g_chain = nullptr;
  moe_status s = validate(d);
  if (s != MOE_OK) return s;
  const size_t need = ws_size(d, MOE_OP_FORWARD);
  if (need > kStaticScratchBytes)
    return fail(MOE_EWORKSPACE,
                "moe_forward_static: this layer needs %zu bytes of scratch, more than the %zu bytes of the static "
                "scratch (use moe_forward with a caller workspace)",
                need, kStaticScratchBytes);
  void* scratch_ptr = nullptr;
  if ((s = static_scratch((hipStream_t)stream, &scratch_ptr)) != MOE_OK) return s;
  g_no_events = true;
  s = forward_impl(d, x, w_router, bias, w_gate, w_up, w_down, sg, su, sd, out, ids_out, w_out, counts_out,
                   scratch_ptr, kStaticScratchBytes, stream);
  g_no_events = false;
  return s;
}

moe_status moe_backward(const moe_desc* d0, const void* x, const void* w_router, const float* bias,
                        const void* w_gate, const void* w_up, const void* w_down, const void* d_out, void* dx,
                        void* dw_router, float* d_bias, void* dw_gate, void* dw_up, void* dw_down, void* ws,
                        size_t ws_bytes, void* stream) {
  g_err.clear();
  g_chain = nullptr;
  moe_status s = validate_backward(d0);
  if (s != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if (d0->T == 0) {
    // no token: every parameter gradient is zero
    if (!dw_router || !dw_gate || !dw_up || !dw_down) return fail(MOE_EINVAL, "NULL gradient output");
    const int64_t HI = (int64_t)d0->H * d0->I * d0->E * 2;
    MOE_TRY_HIP(launch_fill_zero(dw_gate, HI, st), "zero-fill launch");
    MOE_TRY_HIP(launch_fill_zero(dw_up, HI, st), "zero-fill launch");
    MOE_TRY_HIP(launch_fill_zero(dw_down, HI, st), "zero-fill launch");
    MOE_TRY_HIP(launch_fill_zero(dw_router, (int64_t)d0->E * d0->H * 2, st), "zero-fill launch");
    if (d_bias) MOE_TRY_HIP(launch_fill_zero(d_bias, (int64_t)d0->E * 4, st), "zero-fill launch");
    return MOE_OK;
  }
  if ((s = check_ws(d0, MOE_OP_BACKWARD, ws, ws_bytes)) != MOE_OK) return s;
  const void* ptrs[] = {x, w_router, w_gate, w_up, w_down, d_out, dx, dw_router, dw_gate, dw_up, dw_down};
  for (const void* p : ptrs) {
    if (!p) return fail(MOE_EINVAL, "NULL tensor argument");
    if (!aligned16(p)) return fail(MOE_EINVAL, "tensors must be 16-byte aligned");
  }
  const moe_desc bd = backward_desc(d0);
  const moe_desc* d = &bd;
  Carve c{(uint8_t*)ws};
  BackwardWs bw = carve_backward(c, d);
  const int64_t P = pairs(d);
  const int H = d->H, I = d->I, E = d->E, Epad = expert_pad(d->E);

  MOE_TRY_HIP(launch_fill_zero(bw.zeros, 256, st), "zero-fill launch");
  {
    StageTimer tm(MOE_STAGE_ROUTE, st);
    MOE_TRY_HIP(launch_route_topk(x, w_router, bias, d->T, H, E, d->k, 1, d->score, d->renormalize,
                                  d->routed_scale, bw.ids, bw.w, bw.route_part, st),
                "router launch");
  }
  const SchedRequest sgu = sched_req(bw.sched_gu, d, gate_up_ntiles(d));
  const SchedRequest se = bwd_sched_req(bw.sched_e, d, bwd_tiles(I));
  const SchedRequest sdx = bwd_sched_req(bw.sched_dx, d, bwd_tiles(H));
  if ((s = run_permute(d, bw.ids, bw.counts, bw.offsets, bw.perm, bw.inv, bw.touched, bw.pw, sgu, se, st)) != MOE_OK)
    return s;
  {
    StageTimer tm(MOE_STAGE_BWD_MISC, st);
    MOE_TRY_HIP(launch_schedule(bw.offsets, E, sdx, st), "schedule launch");
    MOE_TRY_HIP(launch_gather_rows(x, bw.perm, d->k, P, (int64_t)H * 2, bw.x_sorted, st), "gather launch");
    MOE_TRY_HIP(launch_gather_rows(d_out, bw.perm, d->k, P, (int64_t)H * 2, bw.dout_sorted, st), "gather launch");
  }
  {
    // g and u of every sorted row, recomputed
    StageTimer tm(MOE_STAGE_BWD_RECOMPUTE, st);
    GemmArgs a = gemm_common(d);
    a.act = bw.x_sorted;
    a.w0 = w_gate;
    a.w1 = w_up;
    a.K = H;
    a.N = I;
    a.out = bw.gu;
    a.gu_out = 1;
    a.sched = bw.sched_gu;
    a.offsets = bw.offsets;
    MOE_TRY_HIP(launch_gate_up_bf16(a, grid_for(sgu.capacity), st), "gate/up recompute launch");
  }
  {
    // e = W_down^T dout per sorted row
    StageTimer tm(MOE_STAGE_BWD_DATA, st);
    BwdGemmArgs g{};
    g.a = (const uint16_t*)w_down;
    g.lda = I;
    g.a_gs = (int64_t)H * I;
    g.a_split = g.a_krows = H;
    g.b = bw.dout_sorted;
    g.ldb = H;
    g.zeros = bw.zeros;
    g.M = I;
    g.K = H;
    g.sched = bw.sched_e;
    g.out = bw.ev;
    g.ldo = I;
    g.out_f32 = 1;
    MOE_TRY_HIP(launch_gemm_bwd(g, 0, 0, grid_for(se.capacity), st), "backward GEMM launch");
  }
  {
    StageTimer tm(MOE_STAGE_BWD_MISC, st);
    MOE_TRY_HIP(launch_swiglu_bwd(bw.ev, bw.gu, bw.perm, bw.w, P, I, d->gate_act, bw.dw, bw.ap, bw.dgu, st),
                "gated-activation backward launch");
  }
  {
    // dx of every sorted row: [dg | du] . [W_gate ; W_up]
    StageTimer tm(MOE_STAGE_BWD_DATA, st);
    BwdGemmArgs g{};
    g.a = (const uint16_t*)w_gate;
    g.a2 = (const uint16_t*)w_up;
    g.lda = H;
    g.a_gs = (int64_t)I * H;
    g.a_split = I;
    g.a_krows = 2 * I;
    g.b = bw.dgu;
    g.ldb = 2 * I;
    g.zeros = bw.zeros;
    g.M = H;
    g.K = 2 * I;
    g.sched = bw.sched_dx;
    g.out = bw.dxp;
    g.ldo = H;
    g.out_f32 = 1;
    MOE_TRY_HIP(launch_gemm_bwd(g, 0, 0, grid_for(sdx.capacity), st), "backward GEMM launch");
  }
  {
    // dW_down[e] = sum over the expert's rows of dout (w a)^T
    StageTimer tm(MOE_STAGE_BWD_WEIGHT, st);
    BwdGemmArgs g{};
    g.a = bw.ap;
    g.lda = I;
    g.b = bw.dout_sorted;
    g.ldb = H;
    g.zeros = bw.zeros;
    g.M = I;
    g.n_total = g.n_valid = H;
    g.offsets = bw.offsets;
    g.out = dw_down;
    g.ldo = I;
    g.o_gs = (int64_t)H * I;
    MOE_TRY_HIP(launch_gemm_bwd(g, 1, 0, E * bwd_tiles(I) * bwd_tiles(H), st), "backward GEMM launch");
  }
  {
    // dW_gate[e], dW_up[e] = sum over the expert's rows of [dg | du] x^T
    StageTimer tm(MOE_STAGE_BWD_WEIGHT, st);
    BwdGemmArgs g{};
    g.a = bw.x_sorted;
    g.lda = H;
    g.b = bw.dgu;
    g.ldb = 2 * I;
    g.zeros = bw.zeros;
    g.M = H;
    g.n_total = g.n_valid = 2 * I;
    g.offsets = bw.offsets;
    g.out = dw_gate;
    g.out2 = dw_up;
    g.n_split = I;
    g.ldo = H;
    g.o_gs = (int64_t)I * H;
    MOE_TRY_HIP(launch_gemm_bwd(g, 1, 0, E * bwd_tiles(H) * bwd_tiles(2 * I), st), "backward GEMM launch");
  }
  {
    // router: key gradients, dW_r = dkey^T x, dbias, and dkey . W_r into dx
    StageTimer tm(MOE_STAGE_BWD_ROUTER, st);
    MOE_TRY_HIP(launch_router_bwd(bw.route_part, route_slices(d->T, H, E), d->T, E, Epad, bias, bw.ids, bw.dw,
                                  d->k, d->score, d->renormalize, d->routed_scale, bw.dkey, bw.dkey_b, st),
                "router backward launch");
    if (d_bias) MOE_TRY_HIP(launch_bias_grad(bw.dkey, d->T, E, d_bias, st), "bias gradient launch");
    int kc = 0;
    const int chunks = router_chunks(d, &kc);
    BwdGemmArgs g{};
    g.a = (const uint16_t*)x;
    g.lda = H;
    g.b = bw.dkey_b;
    g.ldb = Epad;
    g.zeros = bw.zeros;
    g.M = H;
    g.K = (int)d->T;
    g.k_chunk = kc;
    g.n_total = Epad;
    g.n_valid = E;
    g.out = bw.dwr_part;
    g.ldo = H;
    g.o_gs = (int64_t)E * H;
    g.out_f32 = 1;
    MOE_TRY_HIP(launch_gemm_bwd(g, 1, 1, chunks * bwd_tiles(H) * bwd_tiles(Epad), st), "backward GEMM launch");
    MOE_TRY_HIP(launch_chunk_sum(bw.dwr_part, chunks, (int64_t)E * H, (uint16_t*)dw_router, st), "sum launch");
    g = BwdGemmArgs{};
    g.a = (const uint16_t*)w_router;
    g.lda = H;
    g.a_split = g.a_krows = E;
    g.b = bw.dkey_b;
    g.ldb = Epad;
    g.zeros = bw.zeros;
    g.M = H;
    g.K = Epad;
    g.n_total = (int)d->T;
    g.out = bw.dxr;
    g.ldo = H;
    g.out_f32 = 1;
    MOE_TRY_HIP(launch_gemm_bwd(g, 0, 1, bwd_tiles(d->T) * bwd_tiles(H), st), "backward GEMM launch");
  }
  {
    StageTimer tm(MOE_STAGE_BWD_MISC, st);
    MOE_TRY_HIP(launch_dx_combine(bw.dxp, bw.dxr, bw.inv, d->T, d->k, H, (uint16_t*)dx, st), "dx combine launch");
  }
  return MOE_OK;
}

size_t moe_packed_weight_bytes(const moe_desc* d, int which) {
  if (validate(d) != MOE_OK || d->w_dtype == MOE_DT_F32) return 0;
  if (which != MOE_PACK_GATE_UP && which != MOE_PACK_DOWN) return 0;
  return packed_bytes(d, which);
}

moe_status moe_pack_weights(const moe_desc* d, int which, const void* w0, const void* w1, void* dst,
                            void* stream) {
  g_err.clear();
  g_chain = nullptr;
  moe_status s = validate(d);
  if (s != MOE_OK) return s;
  if (d->w_dtype == MOE_DT_F32) return fail(MOE_EUNSUPPORTED, "packed weights are bf16 or fp8");
  if (which != MOE_PACK_GATE_UP && which != MOE_PACK_DOWN) return fail(MOE_EINVAL, "which = %d", which);
  const int gate_up = which == MOE_PACK_GATE_UP;
  if (!w0 || !dst || (gate_up && !w1)) return fail(MOE_EINVAL, "NULL tensor argument");
  if (!aligned16(w0) || (gate_up && !aligned16(w1)) || ((uintptr_t)dst & (kAlign - 1)))
    return fail(MOE_EINVAL, "weights must be 16-byte and dst 256-byte aligned");
  const int N = gate_up ? d->I : d->H;
  const int64_t row_bytes = w_row_bytes(d->w_dtype, gate_up ? d->H : d->I);
  MOE_TRY_HIP(launch_pack(w0, w1, gate_up, d->E, N, row_bytes, dst, (hipStream_t)stream), "pack launch");
  return MOE_OK;
}

moe_status moe_timing_enable(int on) {
  g_timing = on != 0;
  return MOE_OK;
}

moe_status moe_timing_read(double* ms, int64_t* launches) {
  if (!ms || !launches) return fail(MOE_EINVAL, "NULL output");
  for (int i = 0; i < MOE_NUM_STAGES; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  moe_status result = MOE_OK;
  for (auto& p : g_pending) {
    float t = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&t, p.start, p.stop) != hipSuccess)
      result = fail(MOE_EHIP, "event timing failed");
    ms[p.stage] += t;
    launches[p.stage] += 1;
  }
  // chained launches share events: return each one to the pool once
  std::vector<hipEvent_t> used;
  for (auto& p : g_pending) {
    used.push_back(p.start);
    used.push_back(p.stop);
  }
  std::sort(used.begin(), used.end());
  used.erase(std::unique(used.begin(), used.end()), used.end());
  for (hipEvent_t e : used) g_event_pool.push_back(e);
  g_pending.clear();
  g_chain = nullptr;
  return result;
}

}  // extern "C"
