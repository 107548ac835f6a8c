// C ABI of the Beam MoE block: argument validation, workspace carving and
// kernel launches on the caller's stream.  The operations and conventions are
// stated in include/beam_moe.h.
#include "../../include/beam_moe.h"

#include <hip/hip_runtime.h>

#include <array>
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>
#include <vector>

namespace beam {
struct Tile;
hipError_t launch_router_logits(const uint16_t* x, const float* wr, float* part, int T, int H, int E, int splits,
                                int k_per_split, hipStream_t st);
hipError_t launch_select(const float* src, int splits, bool from_partials, const float* bias,
                         const float* select_bias, float* scores_out, int T, int E, int G, int TG, int K, float scale,
                         int32_t* ids, float* w, hipStream_t st);
int dispatch_units(int n);
hipError_t launch_dispatch(const int32_t* ids, int n, int E, int32_t* unit_hist, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_slots, Tile* tiles, int mt, int32_t* ntiles, hipStream_t st);
int scale_cols();
bool stream_fits(int H, int I, int R);
hipError_t launch_gateup_stream(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                                int max_tiles, int R, const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                                uint8_t* hscale, int H, int I, int K, hipStream_t st);
hipError_t launch_down_stream(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                              const int32_t* ntiles, int max_tiles, int R, const uint16_t* wd, bool wd_f16,
                              uint16_t* y16, uint8_t* yscale, int H, int I, hipStream_t st);
hipError_t launch_pack_f16(const uint16_t* src, uint16_t* dst, size_t n, hipStream_t st);
hipError_t launch_combine(const uint16_t* y16, const uint8_t* yscale, const float* w, float* out, int T, int H, int K,
                          hipStream_t st);
bool stream_fp8_fits(int H, int I, int R);
hipError_t launch_gateup_stream_fp8(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                                    int max_tiles, int R, const uint8_t* wg, const uint8_t* wu, const float* sg,
                                    const float* su, uint16_t* h, uint8_t* hscale, int H, int I, int K,
                                    hipStream_t st);
hipError_t launch_down_stream_fp8(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                                  const int32_t* ntiles, int max_tiles, int R, const uint8_t* wd, const float* sd,
                                  uint16_t* y16, uint8_t* yscale, int H, int I, hipStream_t st);
hipError_t launch_gateup_grouped_fp8(const uint16_t* x, const int32_t* slots, const Tile* tiles,
                                     const int32_t* ntiles, int max_tiles, const uint8_t* wg, const uint8_t* wu,
                                     const float* sg, const float* su, uint16_t* h, uint8_t* hscale, int H, int I,
                                     int K, hipStream_t st);
hipError_t launch_down_grouped_fp8(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                                   const int32_t* ntiles, int max_tiles, const uint8_t* wd, const float* sd,
                                   uint16_t* y16, uint8_t* yscale, int H, int I, hipStream_t st);
int grouped_gemm_rows();
bool residual_fits(int H);
hipError_t launch_prenorm(const float* stream, const float* g_in, uint16_t* x, int T, int H, float eps,
                          hipStream_t st);
hipError_t launch_combine_residual(const uint16_t* y16, const uint8_t* yscale, const float* w, const float* stream_in,
                                   const float* g_out, float* stream_out, int T, int H, int K, int step, float eps,
                                   hipStream_t st);
hipError_t launch_gateup_grouped(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                                 int max_tiles, const uint16_t* wg, const uint16_t* wu, uint16_t* h, uint8_t* hscale,
                                 int H, int I, int K, hipStream_t st);
hipError_t launch_down_grouped(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                               const int32_t* ntiles, int max_tiles, const uint16_t* wd, bool wd_f16, uint16_t* y16,
                               uint8_t* yscale, int H, int I, hipStream_t st);
}  // namespace beam

namespace {

constexpr size_t kAlign = 256;
constexpr int kTileBytes = 32;          // sizeof(beam::Tile)
constexpr int64_t kMaxPairs = 1 << 28;  // T * K limit

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool dims_ok(const beam_moe_dims* d) {
  if (!d) return false;
  const int E = d->num_experts, G = d->num_groups, TG = d->topk_groups, K = d->topk;
  if (E < 1 || E > 256 || G < 1 || G > 64 || E % G != 0) return false;
  if (TG < 1 || TG > G) return false;
  const int cand = TG * (E / G);
  if (K < 1 || K > 16 || K > cand) return false;
  if (d->hidden < 256 || d->hidden % 256 != 0) return false;
  if (d->intermediate < 128 || d->intermediate % 128 != 0 || d->intermediate > 32768) return false;
  if (!std::isfinite(d->routed_scaling)) return false;
  return true;
}

// Expert-path choice.  The stream kernels take tiles of at most R rows and
// stream an expert's weights once per tile; R is the smallest of 8, 16, 32 and
// 64 that is at least twice the average rows per expert, so nearly every expert
// has one tile.  Above 32 rows per expert on average the grouped GEMMs take the
// batch: they read an expert's weights once per 256-row tile at MFMA-bound
// rates.  Returns R, or 0 for the grouped GEMMs.
int stream_rows(const beam_moe_dims* d, int T, bool fp8 = false) {
  const double avg = (double)T * d->topk / d->num_experts;
  for (int R = 8; R <= 64; R *= 2)
    if (avg * 2.0 <= R)
      return (fp8 ? beam::stream_fp8_fits(d->hidden, d->intermediate, R)
                  : beam::stream_fits(d->hidden, d->intermediate, R))
                 ? R
                 : 0;
  return 0;
}

struct Plan {
  int T, H, I, E, K, n;
  // router
  int splits, k_per_split;
  size_t off_part;
  // dispatch
  int units;
  size_t off_hist;
  // expert tiles
  bool stream;
  int rows;  // stream path: rows per tile
  // one tile table serves both projections: tiles of at most `rows` rows
  // (stream path) or the grouped GEMMs' 256-row tiles; each down kernel reads
  // the activation scales of the gate/up tile its rows belong to
  int mt, max_tiles;
  size_t off_tiles, off_ntiles;
  // activations
  size_t off_h, off_hscale, off_y, off_yscale;
  size_t off_x;  // bf16 [T, H]: the block's input, written by beam_moe_residual_forward
  size_t total;
};

// fp8: the FP8-weight expert kernels (stream or grouped by the same rule).
void make_plan(const beam_moe_dims* d, int T, Plan* p, bool fp8 = false) {
  p->T = T;
  p->H = d->hidden;
  p->I = d->intermediate;
  p->E = d->num_experts;
  p->K = d->topk;
  p->n = T * d->topk;
  const int ksteps = p->H / 32;
  int rtiles = ((T + 63) / 64) * ((p->E + 63) / 64);
  if (rtiles < 1) rtiles = 1;
  int splits = (256 + rtiles - 1) / rtiles;
  if (splits > ksteps) splits = ksteps;
  if (splits > 16) splits = 16;
  if (splits < 1) splits = 1;
  const int steps_per = (ksteps + splits - 1) / splits;
  p->k_per_split = steps_per * 32;
  p->splits = (ksteps + steps_per - 1) / steps_per;
  p->units = beam::dispatch_units(p->n);
  p->rows = stream_rows(d, T, fp8);
  p->stream = p->rows > 0;
  const int touched = p->E < p->n ? p->E : p->n;  // most experts with rows
  p->mt = p->stream ? p->rows : beam::grouped_gemm_rows();
  p->max_tiles = p->n / p->mt + touched;
  size_t off = 0;
  p->off_part = off;
  off = align_up(off + (size_t)p->splits * T * p->E * sizeof(float));
  p->off_hist = off;
  off = align_up(off + (size_t)p->units * p->E * sizeof(int32_t));
  p->off_tiles = off;
  off = align_up(off + (size_t)(p->max_tiles + 1) * kTileBytes);
  p->off_ntiles = off;
  off = align_up(off + sizeof(int32_t));
  p->off_h = off;
  off = align_up(off + (size_t)p->n * p->I * 2);
  p->off_hscale = off;
  off = align_up(off + (size_t)p->n * (p->I / beam::scale_cols()));
  p->off_y = off;
  off = align_up(off + (size_t)p->n * p->H * 2);
  p->off_yscale = off;
  off = align_up(off + (size_t)p->n * (p->H / beam::scale_cols()));
  p->off_x = off;
  off = align_up(off + (size_t)T * p->H * 2);
  p->total = off;
}

// Scratch of the standalone route (split-K partial logits) and dispatch (unit
// histograms) calls; the forward plan holds both inside its own layout.
size_t route_ws_bytes(const Plan& p) { return (size_t)p.splits * p.T * p.E * sizeof(float); }
size_t dispatch_ws_bytes(const Plan& p) { return (size_t)p.units * p.E * sizeof(int32_t); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename Tp>
Tp* at(void* ws, size_t off) {
  return reinterpret_cast<Tp*>(static_cast<char*>(ws) + off);
}

int check_common(const beam_moe_dims* d, int32_t T) {
  if (!d) return BEAM_MOE_ERR_INVALID_ARG;
  if (!dims_ok(d)) return BEAM_MOE_ERR_UNSUPPORTED;
  if (T < 0) return BEAM_MOE_ERR_INVALID_ARG;
  if ((int64_t)T * d->topk > kMaxPairs) return BEAM_MOE_ERR_UNSUPPORTED;
  return BEAM_MOE_OK;
}

int check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return BEAM_MOE_ERR_INVALID_ARG;
  return BEAM_MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? BEAM_MOE_OK : BEAM_MOE_ERR_HIP; }

// ---------------------------------------------------------------------------
// stage timing (diagnostics)
// ---------------------------------------------------------------------------
enum Stage { kStPrenorm = 0, kStRouter, kStSelect, kStDispatch, kStGateUp, kStDown, kStCombine, kNumStages };
const char* const kStageNames[kNumStages] = {"prenorm", "router_logits", "select", "dispatch",
                                             "gate_up", "down", "combine"};

struct Timing {
  std::mutex mu;
  bool enabled = false;
  std::vector<std::array<hipEvent_t, kNumStages + 1>> slots;
  size_t used = 0;
};
Timing& timing() {
  static Timing t;
  return t;
}

// Events of the current forward call, or nullptr when timing is off.
hipEvent_t* timing_slot() {
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  if (!t.enabled) return nullptr;
  if (t.used == t.slots.size()) {
    std::array<hipEvent_t, kNumStages + 1> ev{};
    for (auto& e : ev)
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
    t.slots.push_back(ev);
  }
  return t.slots[t.used++].data();
}

hipError_t mark(hipEvent_t* ev, int i, hipStream_t st) { return ev ? hipEventRecord(ev[i], st) : hipSuccess; }


// Inputs and by-product outputs of one pass of the block.
struct BlockArgs {
  const uint16_t* x;
  const float* w_router;
  const float* logit_bias;
  const float* select_bias;
  const uint16_t* wg;  // bf16 experts (null for FP8 ones)
  const uint16_t* wu;
  const uint16_t* wd;
  bool wd_f16;  // wd holds fp16 weights (beam_moe_pack_weights), not bf16
  const uint8_t* qg;  // FP8 experts: E4M3 codes and per-row scales (null for bf16 ones)
  const uint8_t* qu;
  const uint8_t* qd;
  const float* sg;
  const float* su;
  const float* sd;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* sorted_slots;
};

// The block's arguments with bf16 experts, or with FP8 ones (codes and row
// scales); x may be filled in later (the residual entry points' pre-norm).
BlockArgs bf16_block(const void* x, const float* w_router, const float* logit_bias, const float* select_bias,
                     const void* w_gate, const void* w_up, const void* w_down, int32_t* topk_ids, float* topk_w,
                     int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots) {
  BlockArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w_router = w_router;
  a.logit_bias = logit_bias;
  a.select_bias = select_bias;
  a.wg = static_cast<const uint16_t*>(w_gate);
  a.wu = static_cast<const uint16_t*>(w_up);
  a.wd = static_cast<const uint16_t*>(w_down);
  a.topk_ids = topk_ids;
  a.topk_w = topk_w;
  a.expert_counts = expert_counts;
  a.expert_offsets = expert_offsets;
  a.sorted_slots = sorted_slots;
  return a;
}

BlockArgs fp8_block(const void* x, const float* w_router, const float* logit_bias, const float* select_bias,
                    const uint8_t* w_gate, const float* gate_scale, const uint8_t* w_up, const float* up_scale,
                    const uint8_t* w_down, const float* down_scale, int32_t* topk_ids, float* topk_w,
                    int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots) {
  BlockArgs a = bf16_block(x, w_router, logit_bias, select_bias, nullptr, nullptr, nullptr, topk_ids, topk_w,
                           expert_counts, expert_offsets, sorted_slots);
  a.qg = w_gate;
  a.qu = w_up;
  a.qd = w_down;
  a.sg = gate_scale;
  a.su = up_scale;
  a.sd = down_scale;
  return a;
}

// `pre()` (whatever produces the block's input; nothing for beam_moe_forward),
// then router, selection, dispatch and the expert projections on the caller's
// stream, then `combine(y16, yscale)` (the final step of the entry point).
template <typename PreFn, typename CombineFn>
int run_block(const beam_moe_dims* d, const Plan& p, const BlockArgs& a, void* ws, hipStream_t st, PreFn pre,
              CombineFn combine, bool timed = true) {
  const int T = p.T;
  float* part = at<float>(ws, p.off_part);
  beam::Tile* tiles = at<beam::Tile>(ws, p.off_tiles);
  int32_t* ntiles = at<int32_t>(ws, p.off_ntiles);
  uint16_t* h = at<uint16_t>(ws, p.off_h);
  uint8_t* hscale = at<uint8_t>(ws, p.off_hscale);
  uint16_t* y16 = at<uint16_t>(ws, p.off_y);
  uint8_t* yscale = at<uint8_t>(ws, p.off_yscale);
  hipEvent_t* ev = timed ? timing_slot() : nullptr;
  int rc = BEAM_MOE_OK;
#define BEAM_TRY(expr)                                     \
  do {                                                     \
    if ((rc = hip_status(expr)) != BEAM_MOE_OK) return rc; \
  } while (0)
  BEAM_TRY(mark(ev, kStPrenorm, st));
  BEAM_TRY(pre());
  BEAM_TRY(mark(ev, kStRouter, st));
  BEAM_TRY(beam::launch_router_logits(a.x, a.w_router, part, T, p.H, p.E, p.splits, p.k_per_split, st));
  BEAM_TRY(mark(ev, kStSelect, st));
  BEAM_TRY(beam::launch_select(part, p.splits, true, a.logit_bias, a.select_bias, nullptr, T, p.E, d->num_groups,
                               d->topk_groups, d->topk, d->routed_scaling, a.topk_ids, a.topk_w, st));
  BEAM_TRY(mark(ev, kStDispatch, st));
  BEAM_TRY(beam::launch_dispatch(a.topk_ids, p.n, p.E, at<int32_t>(ws, p.off_hist), a.expert_counts,
                                 a.expert_offsets, a.sorted_slots, tiles, p.mt, ntiles, st));
  BEAM_TRY(mark(ev, kStGateUp, st));
  if (a.qg && p.stream)
    BEAM_TRY(beam::launch_gateup_stream_fp8(a.x, a.sorted_slots, tiles, ntiles, p.max_tiles, p.rows, a.qg, a.qu,
                                            a.sg, a.su, h, hscale, p.H, p.I, p.K, st));
  else if (a.qg)
    BEAM_TRY(beam::launch_gateup_grouped_fp8(a.x, a.sorted_slots, tiles, ntiles, p.max_tiles, a.qg, a.qu, a.sg,
                                             a.su, h, hscale, p.H, p.I, p.K, st));
  else if (p.stream)
    BEAM_TRY(beam::launch_gateup_stream(a.x, a.sorted_slots, tiles, ntiles, p.max_tiles, p.rows, a.wg, a.wu, h,
                                        hscale, p.H, p.I, p.K, st));
  else
    BEAM_TRY(beam::launch_gateup_grouped(a.x, a.sorted_slots, tiles, ntiles, p.max_tiles, a.wg, a.wu, h, hscale,
                                         p.H, p.I, p.K, st));
  BEAM_TRY(mark(ev, kStDown, st));
  if (a.qd && p.stream)
    BEAM_TRY(beam::launch_down_stream_fp8(h, hscale, a.sorted_slots, tiles, ntiles, p.max_tiles, p.rows, a.qd, a.sd,
                                          y16, yscale, p.H, p.I, st));
  else if (a.qd)
    BEAM_TRY(beam::launch_down_grouped_fp8(h, hscale, a.sorted_slots, tiles, ntiles, p.max_tiles, a.qd, a.sd, y16,
                                           yscale, p.H, p.I, st));
  else if (p.stream)
    BEAM_TRY(beam::launch_down_stream(h, hscale, a.sorted_slots, tiles, ntiles, p.max_tiles, p.rows, a.wd,
                                      a.wd_f16, y16, yscale, p.H, p.I, st));
  else
    BEAM_TRY(beam::launch_down_grouped(h, hscale, a.sorted_slots, tiles, ntiles, p.max_tiles, a.wd, a.wd_f16, y16,
                                       yscale, p.H, p.I, st));
  BEAM_TRY(mark(ev, kStCombine, st));
  BEAM_TRY(combine(y16, yscale));
  BEAM_TRY(mark(ev, kNumStages, st));
#undef BEAM_TRY
  return BEAM_MOE_OK;
}

// The block as a residual sublayer: pre-norm of the stream into the workspace's
// x, the block (bf16 or FP8 experts as set in `a`, whose x is filled here), then
// the fused post-norm and stream update.  Weight pointers are checked by the caller.
int residual_block(const beam_moe_dims* d, int32_t T, const float* stream_in, int32_t step, const float* g_in,
                   const float* g_out, float eps, BlockArgs a, bool fp8, float* stream_out, void* ws,
                   size_t ws_bytes, void* stream) {
  if (!beam::residual_fits(d->hidden)) return BEAM_MOE_ERR_UNSUPPORTED;
  if (step < 2 || !std::isfinite(eps) || eps < 0.f) return BEAM_MOE_ERR_INVALID_ARG;
  if (T == 0) return BEAM_MOE_OK;
  int rc;
  if ((rc = check_ptrs({stream_in, a.w_router, stream_out, a.topk_ids, a.topk_w, a.expert_counts, a.expert_offsets,
                        a.sorted_slots})) != BEAM_MOE_OK)
    return rc;
  for (const float* opt : {a.logit_bias, a.select_bias, g_in, g_out})
    if (opt && !aligned16(opt)) return BEAM_MOE_ERR_INVALID_ARG;
  Plan p;
  make_plan(d, T, &p, fp8);
  if (!ws || !aligned16(ws) || ws_bytes < p.total) return BEAM_MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint16_t* x = at<uint16_t>(ws, p.off_x);
  a.x = x;
  const float* topk_w = a.topk_w;
  return run_block(
      d, p, a, ws, st, [&] { return beam::launch_prenorm(stream_in, g_in, x, T, p.H, eps, st); },
      [&](const uint16_t* y16, const uint8_t* yscale) {
        return beam::launch_combine_residual(y16, yscale, topk_w, stream_in, g_out, stream_out, T, p.H, p.K, step, eps,
                                             st);
      });
}

// Checks shared by beam_moe_forward and beam_moe_forward_noalloc (everything but
// the workspace); fills the plan.
int check_forward(const beam_moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                  const float* logit_bias, const float* select_bias, const void* w_gate, const void* w_up,
                  const void* w_down, float* out, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                  int32_t* expert_offsets, int32_t* sorted_slots, Plan* p) {
  int rc = check_common(d, T);
  if (rc != BEAM_MOE_OK || T == 0) return rc;
  if ((rc = check_ptrs({x_bf16, w_router, w_gate, w_up, w_down, out, topk_ids, topk_w, expert_counts,
                        expert_offsets, sorted_slots})) != BEAM_MOE_OK)
    return rc;
  if ((logit_bias && !aligned16(logit_bias)) || (select_bias && !aligned16(select_bias)))
    return BEAM_MOE_ERR_INVALID_ARG;
  make_plan(d, T, p);
  return BEAM_MOE_OK;
}

int forward_bf16(const beam_moe_dims* d, const Plan& p, const void* x_bf16, const float* w_router,
                 const float* logit_bias, const float* select_bias, const void* w_gate, const void* w_up,
                 const void* w_down, float* out, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                 int32_t* expert_offsets, int32_t* sorted_slots, void* ws, hipStream_t st, bool timed,
                 bool wd_f16 = false) {
  BlockArgs a = bf16_block(x_bf16, w_router, logit_bias, select_bias, w_gate, w_up, w_down, topk_ids, topk_w,
                           expert_counts, expert_offsets, sorted_slots);
  a.wd_f16 = wd_f16;
  return run_block(
      d, p, a, ws, st, [] { return hipSuccess; },
      [&](const uint16_t* y16, const uint8_t* yscale) {
        return beam::launch_combine(y16, yscale, topk_w, out, p.T, p.H, p.K, st);
      },
      timed);
}

}  // namespace

// ---------------------------------------------------------------------------
// scratch of beam_moe_forward_noalloc
// ---------------------------------------------------------------------------
// A static device array: every GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` names a host-side stand-in, not the
// device memory: its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device on the first call there, and only
// that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[BEAM_MOE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchTable {
  std::mutex mu;
  std::array<void*, kMaxDevices> ptr{};
};

ScratchTable& scratch_table() {
  static ScratchTable t;
  return t;
}

// Device address of the current GPU's scratch; `st` must belong to that GPU.
int scratch_address(hipStream_t st, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BEAM_MOE_ERR_HIP;
  if (st) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(st, &sdev) != hipSuccess) return BEAM_MOE_ERR_HIP;
    if (sdev != dev) return BEAM_MOE_ERR_INVALID_ARG;
  }
  if (dev < 0 || dev >= kMaxDevices) return BEAM_MOE_ERR_UNSUPPORTED;
  ScratchTable& t = scratch_table();
  std::lock_guard<std::mutex> lock(t.mu);
  if (!t.ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BEAM_MOE_ERR_HIP;
    t.ptr[dev] = p;
  }
  *out = t.ptr[dev];
  return BEAM_MOE_OK;
}

}  // namespace

extern "C" {

size_t beam_moe_workspace_bytes(const beam_moe_dims* dims, int32_t T) {
  if (check_common(dims, T) != BEAM_MOE_OK) return SIZE_MAX;
  // one size for every entry point: the larger of the bf16 and FP8 plans (they differ
  // only if the two kernel families choose different expert paths)
  Plan p, q;
  make_plan(dims, T, &p);
  make_plan(dims, T, &q, true);
  return p.total > q.total ? p.total : q.total;
}

const char* beam_moe_status_str(int status) {
  switch (status) {
    case BEAM_MOE_OK: return "ok";
    case BEAM_MOE_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, negative T)";
    case BEAM_MOE_ERR_UNSUPPORTED: return "unsupported dims";
    case BEAM_MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case BEAM_MOE_ERR_HIP: return "HIP launch failed";
    case BEAM_MOE_ERR_SCRATCH:
      return "batch needs more scratch than the allocation-free entry point holds (BEAM_MOE_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t beam_moe_route_workspace_bytes(const beam_moe_dims* dims, int32_t T) {
  if (check_common(dims, T) != BEAM_MOE_OK) return SIZE_MAX;
  Plan p;
  make_plan(dims, T, &p);
  return route_ws_bytes(p);
}

size_t beam_moe_dispatch_workspace_bytes(const beam_moe_dims* dims, int32_t T) {
  if (check_common(dims, T) != BEAM_MOE_OK) return SIZE_MAX;
  Plan p;
  make_plan(dims, T, &p);
  return dispatch_ws_bytes(p);
}

// Standalone route and dispatch carve their scratch from the start of the
// caller's workspace (the forward entry points place the same buffers inside
// their larger plan).
int beam_moe_route(const beam_moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                   const float* logit_bias, const float* select_bias, int32_t* topk_ids, float* topk_w,
                   float* scores_out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(d, T);
  if (rc != BEAM_MOE_OK || T == 0) return rc;
  if ((rc = check_ptrs({x_bf16, w_router, topk_ids, topk_w})) != BEAM_MOE_OK) return rc;
  if ((logit_bias && !aligned16(logit_bias)) || (select_bias && !aligned16(select_bias)) ||
      (scores_out && !aligned16(scores_out)))
    return BEAM_MOE_ERR_INVALID_ARG;
  Plan p;
  make_plan(d, T, &p);
  if (!ws || !aligned16(ws) || ws_bytes < route_ws_bytes(p)) return BEAM_MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(ws);
  rc = hip_status(beam::launch_router_logits(static_cast<const uint16_t*>(x_bf16), w_router, part, T, p.H, p.E,
                                             p.splits, p.k_per_split, st));
  if (rc != BEAM_MOE_OK) return rc;
  return hip_status(beam::launch_select(part, p.splits, true, logit_bias, select_bias, scores_out, T, p.E,
                                        d->num_groups, d->topk_groups, d->topk, d->routed_scaling, topk_ids, topk_w,
                                        st));
}

int beam_moe_select(const beam_moe_dims* d, int32_t T, const float* scores, const float* select_bias,
                    int32_t* topk_ids, float* topk_w, void* stream) {
  int rc = check_common(d, T);
  if (rc != BEAM_MOE_OK || T == 0) return rc;
  if ((rc = check_ptrs({scores, topk_ids, topk_w})) != BEAM_MOE_OK) return rc;
  if (select_bias && !aligned16(select_bias)) return BEAM_MOE_ERR_INVALID_ARG;
  return hip_status(beam::launch_select(scores, 1, false, nullptr, select_bias, nullptr, T, d->num_experts,
                                        d->num_groups, d->topk_groups, d->topk, d->routed_scaling, topk_ids, topk_w,
                                        static_cast<hipStream_t>(stream)));
}

int beam_moe_dispatch(const beam_moe_dims* d, int32_t T, const int32_t* topk_ids, int32_t* expert_counts,
                      int32_t* expert_offsets, int32_t* sorted_slots, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(d, T);
  if (rc != BEAM_MOE_OK || T == 0) return rc;
  if ((rc = check_ptrs({topk_ids, expert_counts, expert_offsets, sorted_slots})) != BEAM_MOE_OK) return rc;
  Plan p;
  make_plan(d, T, &p);
  if (!ws || !aligned16(ws) || ws_bytes < dispatch_ws_bytes(p)) return BEAM_MOE_ERR_WORKSPACE;
  return hip_status(beam::launch_dispatch(topk_ids, p.n, p.E, static_cast<int32_t*>(ws), expert_counts,
                                          expert_offsets, sorted_slots, nullptr, 0, nullptr,
                                          static_cast<hipStream_t>(stream)));
}

int beam_moe_forward(const beam_moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                     const float* logit_bias, const float* select_bias, const void* w_gate, const void* w_up,
                     const void* w_down, float* out, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                     int32_t* expert_offsets, int32_t* sorted_slots, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int rc = check_forward(d, T, x_bf16, w_router, logit_bias, select_bias, w_gate, w_up, w_down, out, topk_ids,
                         topk_w, expert_counts, expert_offsets, sorted_slots, &p);
  if (rc != BEAM_MOE_OK || T == 0) return rc;
  if (!ws || !aligned16(ws) || ws_bytes < p.total) return BEAM_MOE_ERR_WORKSPACE;
  return forward_bf16(d, p, x_bf16, w_router, logit_bias, select_bias, w_gate, w_up, w_down, out, topk_ids, topk_w,
                      expert_counts, expert_offsets, sorted_slots, ws, static_cast<hipStream_t>(stream), true);
}

int beam_moe_pack_weights(const beam_moe_dims* d, const void* w_down_bf16, void* w_down_packed, void* stream) {
  if (!d) return BEAM_MOE_ERR_INVALID_ARG;
  if (!dims_ok(d)) return BEAM_MOE_ERR_UNSUPPORTED;
  int rc;
  if ((rc = check_ptrs({w_down_bf16, w_down_packed})) != BEAM_MOE_OK) return rc;
  if (w_down_bf16 == w_down_packed) return BEAM_MOE_ERR_INVALID_ARG;
  const size_t n = (size_t)d->num_experts * d->hidden * d->intermediate;
  return hip_status(beam::launch_pack_f16(static_cast<const uint16_t*>(w_down_bf16),
                                          static_cast<uint16_t*>(w_down_packed), n,
                                          static_cast<hipStream_t>(stream)));
}

int beam_moe_forward_packed(const beam_moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                            const float* logit_bias, const float* select_bias, const void* w_gate, const void* w_up,
                            const void* w_down_packed, float* out, int32_t* topk_ids, float* topk_w,
                            int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots, void* ws,
                            size_t ws_bytes, void* stream) {
  Plan p;
  int rc = check_forward(d, T, x_bf16, w_router, logit_bias, select_bias, w_gate, w_up, w_down_packed, out,
                         topk_ids, topk_w, expert_counts, expert_offsets, sorted_slots, &p);
  if (rc != BEAM_MOE_OK || T == 0) return rc;
  if (!ws || !aligned16(ws) || ws_bytes < p.total) return BEAM_MOE_ERR_WORKSPACE;
  return forward_bf16(d, p, x_bf16, w_router, logit_bias, select_bias, w_gate, w_up, w_down_packed, out, topk_ids,
                      topk_w, expert_counts, expert_offsets, sorted_slots, ws, static_cast<hipStream_t>(stream), true,
                      true);
}

int beam_moe_forward_noalloc(const beam_moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                             const float* logit_bias, const float* select_bias, const void* w_gate,
                             const void* w_up, const void* w_down, float* out, int32_t* topk_ids, float* topk_w,
                             int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
                             void* stream) {
  Plan p;
  int rc = check_forward(d, T, x_bf16, w_router, logit_bias, select_bias, w_gate, w_up, w_down, out, topk_ids,
                         topk_w, expert_counts, expert_offsets, sorted_slots, &p);
  if (rc != BEAM_MOE_OK || T == 0) return rc;
  // the documented rule: a batch fits when the one-size workspace does
  if (beam_moe_workspace_bytes(d, T) > (size_t)BEAM_MOE_SCRATCH_BYTES) return BEAM_MOE_ERR_SCRATCH;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((rc = scratch_address(st, &ws)) != BEAM_MOE_OK) return rc;
  return forward_bf16(d, p, x_bf16, w_router, logit_bias, select_bias, w_gate, w_up, w_down, out, topk_ids, topk_w,
                      expert_counts, expert_offsets, sorted_slots, ws, st, false);
}

int beam_moe_forward_fp8(const beam_moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                         const float* logit_bias, const float* select_bias, const uint8_t* w_gate_fp8,
                         const float* gate_scale, const uint8_t* w_up_fp8, const float* up_scale,
                         const uint8_t* w_down_fp8, const float* down_scale, float* out, int32_t* topk_ids,
                         float* topk_w, int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
                         void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(d, T);
  if (rc != BEAM_MOE_OK) return rc;
  if (!beam::stream_fp8_fits(d->hidden, d->intermediate, 8)) return BEAM_MOE_ERR_UNSUPPORTED;
  if (T == 0) return BEAM_MOE_OK;
  if ((rc = check_ptrs({x_bf16, w_router, w_gate_fp8, gate_scale, w_up_fp8, up_scale, w_down_fp8, down_scale, out,
                        topk_ids, topk_w, expert_counts, expert_offsets, sorted_slots})) != BEAM_MOE_OK)
    return rc;
  if ((logit_bias && !aligned16(logit_bias)) || (select_bias && !aligned16(select_bias)))
    return BEAM_MOE_ERR_INVALID_ARG;
  Plan p;
  make_plan(d, T, &p, true);
  if (!ws || !aligned16(ws) || ws_bytes < p.total) return BEAM_MOE_ERR_WORKSPACE;
  BlockArgs a = fp8_block(x_bf16, w_router, logit_bias, select_bias, w_gate_fp8, gate_scale, w_up_fp8, up_scale,
                          w_down_fp8, down_scale, topk_ids, topk_w, expert_counts, expert_offsets, sorted_slots);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return run_block(
      d, p, a, ws, st, [] { return hipSuccess; },
      [&](const uint16_t* y16, const uint8_t* yscale) {
        return beam::launch_combine(y16, yscale, topk_w, out, T, p.H, p.K, st);
      });
}

int beam_moe_residual_forward(const beam_moe_dims* d, int32_t T, const float* stream_in, int32_t step,
                              const float* norm_in_weight, const float* norm_out_weight, float norm_eps,
                              const float* w_router, const float* logit_bias, const float* select_bias,
                              const void* w_gate, const void* w_up, const void* w_down, float* stream_out,
                              int32_t* topk_ids, float* topk_w, int32_t* expert_counts, int32_t* expert_offsets,
                              int32_t* sorted_slots, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(d, T);
  if (rc != BEAM_MOE_OK) return rc;
  if (T > 0 && (rc = check_ptrs({w_gate, w_up, w_down})) != BEAM_MOE_OK) return rc;
  BlockArgs a = bf16_block(nullptr, w_router, logit_bias, select_bias, w_gate, w_up, w_down, topk_ids, topk_w,
                           expert_counts, expert_offsets, sorted_slots);
  return residual_block(d, T, stream_in, step, norm_in_weight, norm_out_weight, norm_eps, a, false, stream_out, ws,
                        ws_bytes, stream);
}

int beam_moe_residual_forward_fp8(const beam_moe_dims* d, int32_t T, const float* stream_in, int32_t step,
                                  const float* norm_in_weight, const float* norm_out_weight, float norm_eps,
                                  const float* w_router, const float* logit_bias, const float* select_bias,
                                  const uint8_t* w_gate_fp8, const float* gate_scale, const uint8_t* w_up_fp8,
                                  const float* up_scale, const uint8_t* w_down_fp8, const float* down_scale,
                                  float* stream_out, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                                  int32_t* expert_offsets, int32_t* sorted_slots, void* ws, size_t ws_bytes,
                                  void* stream) {
  int rc = check_common(d, T);
  if (rc != BEAM_MOE_OK) return rc;
  if (!beam::stream_fp8_fits(d->hidden, d->intermediate, 8)) return BEAM_MOE_ERR_UNSUPPORTED;
  if (T > 0 &&
      (rc = check_ptrs({w_gate_fp8, gate_scale, w_up_fp8, up_scale, w_down_fp8, down_scale})) != BEAM_MOE_OK)
    return rc;
  BlockArgs a = fp8_block(nullptr, w_router, logit_bias, select_bias, w_gate_fp8, gate_scale, w_up_fp8, up_scale,
                          w_down_fp8, down_scale, topk_ids, topk_w, expert_counts, expert_offsets, sorted_slots);
  return residual_block(d, T, stream_in, step, norm_in_weight, norm_out_weight, norm_eps, a, true, stream_out, ws,
                        ws_bytes, stream);
}

int beam_moe_stream_rows(const beam_moe_dims* d, int32_t T, int fp8) {
  const int rc = check_common(d, T);
  if (rc != BEAM_MOE_OK) return rc;
  return stream_rows(d, T, fp8 != 0);
}

int beam_moe_timing_enable(int enable) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  t.enabled = enable != 0;
  return BEAM_MOE_OK;
}

int beam_moe_timing_read(float* stage_ms, int32_t max_stages, int32_t* n_stages, int32_t* calls) {
  if (!stage_ms || !n_stages || !calls || max_stages < 0) return BEAM_MOE_ERR_INVALID_ARG;
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  const int ns = max_stages < kNumStages ? max_stages : kNumStages;
  for (int s = 0; s < ns; ++s) stage_ms[s] = 0.f;
  *n_stages = ns;
  *calls = (int32_t)t.used;
  if (t.used > 0 && hipEventSynchronize(t.slots[t.used - 1][kNumStages]) != hipSuccess) return BEAM_MOE_ERR_HIP;
  for (size_t c = 0; c < t.used; ++c) {
    for (int s = 0; s < ns; ++s) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, t.slots[c][s], t.slots[c][s + 1]) != hipSuccess) return BEAM_MOE_ERR_HIP;
      stage_ms[s] += ms;
    }
  }
  t.used = 0;
  return BEAM_MOE_OK;
}

const char* beam_moe_stage_name(int32_t stage) {
  return (stage >= 0 && stage < kNumStages) ? kStageNames[stage] : nullptr;
}

}  // extern "C"
