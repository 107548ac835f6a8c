// Expert kernels of the Beam MoE block for batches with few rows per expert
// (decode), and the weighted combine (gfx950, FP32 accumulation).
//
// "Welcome Beam: a 501B open model you can own, customize, and scale", its
// mixture-of-experts paragraph, and the Chinese translation of that post,
// 「Reflection 发布 Beam 501B 开源模型，支持 1M tokens 上下文」, section 专家混合模型:
// each expert is a SwiGLU MLP with intermediate size 2560 (hidden 5120);
// section 残差流 (residual stream): the SwiGLU product is computed in FP32.  Per expert e and routed row r:
//   h[r] = silu(W_gate[e] x[r]) * (W_up[e] x[r])   bf16 MFMA, SwiGLU in FP32
//   y[r] = W_down[e] h[r]                           fp16 MFMA, FP32 accumulation
// h is handed to the down projection as fp16 (11 significant bits against
// bf16's 8) with a power-of-two scale 2^-s per block of 64 columns of a row
// tile, s chosen so the block's largest magnitude stays below 2^15; W_down is
// converted from bf16 to fp16 exactly as it is read (or given in fp16 once
// packed), and the FP32 accumulators are kept in units of 2^s of the
// activation block they consume (rescaled exactly when s changes), so the
// weights never carry the scale.  y goes to the combine the same way: fp16
// scaled by 2^-s per (row tile, 64 columns).
// Rows are processed in expert-sorted order (the dispatch permutation); a
// tile table produced by the dispatch maps workgroups to row tiles of one
// expert each.
//
// With few rows per expert the step is bound by streaming each touched
// expert's weights from HBM: a workgroup owns one tile of at most R rows
// (the smallest of 8, 16, 32, 64 that holds twice the batch's average rows
// per expert) and 64 output
// columns, each wave 16 columns over the whole K, so no cross-wave reduction
// is needed; weights and the tile's activation rows are copied into LDS in
// whole 256-byte row segments.  Batches with more rows per expert use the
// grouped GEMMs (grouped_gemm.hip), which read an expert's weights once per
// 256-row tile.
#include <atomic>

#include <algorithm>

#include "common.h"

namespace beam {

// ---------------------------------------------------------------------------
// stream kernels (up to R rows per expert tile)
// ---------------------------------------------------------------------------
// The dispatch cuts each expert's rows into tiles of at most R rows; one
// workgroup takes one tile and 64 output columns and streams those columns'
// weights once over the whole K, against all the tile's rows.  R follows the
// batch (twice the average rows per expert, 8 .. 64), so an expert's weights
// are read once per tile and nearly every expert has one tile.

// Destination slots of this lane's rows (16 f + 4 (lane / 16) + r) of a tile,
// read when the tile starts so that the loads complete under its main loop;
// rows past the tile's end read its last row and are never stored.
template <int NF>
__device__ __forceinline__ void load_y_slots(const int32_t* __restrict__ slot_of, int nrows,
                                             int32_t (&yslot)[NF][4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) yslot[f][r] = slot_of[min(16 * f + (lane >> 4) * 4 + r, nrows - 1)];
}

// Writes one tile of y: fp16 bits of acc * 2^-s, s from the largest magnitude
// of the tile's rows in each 64-column block, and s per (row, block).  Each wave
// holds NB column fragments (columns col + 16 j); the workgroup's 64 NB columns
// start at block cb * NB, and wave w's columns lie in block cb * NB + w * NB / 4.
template <int NF, int NB>
__device__ __forceinline__ void store_y_tile(const f32x4 (&acc)[NB][NF], int nrows, const int32_t (&yslot)[NF][4],
                                             uint16_t* __restrict__ y16, uint8_t* __restrict__ yscale, int H,
                                             int cb, int col, float* smax) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * f + (lane >> 4) * 4 + r < nrows) mx = fmaxf(mx, fabsf(acc[j][f][r]));
  mx = wave_max(mx);
  if (lane == 0) smax[wave] = mx;
  __syncthreads();
  constexpr int kGroup = 4 / NB;  // waves sharing a 64-column block
  const int g0 = wave / kGroup * kGroup;
  float bm = smax[g0];
#pragma unroll
  for (int i = 1; i < kGroup; ++i) bm = fmaxf(bm, smax[g0 + i]);
  const int sexp = act_scale_exp(bm);
  const int blk = cb * NB + wave / kGroup;
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * f + (lane >> 4) * 4 + r;
      if (row < nrows) {
        const size_t slot = (size_t)yslot[f][r];
#pragma unroll
        for (int j = 0; j < NB; ++j)
          y16[slot * H + col + 16 * j] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(acc[j][f][r], -sexp));
        if (wave == g0 && (lane & 15) == 0) yscale[slot * (H / kScaleCols) + blk] = (uint8_t)sexp;
      }
    }
}

// Writes one tile of h: SwiGLU values v (FP32, zero past the tile's end) as fp16
// times 2^-s, s from the tile's largest magnitude in the workgroup's 64 columns.
template <int NF>
__device__ __forceinline__ void store_h_tile(const float (&v)[NF][4], float mx, const Tile& tl,
                                             uint16_t* __restrict__ h, uint8_t* __restrict__ hscale, int I, int cb,
                                             int col, float* smax) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  mx = wave_max(mx);
  if (lane == 0) smax[wave] = mx;
  __syncthreads();
  const int sexp = act_scale_exp(fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3])));
  const int nsb = I / kScaleCols;
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * f + (lane >> 4) * 4 + r;
      if (row < tl.rows) {
        const size_t gr = (size_t)(tl.row_start + row);
        h[gr * I + col] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(v[f][r], -sexp));
        if (wave == 0 && (lane & 15) == 0) hscale[gr * nsb + cb] = (uint8_t)sexp;
      }
    }
}

int scale_cols() { return kScaleCols; }

// Placement of a stream workgroup: (tile, 64-column block).  The grid is 1-D,
// sized for the most tiles a batch can have times ncb column blocks; the order
// spans the tiles this batch has (read on the device), and each XCD (block b runs
// on XCD b % 8) takes a contiguous range of the tile-major order, so the column
// blocks of one tile run side by side on one XCD and share its activation rows
// in that XCD's L2.  Returns false for the surplus blocks, which exit.
__device__ __forceinline__ bool stream_block(const int32_t* __restrict__ ntiles, int ncb, int& tile, int& cb) {
  const int real = ntiles[0] * ncb;
  const int b = blockIdx.x;
  if (b >= real) return false;
  const int full = real & ~7;
  const int lin = b >= full ? b : (b & 7) * (full >> 3) + (b >> 3);
  tile = lin / ncb;
  cb = lin - tile * ncb;
  return true;
}

// One tile of at most R rows per workgroup, 64 output columns, each wave 16
// columns over the whole K and all the tile's rows (R / 16 row fragments, one
// for R = 8); weights and the tile's activation rows reach the MFMAs through LDS.
// Per stage of kSk = 128 of K, the load unit copies the workgroup's weight rows
// and the activation rows into a ring slot (global_load_lds), each copy taking
// 4 rows x 256 contiguous bytes: register operand loads touch 16 rows x 64
// bytes each, which caps the stream near 6.0 TB/s, while whole 256-byte row
// segments stream at about 6.5 TB/s.  Inside a slot every row is 256 bytes and
// its 16-byte chunk c sits at position c ^ (r & 15), so the 16 rows read by one
// MFMA operand load fall on distinct banks.  A copy of row r fetches, for its
// lane at position p, the chunk p ^ (r & 15).
constexpr int kSk = 128;  // K per stage

// Stage geometry for SK elements of K per stage: rows of SK * 2 bytes; one copy
// (1 KB) covers RPI rows with LPR lanes per row.
template <int SK>
struct StageGeom {
  static constexpr int kRowBytes = SK * 2;
  static constexpr int kRPI = 1024 / kRowBytes;
  static constexpr int kLPR = 64 / kRPI;
  static_assert(kRPI >= 1 && kRPI * kRowBytes == 1024, "a copy covers whole rows");
  // the swizzle XORs a chunk index with (row & 15): rows need at least 16 chunks
  // of 16 bytes so that every swizzled chunk stays inside its row's segment
  static_assert(kRowBytes >= 256, "stage rows of at least 16 chunks");
};

// Activation rows of a tile of R rows: each of the 4 waves copies R / 4 of them,
// kRPI rows per copy; at R = 8 a wave's two rows take half of one copy's lanes.
template <int SK, int R>
struct ActCopies {
  using G = StageGeom<SK>;
  static constexpr int kPer = R / 4;                               // rows per wave
  static constexpr int kCopies = (kPer + G::kRPI - 1) / G::kRPI;  // copy instructions per wave and stage
  static constexpr int kLanes = kPer < G::kRPI ? kPer * G::kLPR : 64;
  static_assert(R % 8 == 0 && (kPer < G::kRPI || kPer % G::kRPI == 0), "whole copies or one partial one");
};

// Source of lane `lane` for a copy whose lanes cover row r at positions
// lane % LPR: the chunk (lane % LPR) ^ (r & 15) of the row starting at row_ptr.
template <int SK>
__device__ __forceinline__ const uint16_t* stage_src(const uint16_t* row_ptr, int r, int lane) {
  const int pos = lane % StageGeom<SK>::kLPR;
  return row_ptr + ((pos ^ (r & 15)) << 3);
}

// Byte offset of (row, chunk) in a slot.
template <int SK>
__device__ __forceinline__ int stage_off(int row, int chunk) {
  return row * StageGeom<SK>::kRowBytes + ((chunk ^ (row & 15)) << 4);
}

// Waits until this wave's copies of stage st have landed, `later` stages (at most
// two) having been requested after it, each with COPIES copy instructions.
template <int COPIES>
__device__ __forceinline__ void wait_stage(int later) {
  if (later >= 2)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * COPIES));
  else if (later == 1)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(COPIES));
  else
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
}

// grid: max_tiles * I / 64 (see stream_block); block 256; dynamic LDS SLOTS * (128 + R) * 256 bytes.
// Slot rows: 0..63 gate rows of the workgroup's columns, 64..127 the up rows,
// 128 .. 128 + R - 1 the activation rows of the tile.
template <int SLOTS, int SK, int R>
__global__ __launch_bounds__(256) void gateup_stream_lds_kernel(const uint16_t* __restrict__ x,
                                                                const int32_t* __restrict__ sorted_slots,
                                                                const Tile* __restrict__ tiles,
                                                                const int32_t* __restrict__ ntiles,
                                                                const uint16_t* __restrict__ wg,
                                                                const uint16_t* __restrict__ wu,
                                                                uint16_t* __restrict__ h,
                                                                uint8_t* __restrict__ hscale, int H, int I, int K) {
  using G = StageGeom<SK>;
  using AC = ActCopies<SK, R>;
  constexpr int kRows = 128 + R;
  constexpr int kSlot = kRows * G::kRowBytes;
  constexpr int kWCopies = 32 / G::kRPI;  // weight copies per wave per stage (32 rows)
  constexpr int kCopies = kWCopies + AC::kCopies;
  constexpr int kNF = (R + 15) / 16;      // row fragments
  extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
  __shared__ float smax[4];
  int ti, cb;
  if (!stream_block(ntiles, I / 64, ti, cb)) return;
  const Tile tl = tiles[ti];  // at most R rows
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = lane & 15;
  const int col = cb * 64 + wave * 16 + m;
  const int nst = H / SK;
  const size_t ebase = (size_t)tl.expert * I * H;
  const int nrows = tl.rows;

  // weight copies: wave w fills slot rows 32w .. 32w+31 (w < 2: gate, else up)
  const uint16_t* wsrc[kWCopies];
#pragma unroll
  for (int q = 0; q < kWCopies; ++q) {
    const int r = 32 * wave + G::kRPI * q + lane / G::kLPR;
    const uint16_t* base = (r < 64 ? wg : wu) + ebase + (size_t)(cb * 64 + (r & 63)) * H;
    wsrc[q] = stage_src<SK>(base, r, lane);
  }
  // activation copies: wave w fills activation rows AC::kPer w .. AC::kPer (w + 1) - 1;
  // rows past the tile's end repeat its last row
  const uint16_t* xsrc[AC::kCopies];
#pragma unroll
  for (int q = 0; q < AC::kCopies; ++q) {
    const int xr = AC::kPer * wave + G::kRPI * q + lane / G::kLPR;
    const int tok = sorted_slots[tl.row_start + min(xr, nrows - 1)] / K;
    xsrc[q] = stage_src<SK>(x + (size_t)tok * H, 128 + xr, lane);
  }
  auto issue = [&](int st, int slot) {
    unsigned char* sl = ring + slot * kSlot;
    const int k = st * SK;
#pragma unroll
    for (int q = 0; q < kWCopies; ++q) lds_copy16(wsrc[q] + k, lds_addr(sl + (32 * wave + G::kRPI * q) * G::kRowBytes));
#pragma unroll
    for (int q = 0; q < AC::kCopies; ++q)
      if (lane < AC::kLanes)
        lds_copy16(xsrc[q] + k, lds_addr(sl + (128 + AC::kPer * wave + G::kRPI * q) * G::kRowBytes));
  };
  f32x4 ag[kNF], au[kNF];
  int arow[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
    ag[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    au[f] = ag[f];
    const int ar = 16 * f + m;  // at R = 8, operand rows 8..15 read row 0: never stored
    arow[f] = 128 + (ar < R ? ar : 0);
  }
  const int grow = wave * 16 + m, urow = 64 + wave * 16 + m;
#pragma unroll
  for (int s = 0; s < SLOTS - 1; ++s)
    if (s < nst) issue(s, s);
  for (int st = 0; st < nst; ++st) {
    wait_stage<kCopies>(min(SLOTS - 2, nst - 1 - st));
    __builtin_amdgcn_s_barrier();  // stage st complete for all waves; stage st - 1's slot is free
    if (st + SLOTS - 1 < nst) issue(st + SLOTS - 1, (st + SLOTS - 1) % SLOTS);
    const unsigned char* sl = ring + (st % SLOTS) * kSlot;
#pragma unroll
    for (int s = 0; s < SK / 32; ++s) {
      const int c = 4 * s + (lane >> 4);
      const u32x4 g = *reinterpret_cast<const u32x4*>(sl + stage_off<SK>(grow, c));
      const u32x4 u = *reinterpret_cast<const u32x4*>(sl + stage_off<SK>(urow, c));
#pragma unroll
      for (int f = 0; f < kNF; ++f) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sl + stage_off<SK>(arow[f], c));
        ag[f] = mfma16x16x32(a, g, ag[f]);
        au[f] = mfma16x16x32(a, u, au[f]);
      }
    }
  }
  // SwiGLU in FP32; one power-of-two scale per (tile, 64 columns)
  float v[kNF][4];
  float mx = 0.f;
#pragma unroll
  for (int f = 0; f < kNF; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * f + (lane >> 4) * 4 + r;
      v[f][r] = (row < nrows) ? silu_f32(ag[f][r]) * au[f][r] : 0.f;
      mx = fmaxf(mx, fabsf(v[f][r]));
    }
  store_h_tile<kNF>(v, mx, tl, h, hscale, I, cb, col, smax);
}

// grid: max_tiles * H / (64 NB) (see stream_block); block 256; dynamic LDS
// SLOTS * (64 NB + R) * 256 bytes + the tile's scales.  y leaves through
// store_y_tile.  Each wave owns NB fragments of 16 output columns: the workgroup
// covers 64 NB columns, so wide tiles (NB = 2) read their activation rows half as
// often per weight byte, in LDS and from L2.  Slot rows: 0 .. 64 NB - 1 W_down
// rows of the workgroup's columns, then the R activation rows (h, fp16) of the tile.
// WF16: W_down given in fp16 (beam_moe_pack_weights), used as read.
template <int SLOTS, int SK, int R, int NB, bool WF16>
__global__ __launch_bounds__(256) void down_stream_lds_kernel(const uint16_t* __restrict__ h,
                                                              const uint8_t* __restrict__ hscale,
                                                              const int32_t* __restrict__ sorted_slots,
                                                              const Tile* __restrict__ tiles,
                                                              const int32_t* __restrict__ ntiles,
                                                              const uint16_t* __restrict__ wd,
                                                              uint16_t* __restrict__ y16,
                                                              uint8_t* __restrict__ yscale, int H, int I) {
  using G = StageGeom<SK>;
  using AC = ActCopies<SK, R>;
  constexpr int kWRows = 64 * NB;
  constexpr int kRows = kWRows + R;
  constexpr int kSlot = kRows * G::kRowBytes;
  constexpr int kWCopies = 16 * NB / G::kRPI;  // weight copies per wave per stage (16 NB rows)
  constexpr int kCopies = kWCopies + AC::kCopies;
  constexpr int kNF = (R + 15) / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
  __shared__ int sany;
  __shared__ float smax[4];
  uint8_t* ssc = ring + SLOTS * kSlot;  // the tile's activation scales
  int ti, cb;
  if (!stream_block(ntiles, H / kWRows, ti, cb)) return;
  const Tile tl = tiles[ti];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 15;
  const int col = cb * kWRows + wave * 16 * NB + m;  // + 16 j for fragment j
  const int nsb = I / kScaleCols;
  const int nst = I / SK;
  const int nrows = tl.rows;

  const uint16_t* wsrc[kWCopies];
#pragma unroll
  for (int q = 0; q < kWCopies; ++q) {
    const int r = 16 * NB * wave + G::kRPI * q + lane / G::kLPR;
    const uint16_t* base = wd + (size_t)tl.expert * H * I + (size_t)(cb * kWRows + r) * I;
    wsrc[q] = stage_src<SK>(base, r, lane);
  }
  int32_t yslot[kNF][4];
  load_y_slots<kNF>(sorted_slots + tl.row_start, nrows, yslot);
  const uint16_t* xsrc[AC::kCopies];
#pragma unroll
  for (int q = 0; q < AC::kCopies; ++q) {
    const int xr = AC::kPer * wave + G::kRPI * q + lane / G::kLPR;
    xsrc[q] = stage_src<SK>(h + (size_t)(tl.row_start + min(xr, nrows - 1)) * I, kWRows + xr, lane);
  }
  auto issue = [&](int st, int slot) {
    unsigned char* sl = ring + slot * kSlot;
    const int k = st * SK;
#pragma unroll
    for (int q = 0; q < kWCopies; ++q)
      lds_copy16(wsrc[q] + k, lds_addr(sl + (16 * NB * wave + G::kRPI * q) * G::kRowBytes));
#pragma unroll
    for (int q = 0; q < AC::kCopies; ++q)
      if (lane < AC::kLanes)
        lds_copy16(xsrc[q] + k, lds_addr(sl + (kWRows + AC::kPer * wave + G::kRPI * q) * G::kRowBytes));
  };
#pragma unroll
  for (int s = 0; s < SLOTS - 1; ++s)
    if (s < nst) issue(s, s);
  if (tid == 0) sany = 0;
  __syncthreads();
  for (int i = tid; i < nsb; i += 256) {
    const uint8_t sv = hscale[(size_t)tl.row_start * nsb + i];  // one scale per (tile, 64 columns)
    ssc[i] = sv;
    if (sv) sany = 1;
  }
  __syncthreads();
  const bool scaled = sany != 0;
  f32x4 acc[NB][kNF];
  int arow[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ar = 16 * f + m;
    arow[f] = kWRows + (ar < R ? ar : 0);
  }
  const int brow = wave * 16 * NB + m;  // + 16 j
  int s_acc = 0;  // acc holds y * 2^-s_acc (the activation block consumed last)
  for (int st = 0; st < nst; ++st) {
    wait_stage<kCopies>(min(SLOTS - 2, nst - 1 - st));
    __builtin_amdgcn_s_barrier();
    if (st + SLOTS - 1 < nst) issue(st + SLOTS - 1, (st + SLOTS - 1) % SLOTS);
    const unsigned char* sl = ring + (st % SLOTS) * kSlot;
#pragma unroll
    for (int s = 0; s < SK / 32; ++s) {
      const int c = 4 * s + (lane >> 4);
      u32x4 b[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j)
      {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(sl + stage_off<SK>(brow + 16 * j, c));
        b[j] = WF16 ? raw : bf16x8_to_f16x8(raw);  // WF16: the weights are fp16 already
      }
      if (scaled) {
        const int sk = __builtin_amdgcn_readfirstlane(ssc[(st * SK + 32 * s) / kScaleCols]);
        if (sk != s_acc) {
#pragma unroll
          for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int f = 0; f < kNF; ++f) acc[j][f] = ldexp4(acc[j][f], s_acc - sk);
          s_acc = sk;
        }
      }
#pragma unroll
      for (int f = 0; f < kNF; ++f) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sl + stage_off<SK>(arow[f], c));
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[j][f] = mfma16x16x32_f16(a, b[j], acc[j][f]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int f = 0; f < kNF; ++f) acc[j][f] = ldexp4(acc[j][f], s_acc);
  store_y_tile<kNF, NB>(acc, nrows, yslot, y16, yscale, H, cb, col, smax);
}

// ---------------------------------------------------------------------------
// stream kernels with FP8 (E4M3) expert weights
// ---------------------------------------------------------------------------
// 「Reflection 放出 501B 的 Beam 权重：四套精度、滑动窗口和一场榜单落差」, the
// FP8 repository's parameter-precision listing: every expert weight is E4M3;
// the granularity of its scales is not given, taken here as one fp32 scale
// per output row.  W[r, :] = decode(q[r, :]) * scale[r]: the codes are decoded
// exactly to bf16 (gate/up, against bf16 activations) or fp16 (down, against
// the fp16 activations, whose 2^s the accumulator carries) in registers, the
// MFMAs accumulate in FP32 and the row scale multiplies the accumulator.  Half
// the bytes of the bf16 weights for the same arithmetic.
//
// Stage of kF8Sk = 256 of K: weight rows of 256 bytes (256 codes) and
// activation rows of 512 bytes (256 bf16 / fp16 values), both with 16-byte
// chunk c of row r at position c ^ (r & 15).  Per 64 of K a lane reads one
// 16-byte chunk of codes (16 K values) and the two matching 16-byte chunks of
// its activation row: two MFMAs of K = 32, the first on the chunk's 8 low
// codes, the second on its 8 high ones.  A and B agree on which K each operand
// slot holds, which is all a contraction needs.
constexpr int kF8Sk = 256;     // K per stage
constexpr int kF8WRow = 256;   // bytes of a staged weight row
constexpr int kF8ARow = 512;   // bytes of a staged activation row

__device__ __forceinline__ int f8_woff(int row, int chunk) { return row * kF8WRow + ((chunk ^ (row & 15)) << 4); }
__device__ __forceinline__ int f8_aoff(int row, int chunk) { return row * kF8ARow + ((chunk ^ (row & 15)) << 4); }

// Activation rows of 512 bytes: each wave copies R / 4 of them, two per copy.
template <int R>
struct F8ActCopies {
  static constexpr int kPer = R / 4;
  static constexpr int kCopies = kPer / 2;
  static_assert(R % 8 == 0, "whole copies");
};

// 16 E4M3 codes -> two operands of 8 bf16 (exact: E4M3 values are bf16 values).
__device__ __forceinline__ void fp8x16_to_bf16(u32x4 q, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    lo[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i], 1.0f, false));
    lo[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i], 1.0f, true));
    hi[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i + 2], 1.0f, false));
    hi[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i + 2], 1.0f, true));
  }
}

// 16 E4M3 codes -> two operands of 8 fp16 (exact: every E4M3 value, at most 448
// in magnitude, is an fp16 value).
__device__ __forceinline__ void fp8x16_to_f16(u32x4 q, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    lo[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q[i], 1.0f, false));
    lo[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q[i], 1.0f, true));
    hi[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q[i + 2], 1.0f, false));
    hi[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q[i + 2], 1.0f, true));
  }
}

// grid: max_tiles * I / 64 (see stream_block); block 256; dynamic LDS SLOTS * (128 * 256 + R * 512) bytes.
// Slot: 128 weight rows (0..63 gate, 64..127 up, of the workgroup's columns), then
// the tile's R activation rows.
template <int SLOTS, int R>
__global__ __launch_bounds__(256) void gateup_stream_fp8_kernel(const uint16_t* __restrict__ x,
                                                                const int32_t* __restrict__ sorted_slots,
                                                                const Tile* __restrict__ tiles,
                                                                const int32_t* __restrict__ ntiles,
                                                                const uint8_t* __restrict__ wg,
                                                                const uint8_t* __restrict__ wu,
                                                                const float* __restrict__ sg,
                                                                const float* __restrict__ su,
                                                                uint16_t* __restrict__ h,
                                                                uint8_t* __restrict__ hscale, int H, int I, int K) {
  using AC = F8ActCopies<R>;
  constexpr int kWBytes = 128 * kF8WRow;
  constexpr int kSlot = kWBytes + R * kF8ARow;
  constexpr int kWCopies = 8;  // 32 weight rows of 256 bytes per wave: 4 rows per copy
  constexpr int kCopies = kWCopies + AC::kCopies;
  constexpr int kNF = (R + 15) / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
  __shared__ float smax[4];
  int ti, cb;
  if (!stream_block(ntiles, I / 64, ti, cb)) return;
  const Tile tl = tiles[ti];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = lane & 15;
  const int col = cb * 64 + wave * 16 + m;
  const int nst = H / kF8Sk;
  const size_t ebase = (size_t)tl.expert * I * H;
  const int nrows = tl.rows;

  // weight copies: wave w fills slot rows 32w .. 32w+31 (w < 2: gate, else up), 16 lanes a row
  const uint8_t* wsrc[kWCopies];
#pragma unroll
  for (int q = 0; q < kWCopies; ++q) {
    const int r = 32 * wave + 4 * q + (lane >> 4);
    const uint8_t* base = (r < 64 ? wg : wu) + ebase + (size_t)(cb * 64 + (r & 63)) * H;
    wsrc[q] = base + (((lane & 15) ^ (r & 15)) << 4);
  }
  const float scale_g = sg[(size_t)tl.expert * I + col];
  const float scale_u = su[(size_t)tl.expert * I + col];
  // activation copies: wave w fills rows AC::kPer w .., two rows of 32 lanes per copy
  const unsigned char* xsrc[AC::kCopies];
#pragma unroll
  for (int q = 0; q < AC::kCopies; ++q) {
    const int xr = AC::kPer * wave + 2 * q + (lane >> 5);
    const int tok = sorted_slots[tl.row_start + min(xr, nrows - 1)] / K;
    xsrc[q] = reinterpret_cast<const unsigned char*>(x + (size_t)tok * H) + (((lane & 31) ^ (xr & 15)) << 4);
  }
  auto issue = [&](int st, int slot) {
    unsigned char* sl = ring + slot * kSlot;
#pragma unroll
    for (int q = 0; q < kWCopies; ++q)
      lds_copy16(wsrc[q] + (size_t)st * kF8Sk, lds_addr(sl + (32 * wave + 4 * q) * kF8WRow));
#pragma unroll
    for (int q = 0; q < AC::kCopies; ++q)
      lds_copy16(xsrc[q] + (size_t)st * kF8Sk * 2, lds_addr(sl + kWBytes + (AC::kPer * wave + 2 * q) * kF8ARow));
  };
  f32x4 ag[kNF], au[kNF];
  int arow[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
    ag[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    au[f] = ag[f];
    const int ar = 16 * f + m;
    arow[f] = ar < R ? ar : 0;
  }
  const int grow = wave * 16 + m, urow = 64 + wave * 16 + m;
#pragma unroll
  for (int s = 0; s < SLOTS - 1; ++s)
    if (s < nst) issue(s, s);
  for (int st = 0; st < nst; ++st) {
    wait_stage<kCopies>(min(SLOTS - 2, nst - 1 - st));
    __builtin_amdgcn_s_barrier();  // stage st complete for all waves; stage st - 1's slot is free
    if (st + SLOTS - 1 < nst) issue(st + SLOTS - 1, (st + SLOTS - 1) % SLOTS);
    const unsigned char* sl = ring + (st % SLOTS) * kSlot;
    const unsigned char* sa = sl + kWBytes;
#pragma unroll
    for (int j = 0; j < kF8Sk / 64; ++j) {
      const int cw = 4 * j + (lane >> 4);
      u32x4 g0, g1, u0, u1;
      fp8x16_to_bf16(*reinterpret_cast<const u32x4*>(sl + f8_woff(grow, cw)), g0, g1);
      fp8x16_to_bf16(*reinterpret_cast<const u32x4*>(sl + f8_woff(urow, cw)), u0, u1);
#pragma unroll
      for (int f = 0; f < kNF; ++f) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(sa + f8_aoff(arow[f], 2 * cw));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(sa + f8_aoff(arow[f], 2 * cw + 1));
        ag[f] = mfma16x16x32(a0, g0, ag[f]);
        au[f] = mfma16x16x32(a0, u0, au[f]);
        ag[f] = mfma16x16x32(a1, g1, ag[f]);
        au[f] = mfma16x16x32(a1, u1, au[f]);
      }
    }
  }
  // row scales, then SwiGLU in FP32; one power-of-two scale per (tile, 64 columns)
  float v[kNF][4];
  float mx = 0.f;
#pragma unroll
  for (int f = 0; f < kNF; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * f + (lane >> 4) * 4 + r;
      v[f][r] = (row < nrows) ? silu_f32(ag[f][r] * scale_g) * (au[f][r] * scale_u) : 0.f;
      mx = fmaxf(mx, fabsf(v[f][r]));
    }
  store_h_tile<kNF>(v, mx, tl, h, hscale, I, cb, col, smax);
}

// grid: max_tiles * H / (64 NB) (see stream_block); block 256; dynamic LDS
// SLOTS * (64 NB * 256 + R * 512) bytes + the tile's scales.  Slot: 64 NB W_down rows
// of the workgroup's columns (NB fragments of 16 per wave, as the bf16 kernel), then
// the tile's R h rows.
template <int SLOTS, int R, int NB>
__global__ __launch_bounds__(256) void down_stream_fp8_kernel(const uint16_t* __restrict__ h,
                                                              const uint8_t* __restrict__ hscale,
                                                              const int32_t* __restrict__ sorted_slots,
                                                              const Tile* __restrict__ tiles,
                                                              const int32_t* __restrict__ ntiles,
                                                              const uint8_t* __restrict__ wd,
                                                              const float* __restrict__ sd,
                                                              uint16_t* __restrict__ y16,
                                                              uint8_t* __restrict__ yscale, int H, int I) {
  using AC = F8ActCopies<R>;
  constexpr int kWRows = 64 * NB;
  constexpr int kWBytes = kWRows * kF8WRow;
  constexpr int kSlot = kWBytes + R * kF8ARow;
  constexpr int kWCopies = 4 * NB;  // 16 NB weight rows of 256 bytes per wave, 4 rows per copy
  constexpr int kCopies = kWCopies + AC::kCopies;
  constexpr int kNF = (R + 15) / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
  __shared__ int sany;
  __shared__ float smax[4];
  uint8_t* ssc = ring + SLOTS * kSlot;  // the tile's activation scales
  int ti, cb;
  if (!stream_block(ntiles, H / kWRows, ti, cb)) return;
  const Tile tl = tiles[ti];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 15;
  const int col = cb * kWRows + wave * 16 * NB + m;  // + 16 j for fragment j
  const int nsb = I / kScaleCols;
  const int nst = I / kF8Sk;
  const int nrows = tl.rows;

  const uint8_t* wsrc[kWCopies];
#pragma unroll
  for (int q = 0; q < kWCopies; ++q) {
    const int r = 16 * NB * wave + 4 * q + (lane >> 4);
    const uint8_t* base = wd + (size_t)tl.expert * H * I + (size_t)(cb * kWRows + r) * I;
    wsrc[q] = base + (((lane & 15) ^ (r & 15)) << 4);
  }
  float scale_d[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) scale_d[j] = sd[(size_t)tl.expert * H + col + 16 * j];
  int32_t yslot[kNF][4];
  load_y_slots<kNF>(sorted_slots + tl.row_start, nrows, yslot);
  const unsigned char* xsrc[AC::kCopies];
#pragma unroll
  for (int q = 0; q < AC::kCopies; ++q) {
    const int xr = AC::kPer * wave + 2 * q + (lane >> 5);
    xsrc[q] = reinterpret_cast<const unsigned char*>(h + (size_t)(tl.row_start + min(xr, nrows - 1)) * I) +
              (((lane & 31) ^ (xr & 15)) << 4);
  }
  auto issue = [&](int st, int slot) {
    unsigned char* sl = ring + slot * kSlot;
#pragma unroll
    for (int q = 0; q < kWCopies; ++q)
      lds_copy16(wsrc[q] + (size_t)st * kF8Sk, lds_addr(sl + (16 * NB * wave + 4 * q) * kF8WRow));
#pragma unroll
    for (int q = 0; q < AC::kCopies; ++q)
      lds_copy16(xsrc[q] + (size_t)st * kF8Sk * 2, lds_addr(sl + kWBytes + (AC::kPer * wave + 2 * q) * kF8ARow));
  };
#pragma unroll
  for (int s = 0; s < SLOTS - 1; ++s)
    if (s < nst) issue(s, s);
  if (tid == 0) sany = 0;
  __syncthreads();
  for (int i = tid; i < nsb; i += 256) {
    const uint8_t sv = hscale[(size_t)tl.row_start * nsb + i];
    ssc[i] = sv;
    if (sv) sany = 1;
  }
  __syncthreads();
  const bool scaled = sany != 0;
  f32x4 acc[NB][kNF];
  int arow[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ar = 16 * f + m;
    arow[f] = ar < R ? ar : 0;
  }
  const int brow = wave * 16 * NB + m;  // + 16 j
  int s_acc = 0;  // acc holds y * 2^-s_acc (the activation block consumed last)
  for (int st = 0; st < nst; ++st) {
    wait_stage<kCopies>(min(SLOTS - 2, nst - 1 - st));
    __builtin_amdgcn_s_barrier();
    if (st + SLOTS - 1 < nst) issue(st + SLOTS - 1, (st + SLOTS - 1) % SLOTS);
    const unsigned char* sl = ring + (st % SLOTS) * kSlot;
    const unsigned char* sa = sl + kWBytes;
#pragma unroll
    for (int jk = 0; jk < kF8Sk / 64; ++jk) {
      const int cw = 4 * jk + (lane >> 4);
      u32x4 b0[NB], b1[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fp8x16_to_f16(*reinterpret_cast<const u32x4*>(sl + f8_woff(brow + 16 * j, cw)), b0[j], b1[j]);
      // the 64 K values of step jk share one activation scale block
      if (scaled) {
        const int sk = __builtin_amdgcn_readfirstlane(ssc[(st * kF8Sk) / kScaleCols + jk]);
        if (sk != s_acc) {
#pragma unroll
          for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int f = 0; f < kNF; ++f) acc[j][f] = ldexp4(acc[j][f], s_acc - sk);
          s_acc = sk;
        }
      }
#pragma unroll
      for (int f = 0; f < kNF; ++f) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(sa + f8_aoff(arow[f], 2 * cw));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(sa + f8_aoff(arow[f], 2 * cw + 1));
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          acc[j][f] = mfma16x16x32_f16(a0, b0[j], acc[j][f]);
          acc[j][f] = mfma16x16x32_f16(a1, b1[j], acc[j][f]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      acc[j][f] = ldexp4(acc[j][f], s_acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[j][f][r] *= scale_d[j];
    }
  store_y_tile<kNF, NB>(acc, nrows, yslot, y16, yscale, H, cb, col, smax);
}

// Dynamic LDS the stream kernels may take: 152 KB of a gfx950 CU's 160 KB,
// leaving room for their small static arrays.
constexpr size_t kStreamLdsMax = 152 * 1024;

// Raises `fn`'s dynamic-LDS limit to kStreamLdsMax, once per device (the
// attribute is per device; later launches, graph captures included, only launch).
static hipError_t allow_full_lds(const void* fn, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStreamLdsMax);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Workgroups of 256 threads of `fn` that the device holds at once with `lds` bytes
// of dynamic LDS each (0 if the runtime cannot tell); computed once per kernel, on
// the first device that asks, and used for all (the kernels are built for one GPU
// model; the figure only picks a ring depth, never correctness).  The kernel's
// dynamic-LDS limit is raised first, as for its launches.
static int resident_blocks(const void* fn, size_t lds, std::atomic<int>& cached) {
  int n = cached.load(std::memory_order_acquire);
  if (n >= 0) return n;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStreamLdsMax) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds) != hipSuccess)
    return 0;
  n = cus * per_cu;
  cached.store(n, std::memory_order_release);
  return n;
}

// Ring depth per tile height: three slots while they fit, else two.  A grid that
// the device cannot hold at once with three slots but can with two (a batch of a
// token or two: a few experts' column blocks) takes two, so that no workgroup waits
// for a second round on a quarter of the CUs.
constexpr int gateup_slots(int R) { return (128 + R) * 256 * 3 <= 144 * 1024 ? 3 : 2; }
// The down kernels' shape per tile height, chosen by measurement (T = 256 .. 1024 at
// Beam dims, identical output in every variant): a ring that fits half the LDS lets
// two workgroups share a CU, so one's start-up and tail overlap the other's
// streaming, which beat 128-column workgroups (which read their activation rows
// half as often per weight byte) for bf16 weights at every tile height: 64-row
// tiles 1.35 against 1.50 ms, 32-row 1.17 against 1.20.  With FP8 weights, whose
// 512-byte activation rows outweigh the codes from 64-row tiles, 128 columns win
// there (0.92 ms, against 1.11 with 64 columns and one workgroup per CU).
constexpr int kHalfLds = 78 * 1024;
constexpr int down_nb(int R) { return 1; }
constexpr int down_slots(int R) { return (64 * down_nb(R) + R) * 256 * 3 <= kHalfLds ? 3 : 2; }
constexpr int down_f8_nb(int R) { return R >= 64 ? 2 : 1; }
constexpr int gateup_f8_slots(int R) { return R >= 64 ? 2 : 3; }
constexpr int down_f8_slots(int R) {
  return (64 * down_f8_nb(R) * kF8WRow + R * kF8ARow) * 3 <= kHalfLds ? 3 : 2;
}

size_t gateup_stream_lds_bytes(int R) { return (size_t)gateup_slots(R) * (128 + R) * StageGeom<kSk>::kRowBytes; }
size_t down_stream_lds_bytes(int R, int I) {
  return (size_t)down_slots(R) * (64 * down_nb(R) + R) * StageGeom<kSk>::kRowBytes + I / kScaleCols;
}
size_t gateup_stream_fp8_lds_bytes(int R) { return (size_t)gateup_f8_slots(R) * (128 * kF8WRow + R * kF8ARow); }
size_t down_stream_fp8_lds_bytes(int R, int I) {
  return (size_t)down_f8_slots(R) * (64 * down_f8_nb(R) * kF8WRow + R * kF8ARow) + I / kScaleCols;
}

// Tile heights the stream kernels are built for.  Wider tiles (128 rows) were
// measured slower than the grouped GEMMs at the batches that would use them
// (T = 2048 at Beam dims: 5.1 against 4.4 ms).
bool stream_rows_ok(int R, bool) { return R == 8 || R == 16 || R == 32 || R == 64; }

// Whether the stream kernels with tiles of R rows can run at this shape: K of
// both projections in whole stages, and the staged rows and the down kernel's
// scales fit in LDS.
bool stream_fits(int H, int I, int R) {
  return stream_rows_ok(R, false) && H % kSk == 0 && I % kSk == 0 && H % (64 * down_nb(R)) == 0 &&
         gateup_stream_lds_bytes(R) <= kStreamLdsMax && down_stream_lds_bytes(R, I) <= kStreamLdsMax;
}

bool stream_fp8_fits(int H, int I, int R) {
  return stream_rows_ok(R, true) && H % kF8Sk == 0 && I % kF8Sk == 0 && H % (64 * down_f8_nb(R)) == 0 &&
         gateup_stream_fp8_lds_bytes(R) <= kStreamLdsMax && down_stream_fp8_lds_bytes(R, I) <= kStreamLdsMax;
}

template <int S, int R>
static hipError_t gateup_fp8_s(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                               int max_tiles, const uint8_t* wg, const uint8_t* wu, const float* sg, const float* su,
                               uint16_t* h, uint8_t* hscale, int H, int I, int K, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&gateup_stream_fp8_kernel<S, R>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gateup_stream_fp8_kernel<S, R>), dim3(max_tiles * (I / 64)), dim3(256),
                     (size_t)S * (128 * kF8WRow + R * kF8ARow), st, x, slots, tiles, ntiles, wg, wu, sg, su, h, hscale,
                     H, I, K);
  return hipGetLastError();
}

template <int R>
static hipError_t gateup_fp8_r(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                               int max_tiles, const uint8_t* wg, const uint8_t* wu, const float* sg, const float* su,
                               uint16_t* h, uint8_t* hscale, int H, int I, int K, hipStream_t st) {
  constexpr int S = gateup_f8_slots(R);
  if constexpr (S == 3) {
    static std::atomic<int> fit3{-1}, fit2{-1};
    const int grid = max_tiles * (I / 64);
    if (grid > resident_blocks(reinterpret_cast<const void*>(&gateup_stream_fp8_kernel<3, R>),
                               gateup_stream_fp8_lds_bytes(R), fit3) &&
        grid <= resident_blocks(reinterpret_cast<const void*>(&gateup_stream_fp8_kernel<2, R>),
                                2 * (128 * kF8WRow + R * kF8ARow), fit2))
      return gateup_fp8_s<2, R>(x, slots, tiles, ntiles, max_tiles, wg, wu, sg, su, h, hscale, H, I, K, st);
  }
  return gateup_fp8_s<S, R>(x, slots, tiles, ntiles, max_tiles, wg, wu, sg, su, h, hscale, H, I, K, st);
}

template <int S, int R>
static hipError_t down_fp8_s(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                             const int32_t* ntiles, int max_tiles, const uint8_t* wd, const float* sd, uint16_t* y16,
                             uint8_t* yscale, int H, int I, hipStream_t st) {
  constexpr int NB = down_f8_nb(R);
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&down_stream_fp8_kernel<S, R, NB>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((down_stream_fp8_kernel<S, R, NB>), dim3(max_tiles * (H / (64 * NB))), dim3(256),
                     (size_t)S * (64 * NB * kF8WRow + R * kF8ARow) + I / kScaleCols, st, h, hscale, slots, tiles,
                     ntiles, wd, sd, y16, yscale, H, I);
  return hipGetLastError();
}

template <int R>
static hipError_t down_fp8_r(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                             const int32_t* ntiles, int max_tiles, const uint8_t* wd, const float* sd, uint16_t* y16,
                             uint8_t* yscale, int H, int I, hipStream_t st) {
  constexpr int S = down_f8_slots(R), NB = down_f8_nb(R);
  if constexpr (S == 3) {
    static std::atomic<int> fit3{-1}, fit2{-1};
    const int grid = max_tiles * (H / (64 * NB));
    if (grid > resident_blocks(reinterpret_cast<const void*>(&down_stream_fp8_kernel<3, R, NB>),
                               down_stream_fp8_lds_bytes(R, I), fit3) &&
        grid <= resident_blocks(reinterpret_cast<const void*>(&down_stream_fp8_kernel<2, R, NB>),
                                2 * (64 * NB * kF8WRow + R * kF8ARow) + I / kScaleCols, fit2))
      return down_fp8_s<2, R>(h, hscale, slots, tiles, ntiles, max_tiles, wd, sd, y16, yscale, H, I, st);
  }
  return down_fp8_s<S, R>(h, hscale, slots, tiles, ntiles, max_tiles, wd, sd, y16, yscale, H, I, st);
}

template <int S, int R>
static hipError_t gateup_s(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                           int max_tiles, const uint16_t* wg, const uint16_t* wu, uint16_t* h, uint8_t* hscale, int H,
                           int I, int K, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&gateup_stream_lds_kernel<S, kSk, R>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gateup_stream_lds_kernel<S, kSk, R>), dim3(max_tiles * (I / 64)), dim3(256),
                     (size_t)S * (128 + R) * StageGeom<kSk>::kRowBytes, st, x, slots, tiles, ntiles, wg, wu, h, hscale,
                     H, I, K);
  return hipGetLastError();
}

template <int R>
static hipError_t gateup_r(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                           int max_tiles, const uint16_t* wg, const uint16_t* wu, uint16_t* h, uint8_t* hscale, int H,
                           int I, int K, hipStream_t st) {
  constexpr int S = gateup_slots(R);
  if constexpr (S == 3) {
    static std::atomic<int> fit3{-1}, fit2{-1};
    const int grid = max_tiles * (I / 64);
    if (grid > resident_blocks(reinterpret_cast<const void*>(&gateup_stream_lds_kernel<3, kSk, R>),
                               gateup_stream_lds_bytes(R), fit3) &&
        grid <= resident_blocks(reinterpret_cast<const void*>(&gateup_stream_lds_kernel<2, kSk, R>),
                                2 * (128 + R) * StageGeom<kSk>::kRowBytes, fit2))
      return gateup_s<2, R>(x, slots, tiles, ntiles, max_tiles, wg, wu, h, hscale, H, I, K, st);
  }
  return gateup_s<S, R>(x, slots, tiles, ntiles, max_tiles, wg, wu, h, hscale, H, I, K, st);
}

template <int S, int R, bool WF16>
static hipError_t down_s(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                         const int32_t* ntiles, int max_tiles, const uint16_t* wd, uint16_t* y16, uint8_t* yscale,
                         int H, int I, hipStream_t st) {
  constexpr int NB = down_nb(R);
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e =
      allow_full_lds(reinterpret_cast<const void*>(&down_stream_lds_kernel<S, kSk, R, NB, WF16>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((down_stream_lds_kernel<S, kSk, R, NB, WF16>), dim3(max_tiles * (H / (64 * NB))), dim3(256),
                     (size_t)S * (64 * NB + R) * StageGeom<kSk>::kRowBytes + I / kScaleCols, st, h, hscale, slots,
                     tiles, ntiles, wd, y16, yscale, H, I);
  return hipGetLastError();
}

template <int R, bool WF16>
static hipError_t down_r(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                         const int32_t* ntiles, int max_tiles, const uint16_t* wd, uint16_t* y16, uint8_t* yscale,
                         int H, int I, hipStream_t st) {
  constexpr int S = down_slots(R), NB = down_nb(R);
  if constexpr (S == 3) {
    static std::atomic<int> fit3{-1}, fit2{-1};
    const int grid = max_tiles * (H / (64 * NB));
    if (grid > resident_blocks(reinterpret_cast<const void*>(&down_stream_lds_kernel<3, kSk, R, NB, WF16>),
                               down_stream_lds_bytes(R, I), fit3) &&
        grid <= resident_blocks(reinterpret_cast<const void*>(&down_stream_lds_kernel<2, kSk, R, NB, WF16>),
                                2 * (64 * NB + R) * StageGeom<kSk>::kRowBytes + I / kScaleCols, fit2))
      return down_s<2, R, WF16>(h, hscale, slots, tiles, ntiles, max_tiles, wd, y16, yscale, H, I, st);
  }
  return down_s<S, R, WF16>(h, hscale, slots, tiles, ntiles, max_tiles, wd, y16, yscale, H, I, st);
}

// Launchers of the stream path (tiles of at most R rows from the dispatch; require
// stream_fits / stream_fp8_fits).  Gate/up and down run on the same tile table: the
// down kernel reads one activation scale per (tile, 64 columns).
hipError_t launch_gateup_stream_fp8(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                                    int max_tiles, int R, const uint8_t* wg, const uint8_t* wu, const float* sg,
                                    const float* su, uint16_t* h, uint8_t* hscale, int H, int I, int K,
                                    hipStream_t st) {
  switch (R) {
    case 8: return gateup_fp8_r<8>(x, slots, tiles, ntiles, max_tiles, wg, wu, sg, su, h, hscale, H, I, K, st);
    case 16: return gateup_fp8_r<16>(x, slots, tiles, ntiles, max_tiles, wg, wu, sg, su, h, hscale, H, I, K, st);
    case 32: return gateup_fp8_r<32>(x, slots, tiles, ntiles, max_tiles, wg, wu, sg, su, h, hscale, H, I, K, st);
    case 64: return gateup_fp8_r<64>(x, slots, tiles, ntiles, max_tiles, wg, wu, sg, su, h, hscale, H, I, K, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_down_stream_fp8(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                                  const int32_t* ntiles, int max_tiles, int R, const uint8_t* wd, const float* sd,
                                  uint16_t* y16, uint8_t* yscale, int H, int I, hipStream_t st) {
  switch (R) {
    case 8: return down_fp8_r<8>(h, hscale, slots, tiles, ntiles, max_tiles, wd, sd, y16, yscale, H, I, st);
    case 16: return down_fp8_r<16>(h, hscale, slots, tiles, ntiles, max_tiles, wd, sd, y16, yscale, H, I, st);
    case 32: return down_fp8_r<32>(h, hscale, slots, tiles, ntiles, max_tiles, wd, sd, y16, yscale, H, I, st);
    case 64: return down_fp8_r<64>(h, hscale, slots, tiles, ntiles, max_tiles, wd, sd, y16, yscale, H, I, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gateup_stream(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                                int max_tiles, int R, const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                                uint8_t* hscale, int H, int I, int K, hipStream_t st) {
  switch (R) {
    case 8: return gateup_r<8>(x, slots, tiles, ntiles, max_tiles, wg, wu, h, hscale, H, I, K, st);
    case 16: return gateup_r<16>(x, slots, tiles, ntiles, max_tiles, wg, wu, h, hscale, H, I, K, st);
    case 32: return gateup_r<32>(x, slots, tiles, ntiles, max_tiles, wg, wu, h, hscale, H, I, K, st);
    case 64: return gateup_r<64>(x, slots, tiles, ntiles, max_tiles, wg, wu, h, hscale, H, I, K, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool WF16>
static hipError_t down_stream_any(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                                  const int32_t* ntiles, int max_tiles, int R, const uint16_t* wd, uint16_t* y16,
                                  uint8_t* yscale, int H, int I, hipStream_t st) {
  switch (R) {
    case 8: return down_r<8, WF16>(h, hscale, slots, tiles, ntiles, max_tiles, wd, y16, yscale, H, I, st);
    case 16: return down_r<16, WF16>(h, hscale, slots, tiles, ntiles, max_tiles, wd, y16, yscale, H, I, st);
    case 32: return down_r<32, WF16>(h, hscale, slots, tiles, ntiles, max_tiles, wd, y16, yscale, H, I, st);
    case 64: return down_r<64, WF16>(h, hscale, slots, tiles, ntiles, max_tiles, wd, y16, yscale, H, I, st);
    default: return hipErrorInvalidValue;
  }
}

// wd_f16: W_down given in fp16 (beam_moe_pack_weights) rather than bf16.
hipError_t launch_down_stream(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                              const int32_t* ntiles, int max_tiles, int R, const uint16_t* wd, bool wd_f16,
                              uint16_t* y16, uint8_t* yscale, int H, int I, hipStream_t st) {
  return wd_f16 ? down_stream_any<true>(h, hscale, slots, tiles, ntiles, max_tiles, R, wd, y16, yscale, H, I, st)
                : down_stream_any<false>(h, hscale, slots, tiles, ntiles, max_tiles, R, wd, y16, yscale, H, I, st);
}

// ---------------------------------------------------------------------------
// weight packing: bf16 -> fp16, once, for the down projection
// ---------------------------------------------------------------------------
// Each 16-byte group of 8 bf16 values becomes 8 fp16 values by exactly the
// conversion the down kernels apply as they read bf16 weights (bf16x8_to_f16x8),
// so a forward on the packed weights gives the same bits as one on the bf16
// weights.  Grid-stride over n8 groups of 8 elements.
__global__ __launch_bounds__(256) void pack_f16_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                       size_t n8) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride)
    dst[i] = bf16x8_to_f16x8(src[i]);
}

hipError_t launch_pack_f16(const uint16_t* src, uint16_t* dst, size_t n, hipStream_t st) {
  const size_t n8 = n / 8;  // n % 8 == 0: whole rows of I % 128 == 0 elements
  if (n8 == 0) return hipSuccess;
  const size_t want = (n8 + 255) / 256;
  const unsigned blocks = (unsigned)std::min<size_t>(want, 16384);
  hipLaunchKernelGGL(pack_f16_kernel, dim3(blocks), dim3(256), 0, st, reinterpret_cast<const u32x4*>(src),
                     reinterpret_cast<u32x4*>(dst), n8);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// combine: out[t] = sum_k w[t,k] * y[t*K + k], k ascending, FP32
// ---------------------------------------------------------------------------
constexpr int kCombineMaxThreads = 1024;

// grid: (T, ceil(H / (8 * blockDim.x))); from 512 tokens blockDim.x = H / 8
// rounded up to whole waves (at most 1024), so a token's row is one workgroup up
// to H = 8192; below that 256 (2048 columns per workgroup).  A
// thread owns 8 consecutive columns: the K rows of its token (fp16, each with
// its 64-column scale) are loaded together (up to 16, 16 bytes each), then
// summed in ascending k in FP32.
__global__ __launch_bounds__(kCombineMaxThreads) void combine_kernel(const uint16_t* __restrict__ y16,
                                                                     const uint8_t* __restrict__ yscale,
                                                                     const float* __restrict__ w,
                                                                     float* __restrict__ out, int H, int K) {
  const int t = blockIdx.x;
  const int c = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (c >= H) return;
  const size_t row0 = (size_t)t * K;
  const int nsb = H / kScaleCols;
  u32x4 raw[16];
  int sc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < K) {
      raw[k] = *reinterpret_cast<const u32x4*>(y16 + (row0 + k) * H + c);
      sc[k] = yscale[(row0 + k) * nsb + c / kScaleCols];
    }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < K) {
      const float wk = w[row0 + k];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = __builtin_amdgcn_ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)(raw[k][q] & 0xFFFFu)), sc[k]);
        const float hi = __builtin_amdgcn_ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)(raw[k][q] >> 16)), sc[k]);
        acc[2 * q] += wk * lo;
        acc[2 * q + 1] += wk * hi;
      }
    }
  float* o = out + (size_t)t * H + c;
  *reinterpret_cast<f32x4*>(o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
  *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

hipError_t launch_combine(const uint16_t* y16, const uint8_t* yscale, const float* w, float* out, int T, int H, int K,
                          hipStream_t st) {
  // a workgroup per token row from 512 tokens (0.321 -> 0.292 ms at T = 16384); below that,
  // rows of 2048 columns, so that a decode batch still spreads over the CUs
  const int threads = T >= 512 ? std::min(kCombineMaxThreads, (H / 8 + 63) / 64 * 64) : 256;
  const int cols = threads * 8;
  hipLaunchKernelGGL(combine_kernel, dim3(T, (H + cols - 1) / cols), dim3(threads), 0, st, y16, yscale, w, out, H, K);
  return hipGetLastError();
}

}  // namespace beam
