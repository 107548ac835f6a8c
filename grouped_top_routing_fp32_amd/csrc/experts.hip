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
// bf16's 8) with a power-of-two scale 2^-s per block of 64 columns of a pass
// of rows, s chosen so the block's largest magnitude stays below 2^15; W_down
// is converted from bf16 to fp16 exactly as it is read, and the FP32
// accumulators are kept in units of 2^s of the activation block they consume
// (rescaled exactly when s changes), so the weights never carry the scale.  y
// goes to the combine the same way: fp16 scaled by 2^-s per (row group, 64
// columns).
// Rows are processed in expert-sorted order (the dispatch permutation); a
// tile table produced by the dispatch maps workgroups to experts.
//
// With few rows per expert the step is bound by streaming each touched
// expert's weights from HBM once: a workgroup owns one expert and 64 output
// columns, each wave 16 columns over the whole K, so no cross-wave reduction
// is needed; weights and the pass's activation rows (up to 8) are copied into
// LDS in whole 256-byte row segments.  Batches with more rows per expert use
// the grouped GEMMs (grouped_gemm.hip), which read an expert's weights once
// per 256-row tile rather than once per pass.
#include <atomic>

#include <algorithm>

#include "common.h"

namespace beam {

// ---------------------------------------------------------------------------
// stream kernels (few rows per expert)
// ---------------------------------------------------------------------------
// Destination slots of this lane's rows (4 (lane / 16) + r) of a pass, read
// when the pass starts so that the loads complete under its main loop; rows
// past the pass's end read its last row and are never stored.
__device__ __forceinline__ void load_y_slots(const int32_t* __restrict__ slot_of, int nrows, int32_t (&yslot)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < 4; ++r) yslot[r] = slot_of[min((lane >> 4) * 4 + r, nrows - 1)];
}

// Writes one pass of y: fp16 bits of acc * 2^-s, s from the largest magnitude
// of the pass's rows in the workgroup's 64 columns, and s per (row, block).
__device__ __forceinline__ void store_y_pass(const f32x4& acc, int nrows, const int32_t (&yslot)[4],
                                             uint16_t* __restrict__ y16, uint8_t* __restrict__ yscale, int H,
                                             int col, float* smax) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float mx = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if ((lane >> 4) * 4 + r < nrows) mx = fmaxf(mx, fabsf(acc[r]));
  mx = wave_max(mx);
  if (lane == 0) smax[wave] = mx;
  __syncthreads();
  const int sexp = act_scale_exp(fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3])));
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = (lane >> 4) * 4 + r;
    if (row < nrows) {
      const size_t slot = (size_t)yslot[r];
      y16[slot * H + col] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(acc[r], -sexp));
      if (wave == 0 && (lane & 15) == 0) yscale[slot * (H / kScaleCols) + blockIdx.y] = (uint8_t)sexp;
    }
  }
}

int scale_cols() { return kScaleCols; }

// One expert per workgroup, 64 output columns, each wave 16 columns over the
// whole K; weights and the pass's activation rows (at most kLdsRows) reach the
// MFMAs through LDS.
// Per stage of kSk = 128 of K, the load unit copies the workgroup's weight rows
// and the activation rows into a ring slot (global_load_lds), each copy taking
// 4 rows x 256 contiguous bytes: register operand loads touch 16 rows x 64
// bytes each, which caps the stream near 6.0 TB/s, while whole 256-byte row
// segments stream at about 6.5 TB/s.  Inside a slot every row is 256 bytes and
// its 16-byte chunk c sits at position c ^ (r & 15), so the 16 rows read by one
// MFMA operand load fall on distinct banks.  A copy of row r fetches, for its
// lane at position p, the chunk p ^ (r & 15).
constexpr int kLdsRows = 8;  // activation rows per pass
constexpr int kSk = 128;     // K per stage
constexpr int kSSlots = 3;   // ring depth

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

// grid: (max_tiles, I / 64); block 256; dynamic LDS kSSlots * 136 * 256 bytes.
// Slot rows: 0..63 gate rows of the workgroup's columns, 64..127 the up rows,
// 128..135 the activation rows of the pass.
template <int SLOTS, int SK>
__global__ __launch_bounds__(256) void gateup_stream_lds_kernel(const uint16_t* __restrict__ x,
                                                                const int32_t* __restrict__ sorted_slots,
                                                                const Tile* __restrict__ tiles,
                                                                const int32_t* __restrict__ ntiles,
                                                                const uint16_t* __restrict__ wg,
                                                                const uint16_t* __restrict__ wu,
                                                                uint16_t* __restrict__ h,
                                                                uint8_t* __restrict__ hscale, int H, int I, int K) {
  using G = StageGeom<SK>;
  constexpr int kRows = 128 + kLdsRows;
  constexpr int kSlot = kRows * G::kRowBytes;
  constexpr int kWCopies = 32 / G::kRPI;  // weight copies per wave per stage (32 rows)
  constexpr int kCopies = kWCopies + 1;   // plus one copy (or part of one) of activation rows
  extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
  __shared__ float smax[4];
  if ((int)blockIdx.x >= ntiles[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = lane & 15;
  const int col = blockIdx.y * 64 + wave * 16 + m;
  const int nsb = I / kScaleCols;
  const int nst = H / SK;
  const size_t ebase = (size_t)tl.expert * I * H;

  // weight copies: wave w fills slot rows 32w .. 32w+31 (w < 2: gate, else up)
  const uint16_t* wsrc[kWCopies];
#pragma unroll
  for (int q = 0; q < kWCopies; ++q) {
    const int r = 32 * wave + G::kRPI * q + lane / G::kLPR;
    const uint16_t* base = (r < 64 ? wg : wu) + ebase + (size_t)(blockIdx.y * 64 + (r & 63)) * H;
    wsrc[q] = stage_src<SK>(base, r, lane);
  }

  for (int p = 0; p < tl.rows; p += kLdsRows) {
    const int nrows = min(kLdsRows, tl.rows - p);
    // activation copies: wave w fills activation rows 2w, 2w+1 (lanes 0 .. 2 LPR - 1)
    const int xr = 2 * wave + min(1, lane / G::kLPR);
    const int tok = sorted_slots[tl.row_start + p + min(xr, nrows - 1)] / K;
    const uint16_t* xsrc = stage_src<SK>(x + (size_t)tok * H, 128 + xr, lane);
    auto issue = [&](int st, int slot) {
      unsigned char* sl = ring + slot * kSlot;
      const int k = st * SK;
#pragma unroll
      for (int q = 0; q < kWCopies; ++q) lds_copy16(wsrc[q] + k, lds_addr(sl + (32 * wave + G::kRPI * q) * G::kRowBytes));
      if (lane < 2 * G::kLPR) lds_copy16(xsrc + k, lds_addr(sl + (128 + 2 * wave) * G::kRowBytes));
    };
    f32x4 ag = f32x4{0.f, 0.f, 0.f, 0.f}, au = ag;
    const bool rv = m < nrows;
    const int arow = 128 + (rv ? m : 0);
    const int grow = wave * 16 + m, urow = 64 + wave * 16 + m;
#pragma unroll
    for (int s = 0; s < SLOTS - 1; ++s)
      if (s < nst) issue(s, s);
    for (int st = 0; st < nst; ++st) {
      const int later = min(SLOTS - 2, nst - 1 - st);  // stages requested after stage st
      if (later >= 2)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kCopies));
      else if (later == 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCopies));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();  // stage st complete for all waves; stage st - 1's slot is free
      if (st + SLOTS - 1 < nst) issue(st + SLOTS - 1, (st + SLOTS - 1) % SLOTS);
      const unsigned char* sl = ring + (st % SLOTS) * kSlot;
#pragma unroll
      for (int s = 0; s < SK / 32; ++s) {
        const int c = 4 * s + (lane >> 4);
        const u32x4 a = *reinterpret_cast<const u32x4*>(sl + stage_off<SK>(arow, c));
        const u32x4 g = *reinterpret_cast<const u32x4*>(sl + stage_off<SK>(grow, c));
        const u32x4 u = *reinterpret_cast<const u32x4*>(sl + stage_off<SK>(urow, c));
        const u32x4 az = rv ? a : u32x4{0u, 0u, 0u, 0u};
        ag = mfma16x16x32(az, g, ag);
        au = mfma16x16x32(az, u, au);
      }
    }
    // SwiGLU in FP32; one power-of-two scale per (pass, 64 columns)
    float v[4];
    float mx = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (lane >> 4) * 4 + r;
      v[r] = (row < nrows) ? silu_f32(ag[r]) * au[r] : 0.f;
      mx = fmaxf(mx, fabsf(v[r]));
    }
    mx = wave_max(mx);
    if (lane == 0) smax[wave] = mx;
    __syncthreads();  // also: every wave is done with the ring before the next pass refills it
    const int sexp = act_scale_exp(fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3])));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (lane >> 4) * 4 + r;
      if (row < nrows) {
        const size_t gr = (size_t)(tl.row_start + p + row);
        h[gr * I + col] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(v[r], -sexp));
        if (wave == 0 && m == 0) hscale[gr * nsb + blockIdx.y] = (uint8_t)sexp;
      }
    }
    __syncthreads();  // smax is rewritten by the next pass
  }
}

// grid: (max_tiles, H / 64); block 256; dynamic LDS SLOTS * 72 * 256 bytes + the
// pass's scales.  y leaves through store_y_pass.  Slot rows: 0..63 W_down rows of the workgroup's columns,
// 64..71 the activation rows (h, fp16) of the pass.
template <int SLOTS, int SK>
__global__ __launch_bounds__(256) void down_stream_lds_kernel(const uint16_t* __restrict__ h,
                                                              const uint8_t* __restrict__ hscale,
                                                              const int32_t* __restrict__ sorted_slots,
                                                              const Tile* __restrict__ tiles,
                                                              const int32_t* __restrict__ ntiles,
                                                              const uint16_t* __restrict__ wd,
                                                              uint16_t* __restrict__ y16,
                                                              uint8_t* __restrict__ yscale, int H, int I) {
  using G = StageGeom<SK>;
  constexpr int kRows = 64 + kLdsRows;
  constexpr int kSlot = kRows * G::kRowBytes;
  constexpr int kWCopies = 16 / G::kRPI;  // weight copies per wave per stage (16 rows)
  constexpr int kCopies = kWCopies + 1;   // plus one copy (or part of one) of activation rows
  extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
  __shared__ int sany;
  __shared__ float smax[4];
  uint8_t* ssc = ring + SLOTS * kSlot;  // the pass's activation scales
  if ((int)blockIdx.x >= ntiles[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 15;
  const int col = blockIdx.y * 64 + wave * 16 + m;
  const int nsb = I / kScaleCols;
  const int nst = I / SK;

  const uint16_t* wsrc[kWCopies];
#pragma unroll
  for (int q = 0; q < kWCopies; ++q) {
    const int r = 16 * wave + G::kRPI * q + lane / G::kLPR;
    const uint16_t* base = wd + (size_t)tl.expert * H * I + (size_t)(blockIdx.y * 64 + r) * I;
    wsrc[q] = stage_src<SK>(base, r, lane);
  }

  for (int p = 0; p < tl.rows; p += kLdsRows) {
    const int nrows = min(kLdsRows, tl.rows - p);
    int32_t yslot[4];
    load_y_slots(sorted_slots + tl.row_start + p, nrows, yslot);
    const int xr = 2 * wave + min(1, lane / G::kLPR);
    const uint16_t* xsrc = stage_src<SK>(h + (size_t)(tl.row_start + p + min(xr, nrows - 1)) * I, 64 + xr, lane);
    auto issue = [&](int st, int slot) {
      unsigned char* sl = ring + slot * kSlot;
      const int k = st * SK;
#pragma unroll
      for (int q = 0; q < kWCopies; ++q) lds_copy16(wsrc[q] + k, lds_addr(sl + (16 * wave + G::kRPI * q) * G::kRowBytes));
      if (lane < 2 * G::kLPR) lds_copy16(xsrc + k, lds_addr(sl + (64 + 2 * wave) * G::kRowBytes));
    };
#pragma unroll
    for (int s = 0; s < SLOTS - 1; ++s)
      if (s < nst) issue(s, s);
    if (tid == 0) sany = 0;
    __syncthreads();
    for (int i = tid; i < nsb; i += 256) {
      const uint8_t sv = hscale[(size_t)(tl.row_start + p) * nsb + i];
      ssc[i] = sv;
      if (sv) sany = 1;
    }
    __syncthreads();
    const bool scaled = sany != 0;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool rv = m < nrows;
    const int arow = 64 + (rv ? m : 0);
    const int brow = wave * 16 + m;
    int s_acc = 0;  // acc holds y * 2^-s_acc (the activation block consumed last)
    for (int st = 0; st < nst; ++st) {
      const int later = min(SLOTS - 2, nst - 1 - st);
      if (later >= 2)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kCopies));
      else if (later == 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCopies));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
      if (st + SLOTS - 1 < nst) issue(st + SLOTS - 1, (st + SLOTS - 1) % SLOTS);
      const unsigned char* sl = ring + (st % SLOTS) * kSlot;
#pragma unroll
      for (int s = 0; s < SK / 32; ++s) {
        const int c = 4 * s + (lane >> 4);
        const u32x4 a = *reinterpret_cast<const u32x4*>(sl + stage_off<SK>(arow, c));
        const u32x4 b = *reinterpret_cast<const u32x4*>(sl + stage_off<SK>(brow, c));
        if (scaled) {
          const int sk = __builtin_amdgcn_readfirstlane(ssc[(st * SK + 32 * s) / kScaleCols]);
          if (sk != s_acc) {
            acc = ldexp4(acc, s_acc - sk);
            s_acc = sk;
          }
        }
        acc = mfma16x16x32_f16(rv ? a : u32x4{0u, 0u, 0u, 0u}, bf16x8_to_f16x8(b), acc);
      }
    }
    acc = ldexp4(acc, s_acc);
    store_y_pass(acc, nrows, yslot, y16, yscale, H, col, smax);
    __syncthreads();  // every wave is done with the ring and the scales before the next pass
  }
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
// MFMAs accumulate in FP32 and the row scale multiplies the accumulator.  Half the
// bytes of the bf16 weights for the same arithmetic.
//
// Stage of kF8Sk = 256 of K: weight rows of 256 bytes (256 codes) and
// activation rows of 512 bytes (256 bf16 / fp16 values), both with 16-byte
// chunk c of row r at position c ^ (r & 15) (activation rows keyed by their
// index 0..7).  Per 64 of K a lane reads one 16-byte chunk of codes (16 K
// values) and the two matching 16-byte chunks of its activation row: two
// MFMAs of K = 32, the first on the chunk's 8 low codes, the second on its
// 8 high ones.  A and B agree on which K each operand slot holds, which is
// all a contraction needs.
constexpr int kF8Sk = 256;     // K per stage
constexpr int kF8WRow = 256;   // bytes of a staged weight row
constexpr int kF8ARow = 512;   // bytes of a staged activation row
constexpr int kF8Slots = 3;    // ring depth

__device__ __forceinline__ int f8_woff(int row, int chunk) { return row * kF8WRow + ((chunk ^ (row & 15)) << 4); }
__device__ __forceinline__ int f8_aoff(int row, int chunk) { return row * kF8ARow + ((chunk ^ (row & 15)) << 4); }

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

// grid: (max_tiles, I / 64); block 256; dynamic LDS SLOTS * (128 * 256 + 8 * 512) bytes.
// Slot: 128 weight rows (0..63 gate, 64..127 up, of the workgroup's columns), then
// the pass's 8 activation rows.
template <int SLOTS>
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
  constexpr int kWBytes = 128 * kF8WRow;
  constexpr int kSlot = kWBytes + kLdsRows * kF8ARow;
  constexpr int kWCopies = 8;            // 32 weight rows of 256 bytes per wave: 4 rows per copy
  constexpr int kCopies = kWCopies + 1;  // plus two activation rows of 512 bytes
  extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
  __shared__ float smax[4];
  if ((int)blockIdx.x >= ntiles[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = lane & 15;
  const int col = blockIdx.y * 64 + wave * 16 + m;
  const int nsb = I / kScaleCols;
  const int nst = H / kF8Sk;
  const size_t ebase = (size_t)tl.expert * I * H;

  // weight copies: wave w fills slot rows 32w .. 32w+31 (w < 2: gate, else up), 16 lanes a row
  const uint8_t* wsrc[kWCopies];
#pragma unroll
  for (int q = 0; q < kWCopies; ++q) {
    const int r = 32 * wave + 4 * q + (lane >> 4);
    const uint8_t* base = (r < 64 ? wg : wu) + ebase + (size_t)(blockIdx.y * 64 + (r & 63)) * H;
    wsrc[q] = base + (((lane & 15) ^ (r & 15)) << 4);
  }
  const float scale_g = sg[(size_t)tl.expert * I + col];
  const float scale_u = su[(size_t)tl.expert * I + col];

  for (int p = 0; p < tl.rows; p += kLdsRows) {
    const int nrows = min(kLdsRows, tl.rows - p);
    // activation copy: wave w fills activation rows 2w, 2w+1, 32 lanes a row
    const int xr = 2 * wave + (lane >> 5);
    const int tok = sorted_slots[tl.row_start + p + min(xr, nrows - 1)] / K;
    const unsigned char* xsrc =
        reinterpret_cast<const unsigned char*>(x + (size_t)tok * H) + (((lane & 31) ^ (xr & 15)) << 4);
    auto issue = [&](int st, int slot) {
      unsigned char* sl = ring + slot * kSlot;
#pragma unroll
      for (int q = 0; q < kWCopies; ++q)
        lds_copy16(wsrc[q] + (size_t)st * kF8Sk, lds_addr(sl + (32 * wave + 4 * q) * kF8WRow));
      lds_copy16(xsrc + (size_t)st * kF8Sk * 2, lds_addr(sl + kWBytes + 2 * wave * kF8ARow));
    };
    f32x4 ag = f32x4{0.f, 0.f, 0.f, 0.f}, au = ag;
    const bool rv = m < nrows;
    const int arow = rv ? m : 0;
    const int grow = wave * 16 + m, urow = 64 + wave * 16 + m;
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < SLOTS - 1; ++s)
      if (s < nst) issue(s, s);
    for (int st = 0; st < nst; ++st) {
      const int later = min(SLOTS - 2, nst - 1 - st);  // stages requested after stage st
      if (later >= 2)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kCopies));
      else if (later == 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCopies));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();  // stage st complete for all waves; stage st - 1's slot is free
      if (st + SLOTS - 1 < nst) issue(st + SLOTS - 1, (st + SLOTS - 1) % SLOTS);
      const unsigned char* sl = ring + (st % SLOTS) * kSlot;
      const unsigned char* sa = sl + kWBytes;
#pragma unroll
      for (int j = 0; j < kF8Sk / 64; ++j) {
        const int cw = 4 * j + (lane >> 4);
        const u32x4 gq = *reinterpret_cast<const u32x4*>(sl + f8_woff(grow, cw));
        const u32x4 uq = *reinterpret_cast<const u32x4*>(sl + f8_woff(urow, cw));
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(sa + f8_aoff(arow, 2 * cw));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(sa + f8_aoff(arow, 2 * cw + 1));
        u32x4 g0, g1, u0, u1;
        fp8x16_to_bf16(gq, g0, g1);
        fp8x16_to_bf16(uq, u0, u1);
        const u32x4 az0 = rv ? a0 : zero, az1 = rv ? a1 : zero;
        ag = mfma16x16x32(az0, g0, ag);
        au = mfma16x16x32(az0, u0, au);
        ag = mfma16x16x32(az1, g1, ag);
        au = mfma16x16x32(az1, u1, au);
      }
    }
    // row scales, then SwiGLU in FP32; one power-of-two scale per (pass, 64 columns)
    float v[4];
    float mx = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (lane >> 4) * 4 + r;
      v[r] = (row < nrows) ? silu_f32(ag[r] * scale_g) * (au[r] * scale_u) : 0.f;
      mx = fmaxf(mx, fabsf(v[r]));
    }
    mx = wave_max(mx);
    if (lane == 0) smax[wave] = mx;
    __syncthreads();  // also: every wave is done with the ring before the next pass refills it
    const int sexp = act_scale_exp(fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3])));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (lane >> 4) * 4 + r;
      if (row < nrows) {
        const size_t gr = (size_t)(tl.row_start + p + row);
        h[gr * I + col] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(v[r], -sexp));
        if (wave == 0 && m == 0) hscale[gr * nsb + blockIdx.y] = (uint8_t)sexp;
      }
    }
    __syncthreads();  // smax is rewritten by the next pass
  }
}

// grid: (max_tiles, H / 64); block 256; dynamic LDS SLOTS * (64 * 256 + 8 * 512) bytes + the
// pass's scales.  Slot: 64 W_down rows of the workgroup's columns, then the pass's 8 h rows.
template <int SLOTS>
__global__ __launch_bounds__(256) void down_stream_fp8_kernel(const uint16_t* __restrict__ h,
                                                              const uint8_t* __restrict__ hscale,
                                                              const int32_t* __restrict__ sorted_slots,
                                                              const Tile* __restrict__ tiles,
                                                              const int32_t* __restrict__ ntiles,
                                                              const uint8_t* __restrict__ wd,
                                                              const float* __restrict__ sd,
                                                              uint16_t* __restrict__ y16,
                                                              uint8_t* __restrict__ yscale, int H, int I) {
  constexpr int kWBytes = 64 * kF8WRow;
  constexpr int kSlot = kWBytes + kLdsRows * kF8ARow;
  constexpr int kWCopies = 4;            // 16 weight rows of 256 bytes per wave
  constexpr int kCopies = kWCopies + 1;  // plus two activation rows of 512 bytes
  extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
  __shared__ int sany;
  __shared__ float smax[4];
  uint8_t* ssc = ring + SLOTS * kSlot;  // the pass's activation scales
  if ((int)blockIdx.x >= ntiles[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 15;
  const int col = blockIdx.y * 64 + wave * 16 + m;
  const int nsb = I / kScaleCols;
  const int nst = I / kF8Sk;

  const uint8_t* wsrc[kWCopies];
#pragma unroll
  for (int q = 0; q < kWCopies; ++q) {
    const int r = 16 * wave + 4 * q + (lane >> 4);
    const uint8_t* base = wd + (size_t)tl.expert * H * I + (size_t)(blockIdx.y * 64 + r) * I;
    wsrc[q] = base + (((lane & 15) ^ (r & 15)) << 4);
  }
  const float scale_d = sd[(size_t)tl.expert * H + col];

  for (int p = 0; p < tl.rows; p += kLdsRows) {
    const int nrows = min(kLdsRows, tl.rows - p);
    int32_t yslot[4];
    load_y_slots(sorted_slots + tl.row_start + p, nrows, yslot);
    const int xr = 2 * wave + (lane >> 5);
    const unsigned char* xsrc =
        reinterpret_cast<const unsigned char*>(h + (size_t)(tl.row_start + p + min(xr, nrows - 1)) * I) +
        (((lane & 31) ^ (xr & 15)) << 4);
    auto issue = [&](int st, int slot) {
      unsigned char* sl = ring + slot * kSlot;
#pragma unroll
      for (int q = 0; q < kWCopies; ++q)
        lds_copy16(wsrc[q] + (size_t)st * kF8Sk, lds_addr(sl + (16 * wave + 4 * q) * kF8WRow));
      lds_copy16(xsrc + (size_t)st * kF8Sk * 2, lds_addr(sl + kWBytes + 2 * wave * kF8ARow));
    };
#pragma unroll
    for (int s = 0; s < SLOTS - 1; ++s)
      if (s < nst) issue(s, s);
    if (tid == 0) sany = 0;
    __syncthreads();
    for (int i = tid; i < nsb; i += 256) {
      const uint8_t sv = hscale[(size_t)(tl.row_start + p) * nsb + i];
      ssc[i] = sv;
      if (sv) sany = 1;
    }
    __syncthreads();
    const bool scaled = sany != 0;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool rv = m < nrows;
    const int arow = rv ? m : 0;
    const int brow = wave * 16 + m;
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
    int s_acc = 0;  // acc holds y * 2^-s_acc (the activation block consumed last)
    for (int st = 0; st < nst; ++st) {
      const int later = min(SLOTS - 2, nst - 1 - st);
      if (later >= 2)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kCopies));
      else if (later == 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCopies));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
      if (st + SLOTS - 1 < nst) issue(st + SLOTS - 1, (st + SLOTS - 1) % SLOTS);
      const unsigned char* sl = ring + (st % SLOTS) * kSlot;
      const unsigned char* sa = sl + kWBytes;
#pragma unroll
      for (int j = 0; j < kF8Sk / 64; ++j) {
        const int cw = 4 * j + (lane >> 4);
        const u32x4 bq = *reinterpret_cast<const u32x4*>(sl + f8_woff(brow, cw));
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(sa + f8_aoff(arow, 2 * cw));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(sa + f8_aoff(arow, 2 * cw + 1));
        // the 64 K values of step j share one activation scale block
        if (scaled) {
          const int sk = __builtin_amdgcn_readfirstlane(ssc[(st * kF8Sk) / kScaleCols + j]);
          if (sk != s_acc) {
            acc = ldexp4(acc, s_acc - sk);
            s_acc = sk;
          }
        }
        u32x4 b0, b1;
        fp8x16_to_f16(bq, b0, b1);
        acc = mfma16x16x32_f16(rv ? a0 : zero, b0, acc);
        acc = mfma16x16x32_f16(rv ? a1 : zero, b1, acc);
      }
    }
    acc = ldexp4(acc, s_acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] *= scale_d;
    store_y_pass(acc, nrows, yslot, y16, yscale, H, col, smax);
    __syncthreads();  // every wave is done with the ring and the scales before the next pass
  }
}

// Dynamic LDS the stream kernels may take: 128 KB of a gfx950 CU's 160 KB,
// leaving room for their small static arrays.
constexpr size_t kStreamLdsMax = 128 * 1024;

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

size_t gateup_stream_lds_bytes() { return (size_t)kSSlots * (128 + kLdsRows) * StageGeom<kSk>::kRowBytes; }
size_t down_stream_lds_bytes(int I) {
  return (size_t)kSSlots * (64 + kLdsRows) * StageGeom<kSk>::kRowBytes + I / kScaleCols;
}

// Whether the stream kernels can run at this shape: K of both projections in
// whole stages, and the staged rows and the down kernel's scales fit in LDS.
bool stream_fits(int H, int I) {
  return H % kSk == 0 && I % kSk == 0 && gateup_stream_lds_bytes() <= kStreamLdsMax &&
         down_stream_lds_bytes(I) <= kStreamLdsMax;
}

size_t gateup_stream_fp8_lds_bytes() { return (size_t)kF8Slots * (128 * kF8WRow + kLdsRows * kF8ARow); }
size_t down_stream_fp8_lds_bytes(int I) {
  return (size_t)kF8Slots * (64 * kF8WRow + kLdsRows * kF8ARow) + I / kScaleCols;
}

// Whether the FP8 stream kernels can run at this shape: K of both projections
// in whole 256-value stages, and the staged rows and scales fit in LDS.
bool stream_fp8_fits(int H, int I) {
  return H % kF8Sk == 0 && I % kF8Sk == 0 && gateup_stream_fp8_lds_bytes() <= kStreamLdsMax &&
         down_stream_fp8_lds_bytes(I) <= kStreamLdsMax;
}

hipError_t launch_gateup_stream_fp8(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                                    int max_tiles, const uint8_t* wg, const uint8_t* wu, const float* sg,
                                    const float* su, uint16_t* h, uint8_t* hscale, int H, int I, int K,
                                    hipStream_t st) {
  dim3 grid(max_tiles, I / 64);
  const size_t bytes = gateup_stream_fp8_lds_bytes();
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&gateup_stream_fp8_kernel<kF8Slots>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gateup_stream_fp8_kernel<kF8Slots>), grid, dim3(256), bytes, st, x, slots, tiles, ntiles, wg,
                     wu, sg, su, h, hscale, H, I, K);
  return hipGetLastError();
}

hipError_t launch_down_stream_fp8(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                                  const int32_t* ntiles, int max_tiles, const uint8_t* wd, const float* sd,
                                  uint16_t* y16, uint8_t* yscale, int H, int I, hipStream_t st) {
  dim3 grid(max_tiles, H / 64);
  const size_t bytes = down_stream_fp8_lds_bytes(I);
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&down_stream_fp8_kernel<kF8Slots>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((down_stream_fp8_kernel<kF8Slots>), grid, dim3(256), bytes, st, h, hscale, slots, tiles,
                     ntiles, wd, sd, y16, yscale, H, I);
  return hipGetLastError();
}

// Launchers of the stream path (passes of kLdsRows rows; requires stream_fits).
// Gate/up and down run together: the down kernel reads one activation scale per
// pass of gate/up.
hipError_t launch_gateup_stream(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                                int max_tiles, const uint16_t* wg, const uint16_t* wu, uint16_t* h, uint8_t* hscale,
                                int H, int I, int K, hipStream_t st) {
  dim3 grid(max_tiles, I / 64);  // I % 64 == 0
  const size_t bytes = gateup_stream_lds_bytes();
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&gateup_stream_lds_kernel<kSSlots, kSk>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gateup_stream_lds_kernel<kSSlots, kSk>), grid, dim3(256), bytes, st, x, slots, tiles, ntiles,
                     wg, wu, h, hscale, H, I, K);
  return hipGetLastError();
}

hipError_t launch_down_stream(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                              const int32_t* ntiles, int max_tiles, const uint16_t* wd, uint16_t* y16,
                              uint8_t* yscale, int H, int I, hipStream_t st) {
  dim3 grid(max_tiles, H / 64);  // H % 64 == 0
  const size_t bytes = down_stream_lds_bytes(I);
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&down_stream_lds_kernel<kSSlots, kSk>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((down_stream_lds_kernel<kSSlots, kSk>), grid, dim3(256), bytes, st, h, hscale, slots, tiles,
                     ntiles, wd, y16, yscale, H, I);
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
