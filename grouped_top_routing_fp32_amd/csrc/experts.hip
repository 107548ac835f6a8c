// Expert kernels of the Beam MoE block for batches with few rows per expert
// (decode), and the weighted combine (gfx950, FP32 accumulation).
//
// "Welcome Beam: a 501B open model you can own, customize, and scale", its
// mixture-of-experts paragraph, and the Chinese translation of that post,
// 「Reflection 发布 Beam 501B 开源模型，支持 1M tokens 上下文」, section 专家混合模型:
// each expert is a SwiGLU MLP with intermediate size 2560 (hidden 5120);
// section 残差流 (residual stream): the SwiGLU product is computed in FP32.  Per expert e and routed row r:
//   h[r] = silu(W_gate[e] x[r]) * (W_up[e] x[r])   bf16 MFMA, SwiGLU in FP32
//   y[r] = W_down[e] h[r]                           fp16 MFMA, FP32 out
// h is handed to the down projection as fp16 (11 significant bits against
// bf16's 8) with a power-of-two scale 2^-s per block of 64 columns of a pass
// of rows, s chosen so the block's largest magnitude stays below 2^15; W_down
// is converted from bf16 to fp16 exactly (times 2^s) as it is loaded.
// Rows are processed in expert-sorted order (the dispatch permutation); a
// tile table produced by the dispatch maps workgroups to experts.
//
// With few rows per expert the step is bound by streaming each touched
// expert's weights from HBM once: a workgroup owns one expert and 64 output
// columns, each wave 16 columns over the whole K, so no cross-wave reduction
// is needed, and weights go from memory straight into MFMA operand registers.
//   *_stream_kernel      activation operands loaded from memory with the
//                        weights; passes of 16 rows
//   *_stream_lds_kernel  activation rows of a pass (up to 8) staged in LDS
//                        first, so the K loop issues only weight loads
// Batches with many rows per expert use the grouped GEMMs (grouped_gemm.hip).
#include "common.h"

namespace beam {

constexpr int kMaxScaleBlocks = 512;  // I <= 32768

// ---------------------------------------------------------------------------
// stream kernels, register operands
// ---------------------------------------------------------------------------
// Loads run U MFMA steps ahead of the math (two register stages) and use
// ordinary cached loads: a 16-byte operand load touches half of a 128-byte line,
// and the other half is read by the next step.
constexpr int kStreamRows = 16;  // rows per pass

// grid: (max_tiles, I / 64); block 256.  One tile = all rows of one expert.
// Writes h (fp16 bits, scaled by 2^-s) and s per (row, 64-column block).
template <int U>
__global__ __launch_bounds__(256) void gateup_stream_kernel(const uint16_t* __restrict__ x,
                                                            const int32_t* __restrict__ sorted_slots,
                                                            const Tile* __restrict__ tiles,
                                                            const int32_t* __restrict__ ntiles,
                                                            const uint16_t* __restrict__ wg,
                                                            const uint16_t* __restrict__ wu,
                                                            uint16_t* __restrict__ h, uint8_t* __restrict__ hscale,
                                                            int H, int I, int K) {
  __shared__ float smax[4];
  if ((int)blockIdx.x >= ntiles[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = blockIdx.y * 64 + wave * 16 + (lane & 15);
  const int kk = (lane >> 4) * 8;
  const size_t ebase = (size_t)tl.expert * I * H;
  const uint16_t* pg = wg + ebase + (size_t)col * H + kk;
  const uint16_t* pu = wu + ebase + (size_t)col * H + kk;
  const int nsb = I / kScaleCols;
  const int steps = H / (32 * U);

  for (int p = 0; p < tl.rows; p += kStreamRows) {
    const int m = lane & 15;
    const bool rv = p + m < tl.rows;
    const int tok = rv ? sorted_slots[tl.row_start + p + m] / K : 0;
    const uint16_t* pa = x + (size_t)tok * H + kk;
    f32x4 ag = f32x4{0.f, 0.f, 0.f, 0.f}, au = ag;
    u32x4 g0[U], u0[U], a0[U], g1[U], u1[U], a1[U];
    auto load = [&](u32x4(&g)[U], u32x4(&uu)[U], u32x4(&a)[U], int k) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        g[u] = ldg16(pg + k + 32 * u);
        uu[u] = ldg16(pu + k + 32 * u);
        a[u] = rv ? ldg16(pa + k + 32 * u) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto math = [&](u32x4(&g)[U], u32x4(&uu)[U], u32x4(&a)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ag = mfma16x16x32(a[u], g[u], ag);
        au = mfma16x16x32(a[u], uu[u], au);
      }
    };
    load(g0, u0, a0, 0);
    for (int s = 0; s < steps; s += 2) {
      if (s + 1 < steps) load(g1, u1, a1, (s + 1) * 32 * U);
      math(g0, u0, a0);
      if (s + 2 < steps) load(g0, u0, a0, (s + 2) * 32 * U);
      if (s + 1 < steps) math(g1, u1, a1);
    }
    // SwiGLU in FP32; one power-of-two scale per (16-row pass, 64 columns)
    float v[4];
    float mx = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (lane >> 4) * 4 + r;
      v[r] = (p + row < tl.rows) ? silu_f32(ag[r]) * au[r] : 0.f;
      mx = fmaxf(mx, fabsf(v[r]));
    }
    mx = wave_max(mx);
    if (lane == 0) smax[wave] = mx;
    __syncthreads();
    const int sexp = act_scale_exp(fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3])));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (lane >> 4) * 4 + r;
      if (p + row < tl.rows) {
        const size_t grow = (size_t)(tl.row_start + p + row);
        h[grow * I + col] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(v[r], -sexp));
        if (wave == 0 && (lane & 15) == 0) hscale[grow * nsb + blockIdx.y] = (uint8_t)sexp;
      }
    }
    __syncthreads();  // smax is rewritten by the next pass
  }
}

// grid: (max_tiles, H / 64); block 256.  y[slot] = W_down[e] h (fp16 MFMA,
// W_down converted exactly from bf16 and scaled back by 2^s per 64-column
// block of h).
template <int U>
__global__ __launch_bounds__(256) void down_stream_kernel(const uint16_t* __restrict__ h,
                                                          const uint8_t* __restrict__ hscale,
                                                          const int32_t* __restrict__ sorted_slots,
                                                          const Tile* __restrict__ tiles,
                                                          const int32_t* __restrict__ ntiles,
                                                          const uint16_t* __restrict__ wd, float* __restrict__ y,
                                                          int H, int I) {
  __shared__ uint8_t ssc[kMaxScaleBlocks];
  __shared__ int sany;
  if ((int)blockIdx.x >= ntiles[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = blockIdx.y * 64 + wave * 16 + (lane & 15);
  const int kk = (lane >> 4) * 8;
  const uint16_t* pb = wd + (size_t)tl.expert * H * I + (size_t)col * I + kk;
  const int nsb = I / kScaleCols;
  const int steps = I / (32 * U);

  for (int p = 0; p < tl.rows; p += kStreamRows) {
    const int m = lane & 15;
    const bool rv = p + m < tl.rows;
    const uint16_t* pa = h + (size_t)(tl.row_start + p + (rv ? m : 0)) * I + kk;
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
    u32x4 b0[U], a0[U], b1[U], a1[U];
    auto load = [&](u32x4(&b)[U], u32x4(&a)[U], int k) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        b[u] = ldg16(pb + k + 32 * u);
        a[u] = rv ? ldg16(pa + k + 32 * u) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto math = [&](u32x4(&b)[U], u32x4(&a)[U], int k) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const u32x4 bh = scaled ? bf16x8_to_f16x8_scaled(b[u], ssc[(k + 32 * u) / kScaleCols]) : bf16x8_to_f16x8(b[u]);
        acc = mfma16x16x32_f16(a[u], bh, acc);
      }
    };
    load(b0, a0, 0);
    for (int s = 0; s < steps; s += 2) {
      if (s + 1 < steps) load(b1, a1, (s + 1) * 32 * U);
      math(b0, a0, s * 32 * U);
      if (s + 2 < steps) load(b0, a0, (s + 2) * 32 * U);
      if (s + 1 < steps) math(b1, a1, (s + 1) * 32 * U);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (lane >> 4) * 4 + r;
      if (p + row < tl.rows) y[(size_t)sorted_slots[tl.row_start + p + row] * H + col] = acc[r];
    }
    __syncthreads();  // ssc and sany are rewritten by the next pass
  }
}

int scale_cols() { return kScaleCols; }

// ---------------------------------------------------------------------------
// stream kernels with the activation rows staged in LDS (very few rows per expert)
// ---------------------------------------------------------------------------
// Same work split as the register-operand kernels, but a pass takes at most 8 rows and copies them, whole-K, into
// LDS once; the K loop then issues only weight loads to memory and reads its
// activation operands from LDS.  Rows are padded by 8 elements so the 8 rows
// of one operand read fall on distinct banks.  Rows 8..15 of each MFMA operand
// are zero.  The pass size (8) is shared with the matching down kernel, which
// relies on it for the activation scales.
constexpr int kLdsRows = 8;

// Copies rows [0, nrows) of the pass into LDS (row stride K + 8 elements);
// src_row(r) gives the global row start.  256 threads, four 16-byte chunks in flight each.
template <typename RowFn>
__device__ __forceinline__ void stage_rows(uint16_t* lds, int nrows, int Kdim, RowFn src_row) {
  const int per_row = Kdim / 8;
  const int total = nrows * per_row;
  for (int c0 = threadIdx.x; c0 < total; c0 += 4 * 256) {
    u32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + q * 256;
      if (c < total) v[q] = ldg16(src_row(c / per_row) + (c % per_row) * 8);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + q * 256;
      if (c < total) *reinterpret_cast<u32x4*>(&lds[(c / per_row) * (Kdim + 8) + (c % per_row) * 8]) = v[q];
    }
  }
}

template <int U, int R>
__global__ __launch_bounds__(256) void gateup_stream_lds_kernel(const uint16_t* __restrict__ x,
                                                                const int32_t* __restrict__ sorted_slots,
                                                                const Tile* __restrict__ tiles,
                                                                const int32_t* __restrict__ ntiles,
                                                                const uint16_t* __restrict__ wg,
                                                                const uint16_t* __restrict__ wu,
                                                                uint16_t* __restrict__ h,
                                                                uint8_t* __restrict__ hscale, int H, int I, int K) {
  extern __shared__ __attribute__((aligned(16))) uint16_t sx[];  // R x (H + 8)
  __shared__ float smax[4];
  if ((int)blockIdx.x >= ntiles[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = blockIdx.y * 64 + wave * 16 + (lane & 15);
  const int kk = (lane >> 4) * 8;
  const size_t ebase = (size_t)tl.expert * I * H;
  const uint16_t* pg = wg + ebase + (size_t)col * H + kk;
  const uint16_t* pu = wu + ebase + (size_t)col * H + kk;
  const int nsb = I / kScaleCols;
  const int steps = H / (32 * U);
  const int m = lane & 15;

  for (int p = 0; p < tl.rows; p += R) {
    const int nrows = min(R, tl.rows - p);
    const bool rv = m < nrows;
    const uint16_t* pa = sx + (rv ? m : 0) * (H + 8) + kk;
    f32x4 ag = f32x4{0.f, 0.f, 0.f, 0.f}, au = ag;
    u32x4 g0[U], u0[U], a[U], g1[U], u1[U];
    auto load = [&](u32x4(&g)[U], u32x4(&uu)[U], int k) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        g[u] = ldg16(pg + k + 32 * u);
        uu[u] = ldg16(pu + k + 32 * u);
      }
    };
    auto math = [&](u32x4(&g)[U], u32x4(&uu)[U], int k) {
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = rv ? *reinterpret_cast<const u32x4*>(pa + k + 32 * u) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ag = mfma16x16x32(a[u], g[u], ag);
        au = mfma16x16x32(a[u], uu[u], au);
      }
    };
    load(g0, u0, 0);  // the first weights are on their way while the rows are staged
    stage_rows(sx, nrows, H, [&](int r) { return x + (size_t)(sorted_slots[tl.row_start + p + r] / K) * H; });
    __syncthreads();
    for (int s = 0; s < steps; s += 2) {
      if (s + 1 < steps) load(g1, u1, (s + 1) * 32 * U);
      math(g0, u0, s * 32 * U);
      if (s + 2 < steps) load(g0, u0, (s + 2) * 32 * U);
      if (s + 1 < steps) math(g1, u1, (s + 1) * 32 * U);
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
    __syncthreads();  // also: every wave is done reading sx before the next pass restages it
    const int sexp = act_scale_exp(fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3])));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (lane >> 4) * 4 + r;
      if (row < nrows) {
        const size_t grow = (size_t)(tl.row_start + p + row);
        h[grow * I + col] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(v[r], -sexp));
        if (wave == 0 && (lane & 15) == 0) hscale[grow * nsb + blockIdx.y] = (uint8_t)sexp;
      }
    }
    __syncthreads();  // smax is rewritten by the next pass
  }
}

template <int U, int R>
__global__ __launch_bounds__(256) void down_stream_lds_kernel(const uint16_t* __restrict__ h,
                                                              const uint8_t* __restrict__ hscale,
                                                              const int32_t* __restrict__ sorted_slots,
                                                              const Tile* __restrict__ tiles,
                                                              const int32_t* __restrict__ ntiles,
                                                              const uint16_t* __restrict__ wd, float* __restrict__ y,
                                                              int H, int I) {
  extern __shared__ __attribute__((aligned(16))) uint16_t sh[];  // R x (I + 8), then the scales
  __shared__ int sany;
  if ((int)blockIdx.x >= ntiles[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = blockIdx.y * 64 + wave * 16 + (lane & 15);
  const int kk = (lane >> 4) * 8;
  const uint16_t* pb = wd + (size_t)tl.expert * H * I + (size_t)col * I + kk;
  const int nsb = I / kScaleCols;
  const int steps = I / (32 * U);
  const int m = lane & 15;
  uint8_t* ssc = reinterpret_cast<uint8_t*>(sh + R * (I + 8));

  for (int p = 0; p < tl.rows; p += R) {
    const int nrows = min(R, tl.rows - p);
    const bool rv = m < nrows;
    const uint16_t* pa = sh + (rv ? m : 0) * (I + 8) + kk;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 b0[U], b1[U], a[U];
    auto load = [&](u32x4(&b)[U], int k) {
#pragma unroll
      for (int u = 0; u < U; ++u) b[u] = ldg16(pb + k + 32 * u);
    };
    load(b0, 0);
    if (tid == 0) sany = 0;
    stage_rows(sh, nrows, I, [&](int r) { return h + (size_t)(tl.row_start + p + r) * I; });
    __syncthreads();
    for (int i = tid; i < nsb; i += 256) {
      const uint8_t sv = hscale[(size_t)(tl.row_start + p) * nsb + i];
      ssc[i] = sv;
      if (sv) sany = 1;
    }
    __syncthreads();
    const bool scaled = sany != 0;
    auto math = [&](u32x4(&b)[U], int k) {
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = rv ? *reinterpret_cast<const u32x4*>(pa + k + 32 * u) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const u32x4 bh = scaled ? bf16x8_to_f16x8_scaled(b[u], ssc[(k + 32 * u) / kScaleCols]) : bf16x8_to_f16x8(b[u]);
        acc = mfma16x16x32_f16(a[u], bh, acc);
      }
    };
    for (int s = 0; s < steps; s += 2) {
      if (s + 1 < steps) load(b1, (s + 1) * 32 * U);
      math(b0, s * 32 * U);
      if (s + 2 < steps) load(b0, (s + 2) * 32 * U);
      if (s + 1 < steps) math(b1, (s + 1) * 32 * U);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (lane >> 4) * 4 + r;
      if (row < nrows) y[(size_t)sorted_slots[tl.row_start + p + row] * H + col] = acc[r];
    }
    __syncthreads();  // every wave is done with sh and ssc before the next pass restages them
  }
}

// Stream kernel shape: eight 32-wide K steps per register stage.
constexpr int kStreamU = 8;

// LDS of one gfx950 compute unit, the most one workgroup can take.
constexpr size_t kLdsBytesPerCU = 160 * 1024;

size_t gateup_stream_lds_bytes(int H) { return (size_t)kLdsRows * (H + 8) * 2; }
size_t down_stream_lds_bytes(int I) { return (size_t)kLdsRows * (I + 8) * 2 + I / kScaleCols; }

// Whether the LDS-staged stream kernels can run at this shape (their staged rows fit in LDS).
bool stream_lds_fits(int H, int I) {
  return gateup_stream_lds_bytes(H) <= kLdsBytesPerCU && down_stream_lds_bytes(I) <= kLdsBytesPerCU;
}

// Launchers of the stream path.  `lds` picks the variant with activation rows staged in
// LDS (passes of 8 rows; requires stream_lds_fits); gate/up and down must use the same
// variant, since the down kernel reads one activation scale per pass of gate/up.
hipError_t launch_gateup_stream(bool lds, const uint16_t* x, const int32_t* slots, const Tile* tiles,
                                const int32_t* ntiles, int max_tiles, const uint16_t* wg, const uint16_t* wu,
                                uint16_t* h, uint8_t* hscale, int H, int I, int K, hipStream_t st) {
  // H % 256 == 0: the K loop (H / 256 steps of eight) divides; I % 64 == 0: the column grid divides
  dim3 grid(max_tiles, I / 64);
  if (lds) {
    const size_t bytes = gateup_stream_lds_bytes(H);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gateup_stream_lds_kernel<kStreamU, kLdsRows>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gateup_stream_lds_kernel<kStreamU, kLdsRows>), grid, dim3(256), bytes, st, x, slots, tiles,
                       ntiles, wg, wu, h, hscale, H, I, K);
  } else {
    hipLaunchKernelGGL(gateup_stream_kernel<kStreamU>, grid, dim3(256), 0, st, x, slots, tiles, ntiles, wg, wu, h,
                       hscale, H, I, K);
  }
  return hipGetLastError();
}

hipError_t launch_down_stream(bool lds, const uint16_t* h, const uint8_t* hscale, const int32_t* slots,
                              const Tile* tiles, const int32_t* ntiles, int max_tiles, const uint16_t* wd, float* y,
                              int H, int I, hipStream_t st) {
  dim3 grid(max_tiles, H / 64);
  // I % 128 == 0: I / 32 is a multiple of 4; eight-step stages need I % 256 == 0, else four
  const bool u8 = (I / 32) % 8 == 0;
  if (lds) {
    const size_t bytes = down_stream_lds_bytes(I);
    const void* fn = u8 ? reinterpret_cast<const void*>(&down_stream_lds_kernel<8, kLdsRows>)
                        : reinterpret_cast<const void*>(&down_stream_lds_kernel<4, kLdsRows>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    if (u8)
      hipLaunchKernelGGL((down_stream_lds_kernel<8, kLdsRows>), grid, dim3(256), bytes, st, h, hscale, slots, tiles,
                         ntiles, wd, y, H, I);
    else
      hipLaunchKernelGGL((down_stream_lds_kernel<4, kLdsRows>), grid, dim3(256), bytes, st, h, hscale, slots, tiles,
                         ntiles, wd, y, H, I);
  } else if (u8) {
    hipLaunchKernelGGL(down_stream_kernel<8>, grid, dim3(256), 0, st, h, hscale, slots, tiles, ntiles, wd, y, H, I);
  } else {
    hipLaunchKernelGGL(down_stream_kernel<4>, grid, dim3(256), 0, st, h, hscale, slots, tiles, ntiles, wd, y, H, I);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// combine: out[t] = sum_k w[t,k] * y[t*K + k], k ascending, FP32
// ---------------------------------------------------------------------------
constexpr int kCombineCols = 1024;  // columns per workgroup (256 threads x 4)

// grid: (T, ceil(H / 1024)); block 256.  The K rows of a token are loaded
// together (up to 16), then summed in ascending k.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      float* __restrict__ out, int H, int K) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * kCombineCols + threadIdx.x * 4;
  if (c >= H) return;
  const float* yt = y + (size_t)t * K * H + c;
  const float* wt = w + (size_t)t * K;
  f32x4 v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < K) v[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yt + (size_t)k * H));
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < K) acc += wt[k] * v[k];
  *reinterpret_cast<f32x4*>(out + (size_t)t * H + c) = acc;
}

hipError_t launch_combine(const float* y, const float* w, float* out, int T, int H, int K, hipStream_t st) {
  hipLaunchKernelGGL(combine_kernel, dim3(T, (H + kCombineCols - 1) / kCombineCols), dim3(256), 0, st, y, w, out, H,
                     K);
  return hipGetLastError();
}

}  // namespace beam
