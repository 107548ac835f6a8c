// Grouped SwiGLU expert GEMMs of the Beam MoE block (gfx950, bf16 MFMA,
// FP32 accumulation).
//
// Beam launch blog, "mixture of experts" section: each expert is a SwiGLU
// MLP with intermediate size 2560 (hidden 5120); the "residual stream"
// section puts the SwiGLU product in FP32.  Per expert e and routed row r:
//   h[r] = silu(W_gate[e] x[r]) * (W_up[e] x[r])      FP32, stored as bf16 (RNE)
//   y[r] = W_down[e] h[r]                              FP32
// Rows are processed in expert-sorted order (the dispatch permutation); a
// tile table produced by the dispatch maps workgroups to (expert, rows).
//
// Two kernel families:
//   *_stream_kernel  few rows per expert (decode): weights are streamed once
//       from HBM straight into MFMA operand registers with non-temporal
//       16-byte loads; the K dimension is split over the 4 waves and reduced
//       in LDS in a fixed order; rows are taken 16 at a time.
//   *_tiled_kernel   many rows per expert (prefill): LDS double-buffered
//       BM x BN x 64 tiles, 8 waves, 16x16x32 MFMAs; gate and up share the A
//       tile and the SwiGLU product is formed in registers.
#include "common.h"

namespace beam {

// ---------------------------------------------------------------------------
// stream kernels (small row counts)
// ---------------------------------------------------------------------------
constexpr int kStreamN = 64;  // output columns per workgroup (per gate and per up)
constexpr int kStreamRows = 16;

// grid: (max_tiles, I / 64); block 256.  One tile = all rows of one expert.
__global__ __launch_bounds__(256) void gateup_stream_kernel(const uint16_t* __restrict__ x,
                                                            const int32_t* __restrict__ sorted_slots,
                                                            const Tile* __restrict__ tiles,
                                                            const int32_t* __restrict__ ntiles,
                                                            const uint16_t* __restrict__ wg,
                                                            const uint16_t* __restrict__ wu,
                                                            uint16_t* __restrict__ h, int H, int I, int K) {
  __shared__ __attribute__((aligned(16))) float red[4][8][64][4];
  if ((int)blockIdx.x >= ntiles[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.y * kStreamN;
  const int kq = H / 4;
  const int kbeg = wave * kq;
  const int kk = (lane >> 4) * 8;
  const size_t ebase = (size_t)tl.expert * I * H;
  const uint16_t* pg = wg + ebase + (size_t)(n0 + (lane & 15)) * H + kk;
  const uint16_t* pu = wu + ebase + (size_t)(n0 + (lane & 15)) * H + kk;

  for (int p = 0; p < tl.rows; p += kStreamRows) {
    const int m = lane & 15;
    const bool rv = p + m < tl.rows;
    const int tok = rv ? sorted_slots[tl.row_start + p + m] / K : 0;
    const uint16_t* pa = x + (size_t)tok * H + kk;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int k = kbeg; k < kbeg + kq; k += 32) {
      u32x4 bgv[4], buv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bgv[j] = ldg16_stream(pg + (size_t)j * 16 * H + k);
        buv[j] = ldg16_stream(pu + (size_t)j * 16 * H + k);
      }
      u32x4 a = rv ? ldg16(pa + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = mfma16x16x32(a, bgv[j], acc[j]);
        acc[4 + j] = mfma16x16x32(a, buv[j], acc[4 + j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4*>(&red[wave][j][lane][0]) = acc[j];
    __syncthreads();
    // 16 rows x 64 columns of h; four per thread
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int o = tid + 256 * q;
      const int j = o >> 8;
      const int ln = (o >> 2) & 63;
      const int r = o & 3;
      float g = red[0][j][ln][r], u = red[0][4 + j][ln][r];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        g += red[w][j][ln][r];
        u += red[w][4 + j][ln][r];
      }
      const int row = (ln >> 4) * 4 + r;
      const int col = j * 16 + (ln & 15);
      if (p + row < tl.rows)
        h[(size_t)(tl.row_start + p + row) * I + n0 + col] = f32_to_bf16_rne(silu_f32(g) * u);
    }
    __syncthreads();
  }
}

// grid: (max_tiles, H / 64); block 256.
__global__ __launch_bounds__(256) void down_stream_kernel(const uint16_t* __restrict__ h,
                                                          const int32_t* __restrict__ sorted_slots,
                                                          const Tile* __restrict__ tiles,
                                                          const int32_t* __restrict__ ntiles,
                                                          const uint16_t* __restrict__ wd, float* __restrict__ y,
                                                          int H, int I) {
  __shared__ __attribute__((aligned(16))) float red[4][4][64][4];
  if ((int)blockIdx.x >= ntiles[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.y * kStreamN;
  const int kq = I / 4;
  const int kbeg = wave * kq;
  const int kk = (lane >> 4) * 8;
  const uint16_t* pb = wd + (size_t)tl.expert * H * I + (size_t)(n0 + (lane & 15)) * I + kk;

  for (int p = 0; p < tl.rows; p += kStreamRows) {
    const int m = lane & 15;
    const bool rv = p + m < tl.rows;
    const uint16_t* pa = h + (size_t)(tl.row_start + p + (rv ? m : 0)) * I + kk;
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k = kbeg; k < kbeg + kq; k += 32) {
      u32x4 bv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = ldg16_stream(pb + (size_t)j * 16 * I + k);
      u32x4 a = rv ? ldg16(pa + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma16x16x32(a, bv[j], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4*>(&red[wave][j][lane][0]) = acc[j];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int o = tid + 256 * q;
      const int j = o >> 8;
      const int ln = (o >> 2) & 63;
      const int r = o & 3;
      float s = red[0][j][ln][r];
#pragma unroll
      for (int w = 1; w < 4; ++w) s += red[w][j][ln][r];
      const int row = (ln >> 4) * 4 + r;
      const int col = j * 16 + (ln & 15);
      if (p + row < tl.rows) {
        const int slot = sorted_slots[tl.row_start + p + row];
        y[(size_t)slot * H + n0 + col] = s;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// tiled kernels (many rows per expert)
// ---------------------------------------------------------------------------
constexpr int kBK = 64;
constexpr int kLd = kBK + 8;  // LDS row stride in bf16 (144 bytes: conflict-free 16-byte fragment reads)

// Block tile: BM rows x NB B-rows, where the B tile is [gate BN ; up BN] for
// the gate/up kernel (NB = 2 BN) and [down BN] for the down kernel (NB = BN).
// 8 waves as WM x WN; each wave owns (BM/WM) rows and (NB/WN) B-rows, split
// so that a wave's gate and up columns coincide.
template <bool GATEUP, int BM, int BN, int WM, int WN>
struct TiledCfg {
  static constexpr int NB = GATEUP ? 2 * BN : BN;
  static constexpr int WROWS = BM / WM;  // rows per wave
  static constexpr int WCOLS = BN / WN;  // output columns per wave
  static constexpr int RB = WROWS / 16;  // 16-row blocks per wave
  static constexpr int CB = WCOLS / 16;  // 16-col blocks per wave (per gate / up)
  static constexpr int NACC = GATEUP ? 2 * CB : CB;
  static constexpr int THREADS = 64 * WM * WN;
  static constexpr int A_CHUNKS = BM * kBK / 8 / THREADS;  // 16-byte chunks per thread
  static constexpr int B_CHUNKS = NB * kBK / 8 / THREADS;
  static_assert(WM * WN == 8, "8 waves");
  static_assert(A_CHUNKS * THREADS * 8 == BM * kBK, "A staging");
  static_assert(B_CHUNKS * THREADS * 8 == NB * kBK, "B staging");
};

// XCD-aware block order: hardware places block b on XCD b % 8; give each XCD a
// contiguous range of (tile, column-block) pairs so an expert's tiles share
// one L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int full = total & ~7;
  if (b >= full) return b;
  return (b & 7) * (full >> 3) + (b >> 3);
}

// GATEUP: A rows = x[slot / K] (gathered), B = [W_gate[e] rows n0.. ; W_up[e] rows n0..],
//         out = h[row][n] bf16.  Columns per block: BN of I.
// !GATEUP: A rows = h[row] (contiguous), B = W_down[e] rows n0.., out = y[slot][n] fp32.
template <bool GATEUP, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(512) void expert_tiled_kernel(const uint16_t* __restrict__ act,
                                                           const int32_t* __restrict__ sorted_slots,
                                                           const Tile* __restrict__ tiles,
                                                           const int32_t* __restrict__ ntiles,
                                                           const uint16_t* __restrict__ w0,
                                                           const uint16_t* __restrict__ w1,
                                                           void* __restrict__ out, int Kdim, int Ndim, int topk,
                                                           int nblocks_n, int total_blocks) {
  using C = TiledCfg<GATEUP, BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kLd];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][C::NB * kLd];

  const int lin = xcd_remap(blockIdx.x, total_blocks);
  const int tile_id = lin / nblocks_n;
  const int nblk = lin - tile_id * nblocks_n;
  if (tile_id >= ntiles[0]) return;
  const Tile tl = tiles[tile_id];
  const int n0 = nblk * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  // per-thread staging sources: chunk c = tid + THREADS*i -> row c/8, k-chunk c%8
  const uint16_t* asrc[C::A_CHUNKS];
  int aoff[C::A_CHUNKS];
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) {
    const int c = tid + C::THREADS * i;
    const int r = c >> 3, kc = c & 7;
    const int rr = min(r, tl.rows - 1);  // rows past the tile's end repeat its last row; never stored
    if (GATEUP) {
      const int tok = sorted_slots[tl.row_start + rr] / topk;
      asrc[i] = act + (size_t)tok * Kdim + kc * 8;
    } else {
      asrc[i] = act + (size_t)(tl.row_start + rr) * Kdim + kc * 8;
    }
    aoff[i] = r * kLd + kc * 8;
  }
  const uint16_t* bsrc[C::B_CHUNKS];
  int boff[C::B_CHUNKS];
  const size_t wexp = (size_t)tl.expert * Ndim * Kdim;
#pragma unroll
  for (int i = 0; i < C::B_CHUNKS; ++i) {
    const int c = tid + C::THREADS * i;
    const int r = c >> 3, kc = c & 7;
    if (GATEUP) {
      const uint16_t* base = r < BN ? w0 : w1;
      const int n = n0 + (r < BN ? r : r - BN);
      bsrc[i] = base + wexp + (size_t)n * Kdim + kc * 8;
    } else {
      bsrc[i] = w0 + wexp + (size_t)(n0 + r) * Kdim + kc * 8;
    }
    boff[i] = r * kLd + kc * 8;
  }

  f32x4 acc[C::RB][C::NACC];
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
#pragma unroll
    for (int j = 0; j < C::NACC; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[C::A_CHUNKS], rb[C::B_CHUNKS];
  const int nk = Kdim / kBK;
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) ra[i] = ldg16(asrc[i]);
#pragma unroll
  for (int i = 0; i < C::B_CHUNKS; ++i) rb[i] = ldg16(bsrc[i]);
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) *reinterpret_cast<u32x4*>(&sA[0][aoff[i]]) = ra[i];
#pragma unroll
  for (int i = 0; i < C::B_CHUNKS; ++i) *reinterpret_cast<u32x4*>(&sB[0][boff[i]]) = rb[i];
  __syncthreads();

  const int kk = (lane >> 4) * 8;
  const int arow0 = wm * C::WROWS + (lane & 15);
  const int brow0 = wn * C::WCOLS + (lane & 15);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int koff = (kt + 1) * kBK;
#pragma unroll
      for (int i = 0; i < C::A_CHUNKS; ++i) ra[i] = ldg16(asrc[i] + koff);
#pragma unroll
      for (int i = 0; i < C::B_CHUNKS; ++i) rb[i] = ldg16(bsrc[i] + koff);
    }
    const uint16_t* A = sA[cur];
    const uint16_t* B = sB[cur];
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 32) {
      u32x4 af[C::RB], bf[C::NACC];
#pragma unroll
      for (int i = 0; i < C::RB; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(&A[(arow0 + 16 * i) * kLd + ks + kk]);
#pragma unroll
      for (int j = 0; j < C::CB; ++j) {
        bf[j] = *reinterpret_cast<const u32x4*>(&B[(brow0 + 16 * j) * kLd + ks + kk]);
        if (GATEUP) bf[C::CB + j] = *reinterpret_cast<const u32x4*>(&B[(BN + brow0 + 16 * j) * kLd + ks + kk]);
      }
#pragma unroll
      for (int i = 0; i < C::RB; ++i)
#pragma unroll
        for (int j = 0; j < C::NACC; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < C::A_CHUNKS; ++i) *reinterpret_cast<u32x4*>(&sA[cur ^ 1][aoff[i]]) = ra[i];
#pragma unroll
      for (int i = 0; i < C::B_CHUNKS; ++i) *reinterpret_cast<u32x4*>(&sB[cur ^ 1][boff[i]]) = rb[i];
    }
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane/16)+r and column lane%16 of each 16x16 block
#pragma unroll
  for (int i = 0; i < C::RB; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * C::WROWS + 16 * i + (lane >> 4) * 4 + r;
      if (row >= tl.rows) continue;
      if (GATEUP) {
        uint16_t* hrow = reinterpret_cast<uint16_t*>(out) + (size_t)(tl.row_start + row) * Ndim + n0 +
                         wn * C::WCOLS + (lane & 15);
#pragma unroll
        for (int j = 0; j < C::CB; ++j) hrow[16 * j] = f32_to_bf16_rne(silu_f32(acc[i][j][r]) * acc[i][C::CB + j][r]);
      } else {
        const int slot = sorted_slots[tl.row_start + row];
        float* yrow = reinterpret_cast<float*>(out) + (size_t)slot * Ndim + n0 + wn * C::WCOLS + (lane & 15);
#pragma unroll
        for (int j = 0; j < C::CB; ++j) yrow[16 * j] = acc[i][j][r];
      }
    }
  }
}

// Tile shapes of the tiled path.
constexpr int kGuBM = 256, kGuBN = 128;  // gate/up: 256 rows x (128 gate + 128 up) columns
constexpr int kDnBM = 256, kDnBN = 256;  // down: 256 rows x 256 columns

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
int tiled_gateup_rows() { return kGuBM; }
int tiled_down_rows() { return kDnBM; }
int tiled_gateup_cols() { return kGuBN; }
int tiled_down_cols() { return kDnBN; }

hipError_t launch_gateup_stream(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                                int max_tiles, const uint16_t* wg, const uint16_t* wu, uint16_t* h, int H, int I,
                                int K, hipStream_t st) {
  dim3 grid(max_tiles, I / kStreamN);
  hipLaunchKernelGGL(gateup_stream_kernel, grid, dim3(256), 0, st, x, slots, tiles, ntiles, wg, wu, h, H, I, K);
  return hipGetLastError();
}

hipError_t launch_down_stream(const uint16_t* h, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                              int max_tiles, const uint16_t* wd, float* y, int H, int I, hipStream_t st) {
  dim3 grid(max_tiles, H / kStreamN);
  hipLaunchKernelGGL(down_stream_kernel, grid, dim3(256), 0, st, h, slots, tiles, ntiles, wd, y, H, I);
  return hipGetLastError();
}

hipError_t launch_gateup_tiled(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                               int max_tiles, const uint16_t* wg, const uint16_t* wu, uint16_t* h, int H, int I,
                               int K, hipStream_t st) {
  const int nbn = I / kGuBN;
  const int total = max_tiles * nbn;
  hipLaunchKernelGGL((expert_tiled_kernel<true, kGuBM, kGuBN, 4, 2>), dim3(total), dim3(512), 0, st, x, slots,
                     tiles, ntiles, wg, wu, (void*)h, H, I, K, nbn, total);
  return hipGetLastError();
}

hipError_t launch_down_tiled(const uint16_t* h, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                             int max_tiles, const uint16_t* wd, float* y, int H, int I, hipStream_t st) {
  const int nbn = H / kDnBN;
  const int total = max_tiles * nbn;
  hipLaunchKernelGGL((expert_tiled_kernel<false, kDnBM, kDnBN, 4, 2>), dim3(total), dim3(512), 0, st, h, slots,
                     tiles, ntiles, wd, nullptr, (void*)y, I, H, 0, nbn, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// combine: out[t] = sum_k w[t,k] * y[t*K + k], k ascending, FP32
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      float* __restrict__ out, int H, int K) {
  const int t = blockIdx.x;
  const float* yt = y + (size_t)t * K * H;
  const float* wt = w + (size_t)t * K;
  for (int c = threadIdx.x * 4; c < H; c += 256 * 4) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
      const float wk = wt[k];
      const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yt + (size_t)k * H + c));
      acc += wk * v;
    }
    *reinterpret_cast<f32x4*>(out + (size_t)t * H + c) = acc;
  }
}

hipError_t launch_combine(const float* y, const float* w, float* out, int T, int H, int K, hipStream_t st) {
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(256), 0, st, y, w, out, H, K);
  return hipGetLastError();
}

}  // namespace beam
