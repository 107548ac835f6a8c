// Grouped SwiGLU expert GEMMs of the Beam MoE block (gfx950 MFMA, FP32
// accumulation).
//
// Beam launch blog, "mixture of experts" section: each expert is a SwiGLU
// MLP with intermediate size 2560 (hidden 5120); the "residual stream"
// section puts the SwiGLU product in FP32.  Per expert e and routed row r:
//   h[r] = silu(W_gate[e] x[r]) * (W_up[e] x[r])   bf16 MFMA, SwiGLU in FP32
//   y[r] = W_down[e] h[r]                           fp16 MFMA, FP32 out
// h is handed to the down projection as fp16 (11 significant bits against
// bf16's 8) with a power-of-two scale 2^-s per block of 64 columns of a row
// group, s chosen so the block's largest magnitude stays below 2^15; W_down
// is converted from bf16 to fp16 exactly (times 2^s) as it is loaded.
// Rows are processed in expert-sorted order (the dispatch permutation); a
// tile table produced by the dispatch maps workgroups to (expert, rows).
//
// Two kernel families:
//   *_stream_kernel  few rows per expert (decode): weights are streamed once
//       from HBM straight into MFMA operand registers; rows are taken 16 at a
//       time and the scale group is (16-row pass, 64 columns).
//   *_tiled_kernel   many rows per expert (prefill): LDS double-buffered
//       BM x BN x 64 tiles, 8 waves, 16x16x32 MFMAs; gate and up share the A
//       tile and the SwiGLU product is formed in registers; the scale group
//       is (row tile, BN columns).
#include "common.h"

namespace beam {

constexpr int kMaxScaleBlocks = 512;  // I <= 32768

// ---------------------------------------------------------------------------
// stream kernels (small row counts)
// ---------------------------------------------------------------------------
// A workgroup owns one expert (all its rows, taken 16 at a time) and
// 4 * 16 * CB output columns; wave w owns 16 * CB columns (CB blocks of 16) over
// the whole K range, so no cross-wave reduction is needed and one activation
// operand load feeds CB (down) or 2 * CB (gate and up) weight operand loads.
// Loads run U MFMA steps ahead of the math (two register stages) and use
// ordinary cached loads: a 16-byte operand load touches half of a 128-byte line,
// and the other half is read by the next step.
constexpr int kStreamRows = 16;  // rows per pass

// grid: (max_tiles, I / (64 * CB)); block 256.  One tile = all rows of one expert.
// Writes h (fp16 bits, scaled by 2^-s) and s per (row, 64-column block).
template <int U, int CB>
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
  const int col0 = (blockIdx.y * 4 + wave) * 16 * CB + (lane & 15);  // + 16 j for block j
  const int kk = (lane >> 4) * 8;
  const size_t ebase = (size_t)tl.expert * I * H;
  const uint16_t* pg = wg + ebase + (size_t)col0 * H + kk;
  const uint16_t* pu = wu + ebase + (size_t)col0 * H + kk;
  const int nsb = I / kScaleCols;
  const int steps = H / (32 * U);

  for (int p = 0; p < tl.rows; p += kStreamRows) {
    const int m = lane & 15;
    const bool rv = p + m < tl.rows;
    const int tok = rv ? sorted_slots[tl.row_start + p + m] / K : 0;
    const uint16_t* pa = x + (size_t)tok * H + kk;
    f32x4 ag[CB], au[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) ag[j] = au[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 g0[U][CB], u0[U][CB], a0[U], g1[U][CB], u1[U][CB], a1[U];
    auto load = [&](u32x4(&g)[U][CB], u32x4(&uu)[U][CB], u32x4(&a)[U], int k) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          g[u][j] = ldg16(pg + (size_t)16 * j * H + k + 32 * u);
          uu[u][j] = ldg16(pu + (size_t)16 * j * H + k + 32 * u);
        }
        a[u] = rv ? ldg16(pa + k + 32 * u) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto math = [&](u32x4(&g)[U][CB], u32x4(&uu)[U][CB], u32x4(&a)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          ag[j] = mfma16x16x32(a[u], g[u][j], ag[j]);
          au[j] = mfma16x16x32(a[u], uu[u][j], au[j]);
        }
    };
    load(g0, u0, a0, 0);
    for (int s = 0; s < steps; s += 2) {
      if (s + 1 < steps) load(g1, u1, a1, (s + 1) * 32 * U);
      math(g0, u0, a0);
      if (s + 2 < steps) load(g0, u0, a0, (s + 2) * 32 * U);
      if (s + 1 < steps) math(g1, u1, a1);
    }
    // SwiGLU in FP32; one power-of-two scale per (16-row pass, workgroup columns)
    float v[CB][4];
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = (lane >> 4) * 4 + r;
        v[j][r] = (p + row < tl.rows) ? silu_f32(ag[j][r]) * au[j][r] : 0.f;
        mx = fmaxf(mx, fabsf(v[j][r]));
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
#pragma unroll
        for (int j = 0; j < CB; ++j) h[grow * I + col0 + 16 * j] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(v[j][r], -sexp));
        if (wave == 0 && (lane & 15) < CB) hscale[grow * nsb + blockIdx.y * CB + (lane & 15)] = (uint8_t)sexp;
      }
    }
    __syncthreads();
  }
}

// grid: (max_tiles, H / (64 * CB)); block 256.  y[slot] = W_down[e] h (fp16 MFMA,
// W_down converted exactly from bf16 and scaled back by 2^s per 64-column
// block of h).
template <int U, int CB>
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
  const int col0 = (blockIdx.y * 4 + wave) * 16 * CB + (lane & 15);
  const int kk = (lane >> 4) * 8;
  const uint16_t* pb = wd + (size_t)tl.expert * H * I + (size_t)col0 * I + kk;
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
    f32x4 acc[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 b0[U][CB], a0[U], b1[U][CB], a1[U];
    auto load = [&](u32x4(&b)[U][CB], u32x4(&a)[U], int k) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int j = 0; j < CB; ++j) b[u][j] = ldg16(pb + (size_t)16 * j * I + k + 32 * u);
        a[u] = rv ? ldg16(pa + k + 32 * u) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto math = [&](u32x4(&b)[U][CB], u32x4(&a)[U], int k) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          const u32x4 bh = scaled ? bf16x8_to_f16x8_scaled(b[u][j], ssc[(k + 32 * u) / kScaleCols])
                                  : bf16x8_to_f16x8(b[u][j]);
          acc[j] = mfma16x16x32_f16(a[u], bh, acc[j]);
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
      if (p + row < tl.rows) {
        const size_t slot = (size_t)sorted_slots[tl.row_start + p + row];
#pragma unroll
        for (int j = 0; j < CB; ++j) y[slot * H + col0 + 16 * j] = acc[j][r];
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// tiled kernels (many rows per expert)
// ---------------------------------------------------------------------------
constexpr int kTBK = 64;
constexpr int kTLd = kTBK + 8;  // LDS row stride in bf16 (144 bytes: conflict-free 16-byte fragment reads)

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
  static constexpr int A_CHUNKS = BM * kTBK / 8 / THREADS;  // 16-byte chunks per thread
  static constexpr int B_CHUNKS = NB * kTBK / 8 / THREADS;
  static_assert(WM * WN == 8, "8 waves");
  static_assert(A_CHUNKS * THREADS * 8 == BM * kTBK, "A staging");
  static_assert(B_CHUNKS * THREADS * 8 == NB * kTBK, "B staging");
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
//         bf16 MFMA; out = h[row][n] fp16 bits scaled by 2^-s, s per (tile, 64-column block)
//         written to hscale.  Columns per block: BN of I.
// !GATEUP: A rows = h[row] (contiguous, fp16), B = W_down[e] rows n0.. converted to fp16 while
//         staged and scaled by 2^s of the k-step's 64-column block; fp16 MFMA; out = y[slot][n] fp32.
template <bool GATEUP, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(512) void expert_tiled_kernel(const uint16_t* __restrict__ act,
                                                           const int32_t* __restrict__ sorted_slots,
                                                           const Tile* __restrict__ tiles,
                                                           const int32_t* __restrict__ ntiles,
                                                           const uint16_t* __restrict__ w0,
                                                           const uint16_t* __restrict__ w1,
                                                           void* __restrict__ out, uint8_t* __restrict__ hscale,
                                                           int Kdim, int Ndim, int topk, int nblocks_n,
                                                           int total_blocks) {
  using C = TiledCfg<GATEUP, BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kTLd];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][C::NB * kTLd];
  __shared__ float smax[8];

  // The grid is sized for the most tiles a batch can have; the remap spans the
  // blocks of the tiles this batch has, so every XCD gets an equal share.
  const int real_blocks = min(total_blocks, ntiles[0] * nblocks_n);
  if ((int)blockIdx.x >= real_blocks) return;
  const int lin = xcd_remap(blockIdx.x, real_blocks);
  const int tile_id = lin / nblocks_n;
  const int nblk = lin - tile_id * nblocks_n;
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
    aoff[i] = r * kTLd + kc * 8;
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
    boff[i] = r * kTLd + kc * 8;
  }

  f32x4 acc[C::RB][C::NACC];
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
#pragma unroll
    for (int j = 0; j < C::NACC; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[C::A_CHUNKS], rb[C::B_CHUNKS];
  const int nk = Kdim / kTBK;
  // down projection: scale exponents of this tile's activation blocks (one per 64-wide k-step)
  const uint8_t* tscale = GATEUP ? nullptr : hscale + (size_t)tl.row_start * (Kdim / kScaleCols);
  int snext = GATEUP ? 0 : tscale[0];
  auto stage_b = [&](int buf, int sexp) {
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i) {
      u32x4 v = rb[i];
      if (!GATEUP) v = sexp ? bf16x8_to_f16x8_scaled(v, sexp) : bf16x8_to_f16x8(v);
      *reinterpret_cast<u32x4*>(&sB[buf][boff[i]]) = v;
    }
  };
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) ra[i] = ldg16(asrc[i]);
#pragma unroll
  for (int i = 0; i < C::B_CHUNKS; ++i) rb[i] = ldg16(bsrc[i]);
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) *reinterpret_cast<u32x4*>(&sA[0][aoff[i]]) = ra[i];
  stage_b(0, snext);
  __syncthreads();

  const int kk = (lane >> 4) * 8;
  const int arow0 = wm * C::WROWS + (lane & 15);
  const int brow0 = wn * C::WCOLS + (lane & 15);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int koff = (kt + 1) * kTBK;
#pragma unroll
      for (int i = 0; i < C::A_CHUNKS; ++i) ra[i] = ldg16(asrc[i] + koff);
#pragma unroll
      for (int i = 0; i < C::B_CHUNKS; ++i) rb[i] = ldg16(bsrc[i] + koff);
      if (!GATEUP) snext = tscale[kt + 1];
    }
    const uint16_t* A = sA[cur];
    const uint16_t* B = sB[cur];
#pragma unroll
    for (int ks = 0; ks < kTBK; ks += 32) {
      u32x4 af[C::RB], bf[C::NACC];
#pragma unroll
      for (int i = 0; i < C::RB; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(&A[(arow0 + 16 * i) * kTLd + ks + kk]);
#pragma unroll
      for (int j = 0; j < C::CB; ++j) {
        bf[j] = *reinterpret_cast<const u32x4*>(&B[(brow0 + 16 * j) * kTLd + ks + kk]);
        if (GATEUP) bf[C::CB + j] = *reinterpret_cast<const u32x4*>(&B[(BN + brow0 + 16 * j) * kTLd + ks + kk]);
      }
#pragma unroll
      for (int i = 0; i < C::RB; ++i)
#pragma unroll
        for (int j = 0; j < C::NACC; ++j)
          acc[i][j] = GATEUP ? mfma16x16x32(af[i], bf[j], acc[i][j]) : mfma16x16x32_f16(af[i], bf[j], acc[i][j]);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < C::A_CHUNKS; ++i) *reinterpret_cast<u32x4*>(&sA[cur ^ 1][aoff[i]]) = ra[i];
      stage_b(cur ^ 1, snext);
    }
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane/16)+r and column lane%16 of each 16x16 block
  if (GATEUP) {
    // SwiGLU in FP32, then one power-of-two scale for the whole tile x BN block
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < C::RB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = wm * C::WROWS + 16 * i + (lane >> 4) * 4 + r < tl.rows;
#pragma unroll
        for (int j = 0; j < C::CB; ++j) {
          const float v = ok ? silu_f32(acc[i][j][r]) * acc[i][C::CB + j][r] : 0.f;
          acc[i][j][r] = v;
          mx = fmaxf(mx, fabsf(v));
        }
      }
    mx = wave_max(mx);
    if (lane == 0) smax[wave] = mx;
    __syncthreads();
    float bm = smax[0];
#pragma unroll
    for (int w = 1; w < 8; ++w) bm = fmaxf(bm, smax[w]);
    const int sexp = act_scale_exp(bm);
    const int nsb = Ndim / kScaleCols;
    for (int r = tid; r < tl.rows; r += C::THREADS)
#pragma unroll
      for (int b = 0; b < BN / kScaleCols; ++b)
        hscale[(size_t)(tl.row_start + r) * nsb + n0 / kScaleCols + b] = (uint8_t)sexp;
#pragma unroll
    for (int i = 0; i < C::RB; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * C::WROWS + 16 * i + (lane >> 4) * 4 + r;
        if (row >= tl.rows) continue;
        uint16_t* hrow = reinterpret_cast<uint16_t*>(out) + (size_t)(tl.row_start + row) * Ndim + n0 +
                         wn * C::WCOLS + (lane & 15);
#pragma unroll
        for (int j = 0; j < C::CB; ++j) hrow[16 * j] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(acc[i][j][r], -sexp));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::RB; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * C::WROWS + 16 * i + (lane >> 4) * 4 + r;
        if (row >= tl.rows) continue;
        const int slot = sorted_slots[tl.row_start + row];
        float* yrow = reinterpret_cast<float*>(out) + (size_t)slot * Ndim + n0 + wn * C::WCOLS + (lane & 15);
#pragma unroll
        for (int j = 0; j < C::CB; ++j) yrow[16 * j] = acc[i][j][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// tiled kernel, one wave per SIMD (many rows per expert)
// ---------------------------------------------------------------------------
// Block tile: 256 rows x 256 B-rows (gate/up: 128 gate + 128 up columns;
// down: 256 columns), 4 waves as 2 x 2, each wave 128 rows x 128 B-rows =
// 8 x 8 MFMA 16x16x32 tiles (256 accumulator registers).  K advances 32 per
// stage; stages live in a ring of kGemmStages LDS slots.  Global loads of
// stage t + kGemmStages - 1 are issued at step t into one of two register
// buffers and written to LDS one step later, so a load has two steps of math
// to arrive; the fragments of stage t + 1 are read from LDS while stage t's
// MFMAs run.  LDS rows are 64 bytes (no padding) with the four 16-byte chunks
// of row r permuted by f(r) = ((r >> 1) ^ (r >> 3)) & 3, which keeps the
// 16 rows read by one fragment load on distinct banks.
constexpr int kGemmBM = 256;
constexpr int kGemmBN = 256;      // B-rows per block
constexpr int kGemmStages = 4;
constexpr int kGemmStageHalfs = kGemmBM * 32;  // bf16 elements of one operand per stage

__device__ __forceinline__ int gemm_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// GATEUP: A = x rows gathered through the permutation, B = [W_gate rows n0..n0+127 ;
//         W_up rows n0..n0+127], bf16 MFMA, out h fp16 (scaled) + hscale.
// !GATEUP: A = h rows (fp16), B = W_down rows n0..n0+255 converted to fp16 (x 2^s of the
//         stage's 64-column activation block) as they are written to LDS, fp16 MFMA,
//         out y fp32 at row slot.
template <bool GATEUP>
__global__ __launch_bounds__(256, 1) void expert_gemm_kernel(const uint16_t* __restrict__ act,
                                                            const int32_t* __restrict__ sorted_slots,
                                                            const Tile* __restrict__ tiles,
                                                            const int32_t* __restrict__ ntiles,
                                                            const uint16_t* __restrict__ w0,
                                                            const uint16_t* __restrict__ w1,
                                                            void* __restrict__ out, uint8_t* __restrict__ hscale,
                                                            int Kdim, int Ndim, int topk, int nblocks_n,
                                                            int total_blocks) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[kGemmStages][kGemmStageHalfs];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kGemmStages][kGemmStageHalfs];
  __shared__ float smax[4];

  // The grid is sized for the most tiles a batch can have; the remap spans the
  // blocks of the tiles this batch has, so every XCD gets an equal share.
  const int real_blocks = min(total_blocks, ntiles[0] * nblocks_n);
  if ((int)blockIdx.x >= real_blocks) return;
  const int lin = xcd_remap(blockIdx.x, real_blocks);
  const int tile_id = lin / nblocks_n;
  const int nblk = lin - tile_id * nblocks_n;
  const Tile tl = tiles[tile_id];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int BNc = GATEUP ? kGemmBN / 2 : kGemmBN;  // output columns per block
  const int n0 = nblk * BNc;

  // staging: thread owns chunk (tid & 3) of rows (tid >> 2) + 64 i, i = 0..3, for A and for B.
  // Sources are 32-bit element offsets from per-block base pointers (each base spans < 2^31 elements).
  const int sc = tid & 3;
  uint32_t aoff[4], boff[4];
  int soff[4];
  const uint16_t* abase = act;
  const uint16_t* gbase = w0 + (size_t)tl.expert * Ndim * Kdim;
  const uint16_t* ubase = GATEUP ? w1 + (size_t)tl.expert * Ndim * Kdim : gbase;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 2) + 64 * i;
    const int rr = min(r, tl.rows - 1);  // rows past the tile's end repeat its last row; never stored
    if (GATEUP) {
      aoff[i] = (uint32_t)(sorted_slots[tl.row_start + rr] / topk) * Kdim + sc * 8;
      boff[i] = (uint32_t)(n0 + (r & 127)) * Kdim + sc * 8;  // rows 0..127 gate, 128..255 up (i >= 2)
    } else {
      aoff[i] = (uint32_t)(tl.row_start + rr) * Kdim + sc * 8;
      boff[i] = (uint32_t)(n0 + r) * Kdim + sc * 8;
    }
    soff[i] = r * 32 + ((sc ^ gemm_swz(r)) << 3);
  }
  const uint8_t* tscale = GATEUP ? nullptr : hscale + (size_t)tl.row_start * (Kdim / kScaleCols);

  u32x4 ra[2][4], rb[2][4];
  auto gload = [&](int buf, int stage) {
    const int k = stage * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[buf][i] = ldg16(abase + aoff[i] + k);
      rb[buf][i] = ldg16((GATEUP && i >= 2 ? ubase : gbase) + boff[i] + k);
    }
  };
  auto lstore = [&](int buf, int stage) {
    const int slot = stage % kGemmStages;
    int sexp = 0;
    if (!GATEUP) sexp = tscale[(stage * 32) / kScaleCols];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&sA[slot][soff[i]]) = ra[buf][i];
      u32x4 v = rb[buf][i];
      if (!GATEUP) v = sexp ? bf16x8_to_f16x8_scaled(v, sexp) : bf16x8_to_f16x8(v);
      *reinterpret_cast<u32x4*>(&sB[slot][soff[i]]) = v;
    }
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment addresses: row r = base + 16 i + (lane & 15); the chunk permutation of
  // rows base + 16 i depends only on the parity of i (bases are multiples of 64 rows).
  const int fc = lane >> 4;
  const int ar = wm * 128 + (lane & 15);
  const int br = (GATEUP ? wn * 64 : wn * 128) + (lane & 15);
  const int aoffe = ar * 32 + ((fc ^ gemm_swz(ar)) << 3), aoffo = (ar + 16) * 32 + ((fc ^ gemm_swz(ar + 16)) << 3);
  const int boffe = br * 32 + ((fc ^ gemm_swz(br)) << 3), boffo = (br + 16) * 32 + ((fc ^ gemm_swz(br + 16)) << 3);
  auto afrag = [&](int stage, int i) {
    return *reinterpret_cast<const u32x4*>(&sA[stage % kGemmStages][((i & 1) ? aoffo : aoffe) + (i >> 1) * 32 * 32]);
  };
  auto bfrag = [&](int stage, int j) {
    // gate/up: j < 4 gate rows, j >= 4 the matching up rows (128 B-rows further)
    const int jj = GATEUP ? (j & 3) : j;
    const int extra = GATEUP && j >= 4 ? 128 * 32 : 0;
    return *reinterpret_cast<const u32x4*>(&sB[stage % kGemmStages][((jj & 1) ? boffo : boffe) + (jj >> 1) * 32 * 32 +
                                                                   extra]);
  };
  // One register set of fragments: A[i] is reloaded for the next stage right
  // after its last use, B[j] during the last row block.
  u32x4 fa[8], fb[8];
  auto math = [&](int stage, bool next) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[i][j] = GATEUP ? mfma16x16x32(fa[i], fb[j], acc[i][j]) : mfma16x16x32_f16(fa[i], fb[j], acc[i][j]);
        if (i == 7 && next) fb[j] = bfrag(stage + 1, j);
      }
      if (next) fa[i] = afrag(stage + 1, i);
    }
  };

  const int nk = Kdim / 32;  // >= kGemmStages (Kdim >= 128)
  // prologue: stages 0 .. S-2 into LDS, stage S-1 in flight in register buffer 0
#pragma unroll
  for (int s = 0; s < kGemmStages - 1; ++s) {
    gload(0, s);
    lstore(0, s);
  }
  gload(0, kGemmStages - 1);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) fa[i] = afrag(0, i);
#pragma unroll
  for (int j = 0; j < 8; ++j) fb[j] = bfrag(0, j);
  // step t: MFMAs on stage t while stage t+1's fragments are read; global loads of
  // stage t+S go to register buffer (t+1)&1; register buffer t&1 (stage t+S-1,
  // issued one step earlier) is written to LDS.
  for (int t = 0; t < nk; t += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int st = t + u;
      if (st < nk) {
        if (st + kGemmStages < nk) gload(u ^ 1, st + kGemmStages);
        math(st, st + 1 < nk);
        if (st + kGemmStages - 1 < nk) lstore(u, st + kGemmStages - 1);
        __syncthreads();
      }
    }
  }

  // epilogue: lane holds rows 4*(lane/16)+r and column lane%16 of each 16x16 block
  if (GATEUP) {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = wm * 128 + 16 * i + (lane >> 4) * 4 + r < tl.rows;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = ok ? silu_f32(acc[i][j][r]) * acc[i][4 + j][r] : 0.f;
          acc[i][j][r] = v;
          mx = fmaxf(mx, fabsf(v));
        }
      }
    mx = wave_max(mx);
    if (lane == 0) smax[wave] = mx;
    __syncthreads();
    const int sexp = act_scale_exp(fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3])));
    const int nsb = Ndim / kScaleCols;
    for (int r = tid; r < tl.rows; r += 256)
#pragma unroll
      for (int b = 0; b < 128 / kScaleCols; ++b)
        hscale[(size_t)(tl.row_start + r) * nsb + n0 / kScaleCols + b] = (uint8_t)sexp;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 128 + 16 * i + (lane >> 4) * 4 + r;
        if (row < tl.rows) {
          uint16_t* hrow = reinterpret_cast<uint16_t*>(out) + (size_t)(tl.row_start + row) * Ndim + n0 + wn * 64 +
                           (lane & 15);
#pragma unroll
          for (int j = 0; j < 4; ++j) hrow[16 * j] = f32_to_f16_bits(__builtin_amdgcn_ldexpf(acc[i][j][r], -sexp));
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 128 + 16 * i + (lane >> 4) * 4 + r;
        if (row < tl.rows) {
          const int slot = sorted_slots[tl.row_start + row];
          float* yrow = reinterpret_cast<float*>(out) + (size_t)slot * Ndim + n0 + wn * 128 + (lane & 15);
#pragma unroll
          for (int j = 0; j < 8; ++j) yrow[16 * j] = acc[i][j][r];
        }
      }
  }
}

hipError_t launch_gateup_gemm(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                              int max_tiles, const uint16_t* wg, const uint16_t* wu, uint16_t* h, uint8_t* hscale,
                              int H, int I, int K, hipStream_t st) {
  const int nbn = I / (kGemmBN / 2);
  const int total = max_tiles * nbn;
  hipLaunchKernelGGL(expert_gemm_kernel<true>, dim3(total), dim3(256), 0, st, x, slots, tiles, ntiles, wg, wu,
                     (void*)h, hscale, H, I, K, nbn, total);
  return hipGetLastError();
}

hipError_t launch_down_gemm(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                            const int32_t* ntiles, int max_tiles, const uint16_t* wd, float* y, int H, int I,
                            hipStream_t st) {
  const int nbn = H / kGemmBN;
  const int total = max_tiles * nbn;
  hipLaunchKernelGGL(expert_gemm_kernel<false>, dim3(total), dim3(256), 0, st, h, slots, tiles, ntiles, wd, nullptr,
                     (void*)y, const_cast<uint8_t*>(hscale), I, H, 0, nbn, total);
  return hipGetLastError();
}

// Tile shapes of the tiled path.
constexpr int kGuBM = 256, kGuBN = 128;  // gate/up: 256 rows x (128 gate + 128 up) columns
constexpr int kDnBM = 256, kDnBN = 256;  // down: 256 rows x 256 columns
// the down kernel reads the activation scales of the gate/up tile with the same rows
static_assert(kGuBM == kDnBM, "gate/up and down share one tile table");
static_assert(kGuBN % kScaleCols == 0, "scale blocks tile the gate/up columns");

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
int tiled_gateup_rows() { return kGuBM; }
int tiled_down_rows() { return kDnBM; }
int tiled_gateup_cols() { return kGuBN; }
int tiled_down_cols() { return kDnBN; }

int scale_cols() { return kScaleCols; }

// ---------------------------------------------------------------------------
// stream kernels with the activation rows staged in LDS (very few rows per expert)
// ---------------------------------------------------------------------------
// Same work split as above (one expert per workgroup, 16 columns per wave over
// the whole K), but a pass takes at most 8 rows and copies them, whole-K, into
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

// Stream kernel shapes: 16 columns per wave, eight 32-wide steps per register stage.
constexpr int kGuCB = 1, kGuU = 8;
constexpr int kDnCB = 1, kDnU = 8;

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
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gateup_stream_lds_kernel<8, kLdsRows>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gateup_stream_lds_kernel<8, kLdsRows>), grid, dim3(256), bytes, st, x, slots, tiles, ntiles, wg, wu, h,
                       hscale, H, I, K);
  } else {
    hipLaunchKernelGGL((gateup_stream_kernel<kGuU, kGuCB>), grid, dim3(256), 0, st, x, slots, tiles, ntiles, wg, wu,
                       h, hscale, H, I, K);
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
      hipLaunchKernelGGL((down_stream_lds_kernel<8, kLdsRows>), grid, dim3(256), bytes, st, h, hscale, slots, tiles, ntiles, wd,
                         y, H, I);
    else
      hipLaunchKernelGGL((down_stream_lds_kernel<4, kLdsRows>), grid, dim3(256), bytes, st, h, hscale, slots, tiles, ntiles, wd,
                         y, H, I);
  } else if (u8) {
    hipLaunchKernelGGL((down_stream_kernel<8, 1>), grid, dim3(256), 0, st, h, hscale, slots, tiles, ntiles, wd, y, H,
                       I);
  } else {
    hipLaunchKernelGGL((down_stream_kernel<4, 1>), grid, dim3(256), 0, st, h, hscale, slots, tiles, ntiles, wd, y, H,
                       I);
  }
  return hipGetLastError();
}

hipError_t launch_gateup_tiled(const uint16_t* x, const int32_t* slots, const Tile* tiles, const int32_t* ntiles,
                               int max_tiles, const uint16_t* wg, const uint16_t* wu, uint16_t* h, uint8_t* hscale,
                               int H, int I, int K, hipStream_t st) {
  const int nbn = I / kGuBN;
  const int total = max_tiles * nbn;
  hipLaunchKernelGGL((expert_tiled_kernel<true, kGuBM, kGuBN, 4, 2>), dim3(total), dim3(512), 0, st, x, slots,
                     tiles, ntiles, wg, wu, (void*)h, hscale, H, I, K, nbn, total);
  return hipGetLastError();
}

hipError_t launch_down_tiled(const uint16_t* h, const uint8_t* hscale, const int32_t* slots, const Tile* tiles,
                             const int32_t* ntiles, int max_tiles, const uint16_t* wd, float* y, int H, int I,
                             hipStream_t st) {
  const int nbn = H / kDnBN;
  const int total = max_tiles * nbn;
  hipLaunchKernelGGL((expert_tiled_kernel<false, kDnBM, kDnBN, 4, 2>), dim3(total), dim3(512), 0, st, h, slots,
                     tiles, ntiles, wd, nullptr, (void*)y, const_cast<uint8_t*>(hscale), I, H, 0, nbn, total);
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
