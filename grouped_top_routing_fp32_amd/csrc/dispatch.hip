// Counting-sort dispatch of the Beam MoE block (gfx950).
//
// Every token runs exactly K experts (「Reflection 发布 Beam 501B 开源模型，支持 1M tokens 上下文」,
// section 专家混合模型, mixture of experts), so the T*K (token, slot) pairs are grouped by expert for the
// grouped expert GEMMs: a per-expert histogram, an exclusive scan and a
// stable scatter.  The scatter ranks equal ids inside a wavefront with
// ballots on the id's bits (a wave-level multisplit), never with atomics on
// positions, so the permutation is the unique stable one on every run.
//
// Kernels:
//   dispatch_hist_kernel     one workgroup per unit of kUnit pairs: LDS histogram
//   dispatch_scan_kernel     one workgroup: per-unit bases, counts, offsets and
//                            the grouped-GEMM tile tables
//   dispatch_scatter_kernel  one workgroup per unit: stable placement
//   dispatch_small_kernel    all three in one workgroup for small batches
#include "common.h"

namespace beam {

constexpr int kUnit = 1024;      // pairs per unit (4 waves x 256)
constexpr int kWavePairs = 256;  // pairs per wave inside a unit

__global__ __launch_bounds__(256) void dispatch_hist_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                            int32_t* __restrict__ unit_hist) {
  __shared__ int h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int base = blockIdx.x * kUnit;
  for (int i = tid; i < kUnit; i += 256) {
    const int idx = base + i;
    if (idx < n) {
      const int v = ids[idx];
      if ((unsigned)v < (unsigned)E) atomicAdd(&h[v], 1);
    }
  }
  __syncthreads();
  if (tid < E) unit_hist[(size_t)blockIdx.x * E + tid] = h[tid];
}

// Exclusive scan of one int per thread over a 256-thread block.
__device__ int block_exclusive_scan(int v, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int incl = buf[tid];
  __syncthreads();
  return incl - v;
}

// Writes the tiles of one expert: rows [off, off + cnt) cut into pieces of at
// most `mt` rows, tile i at index first + i, in groups of kTileGroupMax tiles.
__device__ void write_tiles(Tile* tiles, int first, int e, int off, int cnt, int mt) {
  const int nt = (cnt + mt - 1) / mt;
  for (int i = 0, r = 0; r < cnt; ++i, r += mt) {
    const int g0 = i / kTileGroupMax * kTileGroupMax;
    Tile tl;
    tl.expert = e;
    tl.row_start = off + r;
    tl.rows = min(mt, cnt - r);
    tl.group_first = first + g0;
    tl.group_size = min(kTileGroupMax, nt - g0);
    tl.pad[0] = tl.pad[1] = tl.pad[2] = 0;
    tiles[first + i] = tl;
  }
}

// One workgroup of 256 threads; thread e owns expert e.
// unit_hist: in = per-unit counts, out = per-unit base of each expert inside
// the expert's segment (the scatter adds the segment offset).
// tiles (optional): tile table with at most mt rows per tile, count in ntiles[0].
__global__ __launch_bounds__(256) void dispatch_scan_kernel(int32_t* __restrict__ unit_hist, int units, int E, int n,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets, Tile* __restrict__ tiles,
                                                            int mt, int32_t* __restrict__ ntiles) {
  __shared__ int buf[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    int u = 0;
    for (; u + 16 <= units; u += 16) {
      int c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = unit_hist[(size_t)(u + i) * E + e];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        unit_hist[(size_t)(u + i) * E + e] = run;
        run += c[i];
      }
    }
    for (; u < units; ++u) {
      const int c = unit_hist[(size_t)u * E + e];
      unit_hist[(size_t)u * E + e] = run;
      run += c;
    }
  }
  const int cnt = e < E ? run : 0;
  const int off = block_exclusive_scan(cnt, buf);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    if (e == E - 1) offsets[E] = off + cnt;
  }
  if (tiles) {
    const int nt = cnt > 0 ? (cnt + mt - 1) / mt : 0;
    const int first = block_exclusive_scan(nt, buf);
    if (e < E) write_tiles(tiles, first, e, off, cnt, mt);
    if (e == 255) ntiles[0] = first + nt;
  }
}

// Ranks 64 pairs at a time in ascending index order and places them: the
// rank of a pair among equal ids of its round comes from ballots on the id's
// bits; `base` (one LDS array per wave) holds each expert's next position and
// is advanced by the last lane of each run of equal ids.
__device__ __forceinline__ void place_round(const int32_t* __restrict__ ids, int idx, int n, int E, int* base,
                                            int32_t* __restrict__ sorted_slots) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  int v = -1;
  if (idx < n) {
    v = ids[idx];
    if ((unsigned)v >= (unsigned)E) v = -1;
  }
  const bool ok = v >= 0;
  unsigned long long match = __ballot(ok);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool b = ok && ((v >> bit) & 1);
    const unsigned long long m = __ballot(b);
    match &= b ? m : ~m;
  }
  if (ok) sorted_slots[base[v] + __popcll(match & below)] = idx;
  if (ok && (match >> lane) == 1ull) base[v] += __popcll(match);
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                               const int32_t* __restrict__ unit_base,
                                                               const int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_slots) {
  __shared__ int base[4][256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
#pragma unroll
  for (int w = 0; w < 4; ++w) base[w][tid] = 0;
  __syncthreads();
  const int wbase = blockIdx.x * kUnit + wave * kWavePairs;
  // pass 1: per-wave counts
  for (int r = 0; r < kWavePairs; r += 64) {
    const int idx = wbase + r + lane;
    if (idx < n) {
      const int v = ids[idx];
      if ((unsigned)v < (unsigned)E) atomicAdd(&base[wave][v], 1);
    }
  }
  __syncthreads();
  // per-wave bases: segment offset + unit base + earlier waves of this unit
  if (tid < E) {
    int run = offsets[tid] + unit_base[(size_t)blockIdx.x * E + tid];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = base[w][tid];
      base[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  // pass 2: stable placement
  for (int r = 0; r < kWavePairs; r += 64) place_round(ids, wbase + r + lane, n, E, base[wave], sorted_slots);
}

// The three steps in one workgroup, for small batches (n <= kSmallPairs):
// wave w owns the contiguous range [w*q, (w+1)*q) of pairs, q a multiple of 64.
constexpr int kSmallPairs = 4096;

__global__ __launch_bounds__(256) void dispatch_small_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_slots,
                                                             Tile* __restrict__ tiles, int mt,
                                                             int32_t* __restrict__ ntiles) {
  __shared__ int base[4][256];
  __shared__ int buf[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = ((n + 255) / 256) * 64;
  const int w0 = wave * q;
#pragma unroll
  for (int w = 0; w < 4; ++w) base[w][tid] = 0;
  __syncthreads();
  for (int r = 0; r < q; r += 64) {
    const int idx = w0 + r + lane;
    if (idx < n) {
      const int v = ids[idx];
      if ((unsigned)v < (unsigned)E) atomicAdd(&base[wave][v], 1);
    }
  }
  __syncthreads();
  const int e = tid;
  const int cnt = e < E ? base[0][e] + base[1][e] + base[2][e] + base[3][e] : 0;
  const int off = block_exclusive_scan(cnt, buf);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    if (e == E - 1) offsets[E] = off + cnt;
    int run = off;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = base[w][e];
      base[w][e] = run;
      run += c;
    }
  }
  if (tiles) {
    const int nt = cnt > 0 ? (cnt + mt - 1) / mt : 0;
    const int first = block_exclusive_scan(nt, buf);
    if (e < E) write_tiles(tiles, first, e, off, cnt, mt);
    if (e == 255) ntiles[0] = first + nt;
  }
  __syncthreads();
  for (int r = 0; r < q; r += 64) place_round(ids, w0 + r + lane, n, E, base[wave], sorted_slots);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
int dispatch_units(int n) { return (n + kUnit - 1) / kUnit; }

hipError_t launch_dispatch(const int32_t* ids, int n, int E, int32_t* unit_hist, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_slots, Tile* tiles, int mt, int32_t* ntiles, hipStream_t st) {
  if (n <= kSmallPairs) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(256), 0, st, ids, n, E, counts, offsets, sorted_slots,
                       tiles, mt, ntiles);
    return hipGetLastError();
  }
  const int units = dispatch_units(n);
  hipLaunchKernelGGL(dispatch_hist_kernel, dim3(units), dim3(256), 0, st, ids, n, E, unit_hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(256), 0, st, unit_hist, units, E, n, counts, offsets,
                     tiles, mt, ntiles);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(units), dim3(256), 0, st, ids, n, E, unit_hist, offsets,
                     sorted_slots);
  return hipGetLastError();
}

}  // namespace beam
