// Counting-sort dispatch of the Beam MoE block (gfx950).
//
// Every token runs exactly K experts (Beam launch blog, "mixture of experts"
// section), so the T*K (token, slot) pairs are grouped by expert for the
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

// Writes the tiles of one expert: rows [off, off + cnt) cut into pieces of at most `mt` rows.
__device__ void write_tiles(Tile* tiles, int first, int e, int off, int cnt, int mt) {
  for (int i = 0, r = 0; r < cnt; ++i, r += mt) {
    Tile tl;
    tl.expert = e;
    tl.row_start = off + r;
    tl.rows = min(mt, cnt - r);
    tl.pad = 0;
    tiles[first + i] = tl;
  }
}

// One workgroup of 256 threads; thread e owns expert e.
// unit_hist: in = per-unit counts, out = per-unit global base of each expert.
// tiles_a/tiles_b (optional): tile tables with at most mt_a / mt_b rows per tile.
__global__ __launch_bounds__(256) void dispatch_scan_kernel(int32_t* __restrict__ unit_hist, int units, int E, int n,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets, Tile* __restrict__ tiles_a,
                                                            int mt_a, Tile* __restrict__ tiles_b, int mt_b,
                                                            int32_t* __restrict__ ntiles) {
  __shared__ int buf[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int u = 0; u < units; ++u) {
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
    for (int u = 0; u < units; ++u) unit_hist[(size_t)u * E + e] += off;
  }
  if (tiles_a) {
    const int nt = cnt > 0 ? (cnt + mt_a - 1) / mt_a : 0;
    const int first = block_exclusive_scan(nt, buf);
    if (e < E) write_tiles(tiles_a, first, e, off, cnt, mt_a);
    if (e == 255) ntiles[0] = first + nt;
  }
  if (tiles_b) {
    const int nt = cnt > 0 ? (cnt + mt_b - 1) / mt_b : 0;
    const int first = block_exclusive_scan(nt, buf);
    if (e < E) write_tiles(tiles_b, first, e, off, cnt, mt_b);
    if (e == 255) ntiles[1] = first + nt;
  }
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                               const int32_t* __restrict__ unit_base,
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
  // per-wave bases: unit base + earlier waves of this unit
  if (tid < E) {
    int run = unit_base[(size_t)blockIdx.x * E + tid];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = base[w][tid];
      base[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  // pass 2: stable placement, 64 pairs at a time in ascending index order
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = 0; r < kWavePairs; r += 64) {
    const int idx = wbase + r + lane;
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
    if (ok) {
      const int rank = __popcll(match & below);
      const int pos = base[wave][v] + rank;
      sorted_slots[pos] = idx;
    }
    // the last lane of each run of equal ids advances that id's base
    if (ok && (match >> lane) == 1ull) base[wave][v] += __popcll(match);
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
int dispatch_units(int n) { return (n + kUnit - 1) / kUnit; }

hipError_t launch_dispatch(const int32_t* ids, int n, int E, int32_t* unit_hist, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_slots, Tile* tiles_a, int mt_a, Tile* tiles_b, int mt_b, int32_t* ntiles,
                           hipStream_t st) {
  const int units = dispatch_units(n);
  hipLaunchKernelGGL(dispatch_hist_kernel, dim3(units), dim3(256), 0, st, ids, n, E, unit_hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(256), 0, st, unit_hist, units, E, n, counts, offsets,
                     tiles_a, mt_a, tiles_b, mt_b, ntiles);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(units), dim3(256), 0, st, ids, n, E, unit_hist, sorted_slots);
  return hipGetLastError();
}

}  // namespace beam
