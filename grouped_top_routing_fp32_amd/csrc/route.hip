// Router and group-limited top-k selection of the Beam MoE block (gfx950).
//
// 「Reflection 发布 Beam 501B 开源模型，支持 1M tokens 上下文」 (the Chinese
// translation of the Hugging Face post "Welcome Beam: a 501B open model you
// can own, customize, and scale"), section 专家混合模型 (mixture of experts):
// every expert gets a sigmoid score; experts form n_group groups; a group is
// ranked by the sum of its two best scores; the topk_group best groups are
// kept; the top-k experts inside them are chosen; their weights are
// normalised and multiplied by 2.5.  Section 残差流 (residual stream) puts
// the router in FP32.
//
// Two kernels:
//   router_logits_kernel  FP32-exact logits on bf16 MFMA.  x is bf16, W_r is
//       fp32; each W_r element is split exactly into three bf16 pieces
//       (w = hi + mid + lo), so every product x*piece is exact in FP32 and
//       the MFMA accumulates in FP32: an FP32 contraction at bf16-MFMA rate.
//       The K dimension may be split across workgroups; partial sums land in
//       workspace and are added in a fixed order by the select kernel.
//   select_kernel  one wave per token: partial sums + bias + sigmoid, then the
//       group top-2 sums, the kept groups and K rounds of a wave-wide argmax,
//       on the scores or, with a selection-only bias, on score + bias (the
//       weights always from the unbiased scores).
#include <type_traits>

#include "common.h"

namespace beam {

constexpr int kRtM = 64;       // tokens per router tile (128 for large batches, see the launcher)
constexpr int kRtN = 64;       // experts per router tile
constexpr int kRtK = 32;       // K step
constexpr int kRtLd = kRtK + 8;  // LDS row stride in bf16 elements (80 bytes: conflict-free 16-byte reads)

// Exact three-way split of an fp32 value into bf16 pieces (truncation; the
// remainders are exact in fp32 and the last piece has at most 8 significant bits).
__device__ __forceinline__ void split3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  uint32_t u = __float_as_uint(w);
  hi = uint16_t(u >> 16);
  float r1 = w - __uint_as_float(u & 0xFFFF0000u);
  uint32_t v = __float_as_uint(r1);
  mid = uint16_t(v >> 16);
  float r2 = r1 - __uint_as_float(v & 0xFFFF0000u);
  lo = uint16_t(__float_as_uint(r2) >> 16);
}

// grid: (ceil(T/MR), ceil(E/64), splits); block 4 MR (MR/16 waves, wave w = tokens 16w..16w+15).
// A taller token tile (MR = 128) shares each staged W_r step, and its split into
// bf16 pieces, among twice the tokens.
template <int MR>
__global__ __launch_bounds__(4 * MR) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                               const float* __restrict__ wr, float* __restrict__ part,
                                                               int T, int H, int E, int k_per_split) {
  constexpr int kThreads = 4 * MR;
  constexpr int kWC = (kRtN * kRtK / 4) / kThreads;  // 4-float W_r chunks per thread per step
  static_assert(kWC >= 1 && kWC * kThreads == kRtN * kRtK / 4, "W_r staging covers the step");
  __shared__ __attribute__((aligned(16))) uint16_t sA[MR * kRtLd];
  __shared__ __attribute__((aligned(16))) uint16_t sB[3][kRtN * kRtLd];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * MR;
  const int e0 = blockIdx.y * kRtN;
  const int kbeg = blockIdx.z * k_per_split;
  const int kend = min(H, kbeg + k_per_split);

  // staging assignments: x: one 16-byte chunk per thread; W_r: two 4-float chunks per thread
  const int xa_row = tid >> 2, xa_kc = tid & 3;
  const uint16_t* xsrc = x + (size_t)min(t0 + xa_row, T - 1) * H + xa_kc * 8;
  int wb_row[kWC], wb_kc[kWC];
  const float* wsrc[kWC];
#pragma unroll
  for (int i = 0; i < kWC; ++i) {
    int c = tid + kThreads * i;
    wb_row[i] = c >> 3;
    wb_kc[i] = c & 7;
    wsrc[i] = wr + (size_t)min(e0 + wb_row[i], E - 1) * H + wb_kc[i] * 4;
  }

  f32x4 acc_hi[4], acc_lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc_hi[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc_lo[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Operands of step k are loaded during step k - 64 (two steps in flight): a
  // split has few steps at small T, each bound by the latency of its loads.  The
  // two register sets take turns (the loop runs two steps per turn so that each
  // is named at compile time: a register copy would wait for its loads).  Every
  // step issues its loads, from the split's last step where it runs past it, so
  // that the compiler's waits count a fixed number of loads in flight.
  u32x4 xv[2];
  f32x4 wv[2][kWC];
  const int klast = kend - kRtK;
  auto load = [&](u32x4& xr, f32x4(&wr4)[kWC], int k) {
    k = min(k, klast);
    xr = ldg16(xsrc + k);
#pragma unroll
    for (int i = 0; i < kWC; ++i) wr4[i] = *reinterpret_cast<const f32x4*>(wsrc[i] + k);
  };
  auto step = [&](int k, u32x4& xr, f32x4(&wr4)[kWC]) {
    __syncthreads();  // previous step's fragment reads are done
    *reinterpret_cast<u32x4*>(&sA[xa_row * kRtLd + xa_kc * 8]) = xr;
#pragma unroll
    for (int i = 0; i < kWC; ++i) {
      uint16_t hi[4], mid[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) split3(wr4[i][q], hi[q], mid[q], lo[q]);
      const int off = wb_row[i] * kRtLd + wb_kc[i] * 4;
      uint2 ph, pm, pl;
      ph.x = hi[0] | (uint32_t(hi[1]) << 16);
      ph.y = hi[2] | (uint32_t(hi[3]) << 16);
      pm.x = mid[0] | (uint32_t(mid[1]) << 16);
      pm.y = mid[2] | (uint32_t(mid[3]) << 16);
      pl.x = lo[0] | (uint32_t(lo[1]) << 16);
      pl.y = lo[2] | (uint32_t(lo[3]) << 16);
      *reinterpret_cast<uint2*>(&sB[0][off]) = ph;
      *reinterpret_cast<uint2*>(&sB[1][off]) = pm;
      *reinterpret_cast<uint2*>(&sB[2][off]) = pl;
    }
    __syncthreads();
    load(xr, wr4, k + 2 * kRtK);
    const int arow = wave * 16 + (lane & 15);
    const int kk = (lane >> 4) * 8;
    u32x4 a = *reinterpret_cast<const u32x4*>(&sA[arow * kRtLd + kk]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int brow = j * 16 + (lane & 15);
      u32x4 bh = *reinterpret_cast<const u32x4*>(&sB[0][brow * kRtLd + kk]);
      u32x4 bm = *reinterpret_cast<const u32x4*>(&sB[1][brow * kRtLd + kk]);
      u32x4 bl = *reinterpret_cast<const u32x4*>(&sB[2][brow * kRtLd + kk]);
      acc_hi[j] = mfma16x16x32(a, bh, acc_hi[j]);
      acc_lo[j] = mfma16x16x32(a, bl, acc_lo[j]);
      acc_lo[j] = mfma16x16x32(a, bm, acc_lo[j]);
    }
  };
  // kend - kbeg is a positive multiple of kRtK (H % 256 == 0, k_per_split % 32 == 0)
  const int nsteps = (kend - kbeg) / kRtK;
  load(xv[0], wv[0], kbeg);
  load(xv[1], wv[1], kbeg + kRtK);
  int k = kbeg;
  for (int p = 0; p < nsteps / 2; ++p, k += 2 * kRtK) {
    step(k, xv[0], wv[0]);
    step(k + kRtK, xv[1], wv[1]);
  }
  if (nsteps & 1) step(k, xv[0], wv[0]);

  float* dst = part + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + j * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + wave * 16 + (lane >> 4) * 4 + r;
      if (t < T && e < E) dst[(size_t)t * E + e] = acc_hi[j][r] + acc_lo[j][r];
    }
  }
}

// Order used by every selection step: higher score first, lower index on ties.
__device__ __forceinline__ bool beats(float v, int i, float ov, int oi) { return v > ov || (v == ov && i < oi); }

// grid: ceil(T/4); block 256: one wave per token.
// src: partial logits [splits][T][E] (from_partials) or post-sigmoid scores [T][E].
// sel_bias (optional): selection-only bias; groups and experts are ranked by
// c = fl32(s + sel_bias[e]), the weights use the unbiased s.
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ src, int splits, bool from_partials,
                                                     const float* __restrict__ bias,
                                                     const float* __restrict__ sel_bias,
                                                     float* __restrict__ scores_out, int T, int E, int G, int TG,
                                                     int K, float scale, int32_t* __restrict__ ids,
                                                     float* __restrict__ wout) {
#pragma clang fp contract(off)
  __shared__ __attribute__((aligned(16))) float s_sc[4][256];
  __shared__ __attribute__((aligned(16))) float s_gs[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool active = t < T;
  const int gsz = E / G;

  float v[4];  // unbiased scores
  float c[4];  // selection values
  bool valid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = 0.f;
    c[j] = 0.f;
    if (active && e < E) {
      if (from_partials) {
        // split-K partial logits, added in ascending split order; loads are
        // issued eight at a time so they overlap
        const size_t plane = (size_t)T * E;
        const float* ps = src + (size_t)t * E + e;
        float L = 0.f;
        int s = 0;
        for (; s + 8 <= splits; s += 8) {
          float q[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) q[i] = ps[(size_t)(s + i) * plane];
#pragma unroll
          for (int i = 0; i < 8; ++i) L = (s + i == 0) ? q[i] : L + q[i];
        }
        for (; s < splits; ++s) L = (s == 0) ? ps[0] : L + ps[(size_t)s * plane];
        if (bias) L = L + bias[e];
        v[j] = 1.0f / (1.0f + expf(-L));
        if (scores_out) scores_out[(size_t)t * E + e] = v[j];
      } else {
        v[j] = src[(size_t)t * E + e];
      }
      c[j] = sel_bias ? v[j] + sel_bias[e] : v[j];
      s_sc[wave][e] = c[j];
    }
  }
  __syncthreads();

  // group score: sum of the two largest selection values of the group (one lane per group),
  // the values taken in index order; read four at a time where the groups allow it
  if (active && lane < G) {
    float m1 = -INFINITY, m2 = -INFINITY;
    const float* g = &s_sc[wave][lane * gsz];
    if (gsz % 4 == 0) {
#pragma unroll 4
      for (int i = 0; i < gsz; i += 4) {
        const f32x4 q = *reinterpret_cast<const f32x4*>(g + i);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float v = q[u];
          m2 = v > m1 ? m1 : (v > m2 ? v : m2);
          m1 = v > m1 ? v : m1;
        }
      }
    } else {
      for (int i = 0; i < gsz; ++i) {
        const float v = g[i];
        m2 = v > m1 ? m1 : (v > m2 ? v : m2);
        m1 = v > m1 ? v : m1;
      }
    }
    s_gs[wave][lane] = (gsz >= 2) ? (m1 + m2) : m1;
  }
  __syncthreads();

  bool keep = false;
  if (active && lane < G) {
    const float mine = s_gs[wave][lane];
    int rank = 0;
    if (G % 4 == 0) {
      for (int g = 0; g < G; g += 4) {
        const f32x4 q = *reinterpret_cast<const f32x4*>(&s_gs[wave][g]);
#pragma unroll
        for (int u = 0; u < 4; ++u) rank += beats(q[u], g + u, mine, lane) ? 1 : 0;
      }
    } else {
      for (int g = 0; g < G; ++g) rank += beats(s_gs[wave][g], g, mine, lane) ? 1 : 0;
    }
    keep = rank < TG;
  }
  const unsigned long long kept = __ballot(keep);
  if (!active) return;  // no barrier follows

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    valid[j] = e < E && ((kept >> (e / gsz)) & 1ull);
  }

  // K rounds of a wave-wide argmax of (c, e).  Each candidate is one 64-bit key,
  // ordered as beats() orders (c, e): the high word maps c to an unsigned integer
  // of the same order (-0 taken as +0, which beats() ranks equal), the low word is
  // ~e, so equal values go to the lower index.  A round reduces the lane maxima
  // inside each row of 16 lanes with DPP moves (quad swaps, then rotations by 4
  // and 8) and across the four rows with readlanes; the winner's unbiased score
  // comes from its lane for the weights.
  uint64_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = __float_as_uint(c[j] + 0.0f);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    key[j] = ((uint64_t)o << 32) | (uint32_t)~(uint32_t)(lane + 64 * j);
  }
  auto kmax = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  auto dpp_max = [&](uint64_t a, auto ctrl) {
    constexpr int kCtrl = decltype(ctrl)::value;
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)a, kCtrl, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(a >> 32), kCtrl, 0xF, 0xF, false);
    return kmax(a, ((uint64_t)hi << 32) | lo);
  };
  auto read_lane = [](uint64_t a, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)a, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(a >> 32), l);
    return ((uint64_t)hi << 32) | lo;
  };
  float total = 0.f;
  float my_v = 0.f;
  int my_e = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;  // below every candidate's key
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (valid[j]) best = kmax(best, key[j]);
    best = dpp_max(best, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    best = dpp_max(best, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
    best = dpp_max(best, std::integral_constant<int, 0x124>{});  // row_ror:4
    best = dpp_max(best, std::integral_constant<int, 0x128>{});  // row_ror:8
    best = kmax(kmax(read_lane(best, 0), read_lane(best, 16)), kmax(read_lane(best, 32), read_lane(best, 48)));
    const int be = (int)~(uint32_t)best;  // the winner (uniform)
    const int wj = be >> 6, wl = be & 63;
    const float mine = wj == 0 ? v[0] : wj == 1 ? v[1] : wj == 2 ? v[2] : v[3];
    const float bs = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mine), wl));
    if (wl == lane) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == wj) valid[j] = false;
    }
    total = total + bs;
    if (lane == k) {
      my_v = bs;
      my_e = be;
    }
  }
  if (lane < K) {
    const float q = my_v / total;
    ids[(size_t)t * K + lane] = my_e;
    wout[(size_t)t * K + lane] = q * scale;
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const uint16_t* x, const float* wr, float* part, int T, int H, int E, int splits,
                                int k_per_split, hipStream_t st) {
  // 128-token tiles once even they make 512 workgroups (the K split is then 1; measured
  // 0.245 -> 0.209 ms at T = 16384, no change at 8192)
  const int etiles = (E + kRtN - 1) / kRtN;
  if (splits == 1 && ((T + 127) / 128) * etiles >= 512) {
    dim3 grid((T + 127) / 128, etiles, 1);
    hipLaunchKernelGGL(router_logits_kernel<128>, grid, dim3(512), 0, st, x, wr, part, T, H, E, k_per_split);
  } else {
    dim3 grid((T + kRtM - 1) / kRtM, etiles, splits);
    hipLaunchKernelGGL(router_logits_kernel<kRtM>, grid, dim3(4 * kRtM), 0, st, x, wr, part, T, H, E, k_per_split);
  }
  return hipGetLastError();
}

hipError_t launch_select(const float* src, int splits, bool from_partials, const float* bias,
                         const float* select_bias, float* scores_out, int T, int E, int G, int TG, int K, float scale,
                         int32_t* ids, float* w, hipStream_t st) {
  dim3 grid((T + 3) / 4);
  hipLaunchKernelGGL(select_kernel, grid, dim3(256), 0, st, src, splits, from_partials, bias, select_bias, scores_out,
                     T, E, G, TG, K, scale, ids, w);
  return hipGetLastError();
}

}  // namespace beam
