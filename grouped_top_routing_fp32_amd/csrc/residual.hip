// The Beam MoE block as a residual sublayer (gfx950): pre-norm of the stream
// and the fused post-norm + scaled residual update.
//
// 「Reflection 发布 Beam 501B 开源模型，支持 1M tokens 上下文」 (the Chinese
// translation of the Hugging Face post "Welcome Beam: a 501B open model you
// can own, customize, and scale"), section 残差流 (residual stream): the input
// embedding is step 1; at step k a sublayer's output is added with weight
// 1/sqrt(k) and the stream kept with weight sqrt((k-1)/k); every sublayer is
// normalised before and after, in FP32.  The norm is taken as RMSNorm,
// v / sqrt(mean(v^2) + eps) * g (form, weights and eps are not on the pages).
//
//   prenorm_kernel           x[t] = bf16(norm(stream[t]) * g_in)
//   combine_residual_kernel  out = sum_k w[t,k] y[t*K+k] (as the combine),
//                            stream'[t] = a * stream[t] + b * norm(out) * g_out
// The norm statistics are taken in FP64 (FP32 or better, as the pages ask):
// the bf16 rounding of x is then decided by the same value an FP64 oracle
// computes.  One workgroup per token, of ceil(H / 8 / 64) waves; a thread
// owns 8 consecutive columns (c = 8 * tid) and keeps them in registers, so
// each row is read once and H <= 8 * 1024.
#include "common.h"

namespace beam {

constexpr int kResColsPerThread = 8;
constexpr int kResMaxThreads = 1024;  // H <= 8192
constexpr int kResMaxK = 16;

// Sum over the block's waves, FP64, in a fixed order (every thread gets the result).
__device__ double block_sum(double v, double* buf) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0) buf[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < nw; ++i) s += buf[i];
  return s;
}

__device__ __forceinline__ void load8(const float* p, float* v) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = a[q];
    v[q + 4] = b[q];
  }
}

__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// grid: T; block ceil(H / 8 / 64) * 64.  g_in may be null (unit weights).
__global__ __launch_bounds__(kResMaxThreads) void prenorm_kernel(const float* __restrict__ stream,
                                                                 const float* __restrict__ g_in,
                                                                 uint16_t* __restrict__ x, int H, double eps) {
  __shared__ double buf[kResMaxThreads / 64];
  const int t = blockIdx.x;
  const int c = kResColsPerThread * threadIdx.x;
  const bool own = c < H;
  float v[8];
  double ss = 0.0;
  if (own) {
    load8(stream + (size_t)t * H + c, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) ss += (double)v[q] * (double)v[q];
  }
  const double inv = 1.0 / sqrt(block_sum(ss, buf) / H + eps);
  if (own) {
    float g[8];
    if (g_in) {
      load8(g_in + c, g);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) g[q] = 1.f;
    }
    u32x4 packed;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint16_t lo = f32_to_bf16_rne((float)((double)v[2 * q] * inv * (double)g[2 * q]));
      const uint16_t hi = f32_to_bf16_rne((float)((double)v[2 * q + 1] * inv * (double)g[2 * q + 1]));
      packed[q] = lo | ((uint32_t)hi << 16);
    }
    *reinterpret_cast<u32x4*>(x + (size_t)t * H + c) = packed;
  }
}

// grid: T; block ceil(H / 8 / 64) * 64.  y16/yscale/w as for the combine; the K
// rows of a token are loaded together, then summed in ascending k in FP32.
// stream_out may alias stream_in: every element is read and written by the same thread.
__global__ __launch_bounds__(kResMaxThreads) void combine_residual_kernel(
    const uint16_t* __restrict__ y16, const uint8_t* __restrict__ yscale, const float* __restrict__ w,
    const float* stream_in, const float* __restrict__ g_out, float* stream_out, int H, int K, float a, float b,
    double eps) {
  __shared__ double buf[kResMaxThreads / 64];
  const int t = blockIdx.x;
  const int c = kResColsPerThread * threadIdx.x;
  const bool own = c < H;
  const size_t row0 = (size_t)t * K;
  const int nsb = H / kScaleCols;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  double ss = 0.0;
  if (own) {
    u32x4 raw[kResMaxK];
    int sc[kResMaxK];
#pragma unroll
    for (int k = 0; k < kResMaxK; ++k)
      if (k < K) {
        raw[k] = *reinterpret_cast<const u32x4*>(y16 + (row0 + k) * H + c);
        sc[k] = yscale[(row0 + k) * nsb + c / kScaleCols];
      }
#pragma unroll
    for (int k = 0; k < kResMaxK; ++k)
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
#pragma unroll
    for (int q = 0; q < 8; ++q) ss += (double)acc[q] * (double)acc[q];
  }
  const float inv = (float)(1.0 / sqrt(block_sum(ss, buf) / H + eps));
  if (own) {
    float s[8], g[8], r[8];
    load8(stream_in + (size_t)t * H + c, s);
    if (g_out) {
      load8(g_out + c, g);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) g[q] = 1.f;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) r[q] = a * s[q] + b * (acc[q] * inv * g[q]);
    store8(stream_out + (size_t)t * H + c, r);
  }
}

static int res_threads(int H) { return ((H / kResColsPerThread + 63) / 64) * 64; }

bool residual_fits(int H) { return H % kResColsPerThread == 0 && res_threads(H) <= kResMaxThreads; }

hipError_t launch_prenorm(const float* stream, const float* g_in, uint16_t* x, int T, int H, float eps,
                          hipStream_t st) {
  hipLaunchKernelGGL(prenorm_kernel, dim3(T), dim3(res_threads(H)), 0, st, stream, g_in, x, H, (double)eps);
  return hipGetLastError();
}

hipError_t launch_combine_residual(const uint16_t* y16, const uint8_t* yscale, const float* w, const float* stream_in,
                                   const float* g_out, float* stream_out, int T, int H, int K, int step, float eps,
                                   hipStream_t st) {
  if (K > kResMaxK) return hipErrorInvalidValue;
  const float a = (float)sqrt((double)(step - 1) / step), b = (float)(1.0 / sqrt((double)step));
  hipLaunchKernelGGL(combine_residual_kernel, dim3(T), dim3(res_threads(H)), 0, st, y16, yscale, w, stream_in, g_out,
                     stream_out, H, K, a, b, (double)eps);
  return hipGetLastError();
}

}  // namespace beam
