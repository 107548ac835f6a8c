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
// computes.  One workgroup per token; a thread keeps its columns in registers
// (c = 4 * tid + 1024 * j, j < kMaxChunks), so H <= 1024 * kMaxChunks.
#include "common.h"

namespace beam {

constexpr int kMaxChunks = 8;  // H <= 8192
constexpr int kResCols = 1024;  // columns per chunk (256 threads x 4)

// Sum over the block's 256 threads, FP64; every thread gets the result.
__device__ double block_sum(double v, double* buf) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // buf may still be read from a previous use
  if (lane == 0) buf[wave] = v;
  __syncthreads();
  return (buf[0] + buf[1]) + (buf[2] + buf[3]);
}

// grid: T; block 256.  g_in may be null (unit weights).
__global__ __launch_bounds__(256) void prenorm_kernel(const float* __restrict__ stream, const float* __restrict__ g_in,
                                                      uint16_t* __restrict__ x, int H, double eps) {
  __shared__ double buf[4];
  const int t = blockIdx.x;
  const float* row = stream + (size_t)t * H;
  f32x4 v[kMaxChunks];
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int c = 4 * threadIdx.x + kResCols * j;
    if (c < H) {
      v[j] = *reinterpret_cast<const f32x4*>(row + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) ss += (double)v[j][q] * (double)v[j][q];
    }
  }
  const double inv = 1.0 / sqrt(block_sum(ss, buf) / H + eps);
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int c = 4 * threadIdx.x + kResCols * j;
    if (c < H) {
      uint32_t packed[2];
#pragma unroll
      for (int q = 0; q < 4; q += 2) {
        const double g0 = g_in ? (double)g_in[c + q] : 1.0, g1 = g_in ? (double)g_in[c + q + 1] : 1.0;
        const uint16_t lo = f32_to_bf16_rne((float)((double)v[j][q] * inv * g0));
        const uint16_t hi = f32_to_bf16_rne((float)((double)v[j][q + 1] * inv * g1));
        packed[q / 2] = lo | ((uint32_t)hi << 16);
      }
      *reinterpret_cast<uint2*>(x + (size_t)t * H + c) = make_uint2(packed[0], packed[1]);
    }
  }
}

// grid: T; block 256.  y16/yscale/w as for the combine.  stream_out may alias stream_in:
// every element is read and written by the same thread.
__global__ __launch_bounds__(256) void combine_residual_kernel(const uint16_t* __restrict__ y16,
                                                               const uint8_t* __restrict__ yscale,
                                                               const float* __restrict__ w, const float* stream_in,
                                                               const float* __restrict__ g_out, float* stream_out,
                                                               int H, int K, float a, float b, double eps) {
  __shared__ double buf[4];
  const int t = blockIdx.x;
  const size_t row0 = (size_t)t * K;
  const int nsb = H / kScaleCols;
  f32x4 out[kMaxChunks];
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int c = 4 * threadIdx.x + kResCols * j;
    if (c < H) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < K; ++k) {  // ascending k, FP32, as the combine
        const uint2 raw = *reinterpret_cast<const uint2*>(y16 + (row0 + k) * H + c);
        const int s = yscale[(row0 + k) * nsb + c / kScaleCols];
        f32x4 yv;
        yv[0] = __builtin_amdgcn_ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)(raw.x & 0xFFFFu)), s);
        yv[1] = __builtin_amdgcn_ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)(raw.x >> 16)), s);
        yv[2] = __builtin_amdgcn_ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)(raw.y & 0xFFFFu)), s);
        yv[3] = __builtin_amdgcn_ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)(raw.y >> 16)), s);
        acc += w[row0 + k] * yv;
      }
      out[j] = acc;
#pragma unroll
      for (int q = 0; q < 4; ++q) ss += (double)acc[q] * (double)acc[q];
    }
  }
  const float inv = (float)(1.0 / sqrt(block_sum(ss, buf) / H + eps));
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int c = 4 * threadIdx.x + kResCols * j;
    if (c < H) {
      const f32x4 s = *reinterpret_cast<const f32x4*>(stream_in + (size_t)t * H + c);
      f32x4 r;
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = a * s[q] + b * (out[j][q] * inv * (g_out ? g_out[c + q] : 1.f));
      *reinterpret_cast<f32x4*>(stream_out + (size_t)t * H + c) = r;
    }
  }
}

bool residual_fits(int H) { return H <= kResCols * kMaxChunks && H % 4 == 0; }

hipError_t launch_prenorm(const float* stream, const float* g_in, uint16_t* x, int T, int H, float eps,
                          hipStream_t st) {
  hipLaunchKernelGGL(prenorm_kernel, dim3(T), dim3(256), 0, st, stream, g_in, x, H, (double)eps);
  return hipGetLastError();
}

hipError_t launch_combine_residual(const uint16_t* y16, const uint8_t* yscale, const float* w, const float* stream_in,
                                   const float* g_out, float* stream_out, int T, int H, int K, int step, float eps,
                                   hipStream_t st) {
  const float a = (float)sqrt((double)(step - 1) / step), b = (float)(1.0 / sqrt((double)step));
  hipLaunchKernelGGL(combine_residual_kernel, dim3(T), dim3(256), 0, st, y16, yscale, w, stream_in, g_out,
                     stream_out, H, K, a, b, (double)eps);
  return hipGetLastError();
}

}  // namespace beam
