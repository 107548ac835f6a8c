// Device-side helpers shared by the gfx950 kernels of the Beam MoE block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kScaleCols = 64;  // SwiGLU activation columns that share one power-of-two scale

// fp32 -> bf16 bit pattern, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);  // finite inputs only
  return uint16_t(u >> 16);
}

// 16-byte loads: bit-cast helpers between u32x4 and bf16x8 operands.
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// SiLU in FP32: g / (1 + e^-g), with e^-g = 2^(-g log2 e) from the hardware base-2
// exponential and the quotient from the hardware reciprocal (each about 1 ulp);
// large negative g gives e^-g = inf, a zero reciprocal and silu = -0.
__device__ __forceinline__ float silu_f32(float g) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// Eight bf16 values (one 16-byte operand) to eight fp16 values. bf16 has 8
// significant bits and fp16 11, so the conversion is exact for magnitudes in
// fp16's normal range [2^-14, 65504]; smaller magnitudes become fp16
// subnormals rounded toward zero (error below 2^-24).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(v[i] << 16);
    const float hi = __uint_as_float(v[i] & 0xFFFF0000u);
    r[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return r;
}

// acc * 2^d, exact (power-of-two scaling of FP32 values far from its range limits).
__device__ __forceinline__ f32x4 ldexp4(f32x4 v, int d) {
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_ldexpf(v[i], d);
  return r;
}

// Power-of-two scale exponent s >= 0 for a block of SwiGLU activations whose
// largest magnitude is maxabs: maxabs * 2^-s < 2^15, so every value of the
// block fits fp16 (max 65504) after scaling by 2^-s.
// The down projection multiplies the stored h * 2^-s by the unscaled weights
// and keeps its FP32 accumulators in units of 2^s of the block it consumes
// last: moving to a block of exponent s' multiplies them by 2^(s - s'), and
// the output is acc * 2^s at the end.  The weights never carry the scale, so
// no weight range limit comes with large activations.
__device__ __forceinline__ int act_scale_exp(float maxabs) {
  const int e = __builtin_amdgcn_frexp_expf(maxabs);  // maxabs < 2^e
  return e > 15 ? e - 15 : 0;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// s_waitcnt encodings (gfx9): vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = (63 & 15) | (3 << 14) | (7 << 4);

// One 16-byte-per-lane global -> LDS copy by the load unit: lane i's 16 bytes
// from g land at LDS byte lds_base + 16 * i (lds_base wave-uniform, carried in
// M0, which is restored afterwards).  The instruction writes no register and
// counts in vmcnt like a load; callers wait with s_waitcnt and publish with a
// barrier.  Written as inline assembly: the compiler's builtin for it drains
// every outstanding load at each loop head.
__device__ __forceinline__ void lds_copy16(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_base)
      : "memory");
}

// Wave-uniform LDS byte address of p.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// One row tile of the expert kernels (256 rows for the grouped GEMMs, at most
// R for the stream kernels), written by the dispatch: rows [row_start, row_start + rows) of the
// expert-sorted order, all belonging to `expert`.  An expert's consecutive
// tiles are cut into groups of at most kTileGroupMax; each tile carries its
// group's first index and size, which the GEMM block order uses to run a
// group's tiles side by side (they share the expert's weight columns).
constexpr int kTileGroupMax = 8;
struct Tile {
  int32_t expert;
  int32_t row_start;
  int32_t rows;
  int32_t group_first;
  int32_t group_size;
  int32_t pad[3];
};
static_assert(sizeof(Tile) == 32, "tile table entry");

}  // namespace beam
