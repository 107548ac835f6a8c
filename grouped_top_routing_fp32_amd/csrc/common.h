// Device-side helpers shared by the gfx950 kernels of the Beam MoE block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 <-> fp32 on raw bit patterns.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);  // finite inputs only
  return uint16_t(u >> 16);
}

// 16-byte loads: bit-cast helpers between u32x4 and bf16x8 operands.
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ u32x4 ldg16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// One tile of a grouped GEMM: rows [row_start, row_start + rows) of the
// expert-sorted order, all belonging to `expert`.
struct Tile {
  int32_t expert;
  int32_t row_start;
  int32_t rows;
  int32_t pad;
};

}  // namespace beam
