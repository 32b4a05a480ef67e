// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float32 -> bfloat16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Monotone map of a float32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_inv(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// One max step: v = max(v, v of the lane DPP control CTRL selects); lanes
// without a source (or outside ROW_MASK) keep their own value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_step32(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xf, false);
  return o > v ? o : v;
}

// Maximum over the 64 lanes, returned to every lane.  DPP row shifts by
// 1, 2, 4, 8 leave each 16-lane row's maximum in its lane 15; row broadcasts
// of lane 15 and lane 31 then carry it to lane 63, which is read out.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step32<0x111, 0xf>(v);  // row_shr:1
  v = dpp_max_step32<0x112, 0xf>(v);  // row_shr:2
  v = dpp_max_step32<0x114, 0xf>(v);  // row_shr:4
  v = dpp_max_step32<0x118, 0xf>(v);  // row_shr:8
  v = dpp_max_step32<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step32<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// D(16x16) += A(16x32) * B(32x16); lane l supplies A row l%16 / B column l%16,
// eight consecutive k per lane (same k order for A and B).
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// D(32x32) += A(32x16) * B(16x32); lane l supplies A row l%32 / B column l%32.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Logistic sigmoid 1 / (1 + e^-z) with the library exponential.
__device__ __forceinline__ float sigmoid_f32(float z) { return 1.0f / (1.0f + expf(-z)); }

// SiLU(g) * u with the hardware exponential and reciprocal (v_exp_f32,
// v_rcp_f32: ~1 ulp each; the result is rounded to bf16 or compared at fp32
// tolerance, far above that).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

}  // namespace moe
