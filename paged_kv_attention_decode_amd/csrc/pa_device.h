// Device helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockTokens = 16;
constexpr float kNegInf = -__builtin_inff();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));   // MFMA bf16 operands (16x16x32)
typedef short short4_t __attribute__((ext_vector_type(4)));    // MFMA bf16 operands (16x16x16)
typedef float floatx4_t __attribute__((ext_vector_type(4)));   // MFMA 16x16 accumulators
typedef float float2_t __attribute__((ext_vector_type(2)));

// buffer descriptor word 3 on gfx950: raw 32-bit access, no swizzle
constexpr int kBufferWord3 = 0x00020000;

// (lo, hi) rounded to bf16 (round to nearest even), as one packed dword (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){lo, hi}, bf16x2_t));
}

// bf16 halves of a packed dword, widened exactly to fp32
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// a.x*b.x + a.y*b.y + c on packed bf16 pairs, fp32 accumulate (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// fp32 -> bf16 by round-to-nearest-even; NaN stays a quiet NaN
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- cross-lane moves (DPP within a row of 16 lanes) ----------------------
// quad_perm:[1,0,3,2] = 0xB1, quad_perm:[2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// sum over the 4 lanes of a quad; every lane of the quad gets the same bits
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  return x;
}

// reduction over the 16 lanes of a row; every lane of the row gets the same bits
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return x;
}

__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  x = fmaxf(x, dpp_mov<0x141>(x));
  x = fmaxf(x, dpp_mov<0x140>(x));
  return x;
}

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// wave-uniform results (fixed combination order: rows 0+1, 2+3, then the pairs)
__device__ __forceinline__ float wave_max(float x) {
  x = row_max(x);
  return fmaxf(fmaxf(lane_value(x, 0), lane_value(x, 16)), fmaxf(lane_value(x, 32), lane_value(x, 48)));
}

__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum(x);
  return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  const int lane = threadIdx.x & 63;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}

// order LDS traffic among the lanes of one wave
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pa
