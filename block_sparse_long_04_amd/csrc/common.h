// Shared device helpers and launcher declarations of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/flashprefill.h"

namespace fpk {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int intx8 __attribute__((ext_vector_type(8)));

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// OCP e4m3fn code -> fp32 (exact).  bias 7; exponent 0 is subnormal
// (m * 2^-9); S.1111.111 is NaN; there are no infinities.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xfu;
  uint32_t m = c & 0x7u;
  if (e == 0) {
    float v = (float)m * 0.001953125f;  // 2^-9
    return s ? -v : v;
  }
  if (e == 15 && m == 7) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

// e4m3fn code -> bf16 bits (exact: every e4m3 value is a bf16 value)
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t c) {
  return __float_as_uint(e4m3_to_f32(c)) >> 16;
}

__host__ __device__ __forceinline__ int64_t tri_offset(int64_t h, int64_t i, int64_t nb) {
  return h * (nb * (nb + 1) / 2) + i * (i + 1) / 2;
}

}  // namespace fpk

// ---------------------------------------------------------------------------
// Launchers (host side, C++ linkage, internal to the library).  Each returns
// the hipError_t of its launch.
// ---------------------------------------------------------------------------
struct FpDims {
  int L, Hq, Hkv, d, B, nb;
};

hipError_t fpk_launch_pool(const fp_problem& p, const FpDims& dm, float* q_pool, float* k_pool,
                           hipStream_t st);

hipError_t fpk_launch_select(const FpDims& dm, const float* q_pool, const float* k_pool,
                             float sm_scale, float ln_tau, float* row_max, int* counts,
                             int* indices, hipStream_t st);

hipError_t fpk_launch_vtrans(const fp_problem& p, const FpDims& dm, uint16_t* v_t, hipStream_t st);

hipError_t fpk_launch_attn_mfma(const fp_problem& p, const FpDims& dm, const int* counts,
                                const int* indices, const uint16_t* v_t, float sm_scale,
                                hipStream_t st);

hipError_t fpk_launch_attn_generic(const fp_problem& p, const FpDims& dm, const int* counts,
                                   const int* indices, float sm_scale, hipStream_t st);
