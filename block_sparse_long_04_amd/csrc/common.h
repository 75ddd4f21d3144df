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

// OCP e4m3fn codes -> fp32 (exact: bias 7, exponent 0 subnormal, S.1111.111
// NaN, no infinities).  On gfx950 the fp8 conversion instructions read the
// OCP format; one v_cvt_pk_f32_fp8 widens the two codes of a 16-bit half.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* f) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)(c & 0xffu), 0);
}

// S - m of the threshold rule with the score S = acc * scale rounded to fp32
// first.  Contracting the two into one fused multiply-add would compare the
// exact product against a row max taken from rounded products, so a block
// whose score equals the row max could fall below it (FlashPrefill skill
// page, "Core Concept" item 3: exp(S - m) >= tau with m the largest S).
__device__ __forceinline__ float score_minus_max(float acc, float scale, float m) {
#pragma clang fp contract(off)
  const float s = acc * scale;
  return s - m;
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

hipError_t fpk_launch_select_sorted(const FpDims& dm, const float* q_pool, const float* k_pool,
                                    float sm_scale, int rule, float param, float* row_max,
                                    int* counts, int* indices, hipStream_t st);

hipError_t fpk_launch_probe_select(const fp_problem& p, const FpDims& dm, const float* q_pool, float sm_scale,
                                   float ln_tau, float* row_max, int* counts, int* indices, hipStream_t st);

hipError_t fpk_launch_vtrans(const fp_problem& p, const FpDims& dm, uint16_t* v_t, hipStream_t st);

hipError_t fpk_launch_attn_mfma(const fp_problem& p, const FpDims& dm, const int* counts,
                                const int* indices, const uint16_t* v_t, float sm_scale,
                                hipStream_t st);

// Two query heads of one kv group per wave (bf16, d = B = 128, Hq/Hkv even).
hipError_t fpk_launch_attn_pack(const fp_problem& p, const FpDims& dm, const int* counts, const int* indices,
                                const uint16_t* v_t, float sm_scale, hipStream_t st);

// bf16 layers with head_dim or block_size 64 on the matrix cores.
hipError_t fpk_launch_attn_small(const fp_problem& p, const FpDims& dm, const int* counts, const int* indices,
                                 const uint16_t* v_t, float sm_scale, hipStream_t st);

hipError_t fpk_launch_attn_generic(const fp_problem& p, const FpDims& dm, const int* counts,
                                   const int* indices, float sm_scale, hipStream_t st);
