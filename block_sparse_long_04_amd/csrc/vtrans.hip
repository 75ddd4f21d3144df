// V layout change for the matrix-core attention: V [L][Hkv][d] (bf16, or
// e4m3fn codes) -> V^T [Hkv][d][nb*B] bf16, zero past L.
//
// In P.V the contraction runs over keys, while V arrives with the head
// dimension contiguous.  The bf16 matrix-core operands want 8 consecutive
// contraction elements per lane, so the attention kernel reads V^T rows, each
// a contiguous run of keys.  This is one extra streaming pass over V (read V,
// write V^T); e4m3fn codes are widened to bf16 exactly (scale applied at the
// attention output).  Tiles of 64 tokens x 64 dims pass through LDS.
#include "common.h"

namespace {

template <int ESZ>
__global__ __launch_bounds__(256) void vtrans_kernel(const uint8_t* __restrict__ v, int64_t st_tok,
                                                     int64_t st_head, int L, int d, int Lpad,
                                                     uint16_t* __restrict__ vt) {
  __shared__ uint16_t tile[64][66];  // [token][dim], +2 pad
  const int tt = blockIdx.x;         // 64-token tile
  const int dtile = blockIdx.y;      // 64-dim tile
  const int g = blockIdx.z;          // kv head
  const int tid = threadIdx.x;
  constexpr int VEC = 16 / ESZ;      // elements per 16-byte load
  constexpr int CPR = 64 / VEC;      // chunks per 64-dim token row
  constexpr int NCH = 64 * CPR;      // chunks in the tile
  for (int c = tid; c < NCH; c += 256) {
    const int tr = c / CPR;
    const int cc = c - tr * CPR;
    const int tok = tt * 64 + tr;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (tok < L)
      x = *reinterpret_cast<const uint4*>(v + ((int64_t)tok * st_tok + g * st_head + dtile * 64 + cc * VEC) * ESZ);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (ESZ == 2) {
        tile[tr][cc * VEC + 2 * e] = (uint16_t)(w[e] & 0xffffu);
        tile[tr][cc * VEC + 2 * e + 1] = (uint16_t)(w[e] >> 16);
      } else {
        float f[4];
        fpk::e4m3x4_to_f32(w[e], f);  // every e4m3 value is a bf16 value: truncation is exact
#pragma unroll
        for (int b = 0; b < 4; ++b) tile[tr][cc * VEC + 4 * e + b] = (uint16_t)(__float_as_uint(f[b]) >> 16);
      }
    }
  }
  __syncthreads();
  // write: 64 dims x 8 chunks of 8 tokens
  for (int c = tid; c < 512; c += 256) {
    const int dd = c >> 3;
    const int tc = c & 7;
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)tile[tc * 8 + 2 * e][dd] | ((uint32_t)tile[tc * 8 + 2 * e + 1][dd] << 16);
    uint16_t* dst = vt + ((int64_t)g * d + dtile * 64 + dd) * Lpad + tt * 64 + tc * 8;
    *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t fpk_launch_vtrans(const fp_problem& p, const FpDims& dm, uint16_t* v_t, hipStream_t st) {
  const int Lpad = dm.nb * dm.B;
  dim3 grid((unsigned)(Lpad / 64), (unsigned)(dm.d / 64), (unsigned)dm.Hkv);
  if (p.dtype == FP_BF16)
    hipLaunchKernelGGL(vtrans_kernel<2>, grid, dim3(256), 0, st, static_cast<const uint8_t*>(p.v),
                       p.v_stride_tok, p.v_stride_head, dm.L, dm.d, Lpad, v_t);
  else
    hipLaunchKernelGGL(vtrans_kernel<1>, grid, dim3(256), 0, st, static_cast<const uint8_t*>(p.v),
                       p.v_stride_tok, p.v_stride_head, dm.L, dm.d, Lpad, v_t);
  return hipGetLastError();
}
