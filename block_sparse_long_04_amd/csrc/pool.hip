// Step 1: mean-pool Q and K into one fp32 proxy per block of B tokens.
//
// FlashPrefill skill page, "Architecture Overview" (block-level proxies from
// average-pooled queries and keys) and the Stage 1 code of "Implementation
// Steps": nb = ceil(L/B) blocks, block b covers tokens [bB, min((b+1)B, L)),
// the proxy is the mean over the tokens present.
//
// This stage is a pure HBM stream (each Q/K byte read once, 1/B as much
// written).  A workgroup owns one token block and 64 consecutive 16-byte
// column chunks of the [token][head*dim] row; its four waves each sum a
// quarter of the block's tokens (every load instruction of a wave reads 1 KiB
// of one contiguous token row), and the four partial sums meet in LDS.
#include "common.h"

namespace {

struct PoolSrc {
  const uint8_t* base;  // tensor base (bytes)
  int64_t st_tok;       // element strides
  int64_t st_head;
  float* out;           // [H][nb][d]
  int chunks;           // H*d / VEC 16-byte chunks per token
  float scale;          // dequantisation scale (1 for f32/bf16)
};

template <int ESZ>
__device__ __forceinline__ void accum(float* acc, const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (ESZ == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
  } else if constexpr (ESZ == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += fpk::bf16_bits_to_f32(w[e] & 0xffffu);
      acc[2 * e + 1] += fpk::bf16_bits_to_f32(w[e] >> 16);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float f[4];
      fpk::e4m3x4_to_f32(w[e], f);
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[4 * e + b] += f[b];
    }
  }
}

template <int ESZ>
__global__ __launch_bounds__(256) void pool_kernel(PoolSrc qs, PoolSrc ks, int L, int d, int B,
                                                   int nb, int wgq, int wgk) {
  constexpr int VEC = 16 / ESZ;
  __shared__ float red[3][64 * VEC];

  const int per_block = wgq + wgk;
  const int b = blockIdx.x / per_block;
  const int r = blockIdx.x - b * per_block;
  const bool isq = r < wgq;
  const PoolSrc src = isq ? qs : ks;
  const int cgrp = isq ? r : r - wgq;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int chunk = cgrp * 64 + lane;
  const bool active = chunk < src.chunks;
  const int elem = chunk * VEC;
  const int head = active ? elem / d : 0;
  const int col = active ? elem - head * d : 0;

  const int t0 = b * B;
  const int n = min(B, L - t0);
  const int q4 = (B + 3) / 4;
  const int tb = min(n, w * q4);
  const int te = min(n, tb + q4);

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  if (active) {
    const uint8_t* p = src.base + ((int64_t)(t0 + tb) * src.st_tok + head * src.st_head + col) * ESZ;
    const int64_t step = src.st_tok * ESZ;
    int t = tb;
    for (; t + 8 <= te; t += 8) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const uint4*>(p + u * step);
#pragma unroll
      for (int u = 0; u < 8; ++u) accum<ESZ>(acc, v[u]);
      p += 8 * step;
    }
    for (; t < te; ++t) {
      uint4 v = *reinterpret_cast<const uint4*>(p);
      accum<ESZ>(acc, v);
      p += step;
    }
  }

  if (w > 0) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[w - 1][e * 64 + lane] = acc[e];
  }
  __syncthreads();
  if (w == 0 && active) {
    float res[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float s = acc[e] + red[0][e * 64 + lane];
      s += red[1][e * 64 + lane];
      s += red[2][e * 64 + lane];
      res[e] = (s / (float)n) * src.scale;
    }
    float4* o = reinterpret_cast<float4*>(src.out + ((int64_t)head * nb + b) * d + col);
#pragma unroll
    for (int e = 0; e < VEC / 4; ++e)
      o[e] = make_float4(res[4 * e], res[4 * e + 1], res[4 * e + 2], res[4 * e + 3]);
  }
}

}  // namespace

hipError_t fpk_launch_pool(const fp_problem& p, const FpDims& dm, float* q_pool, float* k_pool,
                           hipStream_t st) {
  const int esz = p.dtype == FP_F32 ? 4 : (p.dtype == FP_BF16 ? 2 : 1);
  const int vec = 16 / esz;
  const bool fp8 = p.dtype == FP_FP8_E4M3;
  PoolSrc qs{static_cast<const uint8_t*>(p.q), p.q_stride_tok, p.q_stride_head, q_pool,
             dm.Hq * dm.d / vec, fp8 ? p.q_scale : 1.0f};
  PoolSrc ks{static_cast<const uint8_t*>(p.k), p.k_stride_tok, p.k_stride_head, k_pool,
             dm.Hkv * dm.d / vec, fp8 ? p.k_scale : 1.0f};
  const int wgq = (qs.chunks + 63) / 64;
  const int wgk = (ks.chunks + 63) / 64;
  dim3 grid((unsigned)(dm.nb * (wgq + wgk)));
  if (esz == 4)
    hipLaunchKernelGGL(pool_kernel<4>, grid, dim3(256), 0, st, qs, ks, dm.L, dm.d, dm.B, dm.nb, wgq, wgk);
  else if (esz == 2)
    hipLaunchKernelGGL(pool_kernel<2>, grid, dim3(256), 0, st, qs, ks, dm.L, dm.d, dm.B, dm.nb, wgq, wgk);
  else
    hipLaunchKernelGGL(pool_kernel<1>, grid, dim3(256), 0, st, qs, ks, dm.L, dm.d, dm.B, dm.nb, wgq, wgk);
  return hipGetLastError();
}
