// Query-probe variant of stage 1: the pooled probe of each query block scored
// against every key token, reduced per key block by the max, then the same
// single-pass max threshold and lists as the main selection.
//
// FlashPrefill skill page, "Core Concept" (uniformly distributed query probes;
// the search cost O(L^2/B) against O((L/B)^2)): this is the O(L^2/B) reading,
// S'[h,i,j] = max over tokens t of block j of (Qbar[h,i] . k[t]) * sm_scale,
// which sees a single key token aligned with the probe that the pooled mean
// dilutes by 1/B.
//
// One workgroup (4 waves) owns 32 query-block rows of one q head (heaviest
// first).  Waves stride over key blocks; a key block is four groups of 32
// tokens, each a 32 x 32 tile S^T = K Qbar^T on v_mfma_f32_32x32x16_bf16 (the
// lane is the query-block row, as in the attention kernel).  Qbar is fp32: it
// enters as three bf16 parts (hi, mid, lo: 24 bits in all) against the exact
// bf16 (or widened e4m3) key tokens, so the products keep fp32 precision.  A
// lane's 16 token scores and its partner half-wave's give the group max; the
// block's max goes to LDS.  Then each row: max over j <= i, keep S' - m >=
// ln tau or the diagonal, and compaction.  Rows of scores live in LDS: 32 x
// nb floats, so this variant takes nb <= 1024.
#include "common.h"

namespace {

using fpk::bf16x8;
using fpk::floatx16;

__device__ __forceinline__ uint16_t bf16_hi(float f) { return (uint16_t)(__float_as_uint(f) >> 16); }

// three bf16 parts whose sum is x to 24 bits: hi = x truncated to bf16, then
// the truncated remainders
__device__ __forceinline__ void split3(float x, uint16_t& a, uint16_t& b, uint16_t& c) {
  a = bf16_hi(x);
  const float r1 = x - __uint_as_float((uint32_t)a << 16);
  b = bf16_hi(r1);
  const float r2 = r1 - __uint_as_float((uint32_t)b << 16);
  c = bf16_hi(r2);
}

template <bool kFp8>
__device__ __forceinline__ bf16x8 load_k8(const uint8_t* p) {
  if constexpr (!kFp8) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    float f[8];
    fpk::e4m3x4_to_f32(w.x, f);
    fpk::e4m3x4_to_f32(w.y, f + 4);
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)  // every e4m3 value is a bf16 value: truncation is exact
      o[e] = (__float_as_uint(f[2 * e]) >> 16) | (__float_as_uint(f[2 * e + 1]) & 0xffff0000u);
    return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
  }
}

template <bool kFp8>
__global__ __launch_bounds__(256) void probe_select_kernel(const float* __restrict__ qp, const uint8_t* __restrict__ k,
                                                           int64_t k_st, int64_t k_sh, int L, int Hq, int Hkv,
                                                           int nb, float scale, float ln_tau,
                                                           float* __restrict__ row_max, int* __restrict__ counts,
                                                           int* __restrict__ indices) {
  extern __shared__ float srow[];  // [32][nb]
  constexpr int kEsz = kFp8 ? 1 : 2;
  const int ntile = (nb + 31) >> 5;
  const int rt = ntile - 1 - (int)(blockIdx.x / Hq);
  const int h = (int)(blockIdx.x % Hq);
  const int g = h / (Hq / Hkv);
  const int i0 = rt * 32;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 31;  // query-block row of the tile
  const int hh = lane >> 5;
  const int last = min(i0 + 31, nb - 1);

  // B operands: Qbar row i0 + n, elements 16 s + 8 hh .. + 7, in three parts
  bf16x8 qs[3][8];
  {
    const float* q = qp + ((int64_t)h * nb + min(i0 + n, nb - 1)) * 128 + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint16_t a[8], b[8], c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split3(q[16 * s + e], a[e], b[e], c[e]);
      uint32_t pa[4], pb[4], pc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pa[e] = a[2 * e] | ((uint32_t)a[2 * e + 1] << 16);
        pb[e] = b[2 * e] | ((uint32_t)b[2 * e + 1] << 16);
        pc[e] = c[2 * e] | ((uint32_t)c[2 * e + 1] << 16);
      }
      qs[0][s] = __builtin_bit_cast(bf16x8, make_uint4(pa[0], pa[1], pa[2], pa[3]));
      qs[1][s] = __builtin_bit_cast(bf16x8, make_uint4(pb[0], pb[1], pb[2], pb[3]));
      qs[2][s] = __builtin_bit_cast(bf16x8, make_uint4(pc[0], pc[1], pc[2], pc[3]));
    }
  }
  const uint8_t* kg = k + ((int64_t)g * k_sh + 8 * hh) * kEsz;

  // ---- scores: S'[row][j] for every key block j <= last.  A wave's work is
  // the sequence u = 0, 1, ... of (key block w + 4 (u / 4), token group u % 4);
  // the next group's tokens load while the current group multiplies (two
  // register sets; the address of a group past the end is clamped, its load
  // is unused).
  const int nj = w <= last ? (last - w) / 4 + 1 : 0;
  const int items = 4 * nj;
  auto kload = [&](int u, bf16x8 (&dst)[8]) {
    const int t = (w + 4 * (u >> 2)) * 128 + 32 * (u & 3) + n;  // this lane's token (A row)
    const uint8_t* kr = kg + (int64_t)min(t, L - 1) * k_st * kEsz;
#pragma unroll
    for (int s = 0; s < 8; ++s) dst[s] = load_k8<kFp8>(kr + 16 * s * kEsz);
  };
  float bmax = -INFINITY;
  auto group = [&](int u, const bf16x8 (&ka)[8]) {
    floatx16 acc = {0};
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int p = 0; p < 3; ++p) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qs[p][s], acc, 0, 0, 0);
    // lane holds S^T[token m][row n], m = 8 (r / 4) + 4 hh + r % 4
    const int j = w + 4 * (u >> 2);
    const int tbase = j * 128 + 32 * (u & 3) + 4 * hh;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (tbase + 8 * (r >> 2) + (r & 3) < L) bmax = fmaxf(bmax, acc[r]);
    if ((u & 3) == 3) {  // block done: join the half-waves, store, reset
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
      const float bm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      if (hh == 0) srow[n * nb + j] = bm * scale;
      bmax = -INFINITY;
    }
  };
  if (items > 0) {
    bf16x8 ka[8], kb[8];
    kload(0, ka);
    for (int u = 0; u < items; u += 2) {  // items is a multiple of 4
      kload(u + 1, kb);
      group(u, ka);
      kload(min(u + 2, items - 1), ka);
      group(u + 1, kb);
    }
  }
  __syncthreads();

  // ---- per row: max over j <= i, threshold, diagonal, compaction
  for (int row = w; row < 32; row += 4) {
    const int i = i0 + row;
    if (i > last) break;
    const float* sr = srow + row * nb;
    float m = -INFINITY;
    for (int j = lane; j <= i; j += 64) m = fmaxf(m, sr[j]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    int* out = indices + fpk::tri_offset(h, i, nb);
    int base = 0;
    for (int j0 = 0; j0 <= i; j0 += 64) {
      const int j = j0 + lane;
      const bool keep = j <= i && ((sr[j] - m >= ln_tau) || j == i);
      const uint64_t bits = __ballot(keep);
      if (keep)
        out[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0))] = j;
      base += __popcll(bits);
    }
    if (lane == 0) {
      row_max[(int64_t)h * nb + i] = m;
      counts[(int64_t)h * nb + i] = base;
    }
  }
}

}  // namespace

hipError_t fpk_launch_probe_select(const fp_problem& p, const FpDims& dm, const float* q_pool, float sm_scale,
                                   float ln_tau, float* row_max, int* counts, int* indices, hipStream_t st) {
  const bool fp8 = p.dtype == FP_FP8_E4M3;
  const size_t lds = (size_t)32 * dm.nb * sizeof(float);
  const dim3 grid((unsigned)(((dm.nb + 31) / 32) * dm.Hq));
  const float scale = sm_scale * (fp8 ? p.k_scale : 1.0f);
  auto launch = [&](auto kern) -> hipError_t {
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, q_pool, static_cast<const uint8_t*>(p.k), p.k_stride_tok,
                       p.k_stride_head, dm.L, dm.Hq, dm.Hkv, dm.nb, scale, ln_tau, row_max, counts, indices);
    return hipGetLastError();
  };
  return fp8 ? launch(probe_select_kernel<true>) : launch(probe_select_kernel<false>);
}
