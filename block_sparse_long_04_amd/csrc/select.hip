// Steps 2-4: proxy block scores, single-pass max threshold, and compaction of
// the kept key blocks into ascending per-row lists.
//
// FlashPrefill skill page: "Core Concept" items 2-3 (block-pair importance
// from the pooled proxies; a single max reduction sets the pruning threshold,
// no sort and no cumulative sum) and "Architecture Overview" (the score
// matrix is never materialised; kept indices drive index jumping).  The
// threshold rule: keep (i, j), j <= i, iff S_ij - m_i >= ln(tau), i.e. the
// block's softmax weight is at least tau times the row's largest; the
// diagonal block is always kept.
//
// One workgroup (4 waves) owns 16 consecutive query-block rows of one q head.
// Scores are 16x16 tiles from the fp32 matrix cores (v_mfma_f32_16x16x4f32):
// A = 16 pooled query rows, B = 16 pooled key rows, all of the head dimension.
// Pass 1 takes the row maxima (waves stride over key tiles, meet in LDS);
// pass 2 recomputes the identical tiles (same instruction order, so the same
// bits) and turns the comparison into 16-bit keep masks per (row, key tile)
// held in LDS; pass 3 compacts each row's mask with popcount + a wave-wide
// exclusive scan and writes the ascending list.  Only kept entries reach HBM.
#include "common.h"

namespace {

using fpk::floatx4;

template <int D>
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ qp,
                                                     const float* __restrict__ kp, int Hq, int Hkv,
                                                     int nb, float scale, float ln_tau, int dense,
                                                     float* __restrict__ row_max,
                                                     int* __restrict__ counts,
                                                     int* __restrict__ indices) {
  extern __shared__ uint16_t kmask[];  // [16 rows][ntiles]
  __shared__ float red[4][16];

  const int ntiles = (nb + 15) >> 4;
  const int rt = ntiles - 1 - (int)(blockIdx.x / Hq);  // longest rows first
  const int h = blockIdx.x % Hq;
  const int g = h / (Hq / Hkv);
  const int i0 = rt * 16;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int grp = lane >> 4;

  // A operand: lane supplies Qbar[i0 + c16][16t + 4grp + c] in MFMA step (t, c).
  floatx4 qa[D / 16];
  {
    const int qrow = min(i0 + c16, nb - 1);
    const float* qptr = qp + ((int64_t)h * nb + qrow) * D + 4 * grp;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qa[t] = *reinterpret_cast<const floatx4*>(qptr + 16 * t);
  }
  const float* kbase = kp + (int64_t)g * nb * D + 4 * grp;

  // D layout: lane holds S[i0 + 4grp + r][16jt + c16], r = 0..3.
  auto tile = [&](int jt) -> floatx4 {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    const int krow = min(jt * 16 + c16, nb - 1);
    const float* kptr = kbase + (int64_t)krow * D;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const floatx4 kb = *reinterpret_cast<const floatx4*>(kptr + 16 * t);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[t][0], kb[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[t][1], kb[1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[t][2], kb[2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[t][3], kb[3], acc, 0, 0, 0);
    }
    return acc;
  };

  // ---- pass 1: row maxima over j <= i
  float mr[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int jt = w; jt <= rt; jt += 4) {
    const floatx4 acc = tile(jt);
    const int j = jt * 16 + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 4 * grp + r;
      const float s = acc[r] * scale;
      if (j <= i && i < nb) mr[r] = fmaxf(mr[r], s);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) mr[r] = fmaxf(mr[r], __shfl_xor(mr[r], off));
  }
  if (c16 == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[w][4 * grp + r] = mr[r];
  }
  __syncthreads();
  float m[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * grp + r;
    m[r] = fmaxf(fmaxf(red[0][row], red[1][row]), fmaxf(red[2][row], red[3][row]));
  }
  if (w == 0 && c16 == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 4 * grp + r;
      if (i < nb) row_max[(int64_t)h * nb + i] = m[r];
    }
  }

  // ---- pass 2: keep masks per (row, key tile)
  for (int jt = w; jt <= rt; jt += 4) {
    uint64_t bits[4];
    const int j = jt * 16 + c16;
    if (dense) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * grp + r;
        bits[r] = __ballot(j <= i && i < nb);
      }
    } else {
      const floatx4 acc = tile(jt);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * grp + r;
        const float s = acc[r] * scale;
        const bool keep = (j <= i && i < nb) && ((s - m[r] >= ln_tau) || j == i);
        bits[r] = __ballot(keep);
      }
    }
    if (lane < 16) {
      const int rr = lane & 3;
      const uint64_t b = rr == 0 ? bits[0] : rr == 1 ? bits[1] : rr == 2 ? bits[2] : bits[3];
      kmask[lane * ntiles + jt] = (uint16_t)((b >> (16 * (lane >> 2))) & 0xffffu);
    }
  }
  __syncthreads();

  // ---- pass 3: compaction, wave w owns rows 4w .. 4w+3
  for (int rr = 0; rr < 4; ++rr) {
    const int row = 4 * w + rr;
    const int i = i0 + row;
    if (i >= nb) break;
    const int nwords = (i + 64) >> 6;  // 64-column words covering j = 0..i
    int* out = indices + fpk::tri_offset(h, i, nb);
    int base = 0;
    for (int wd0 = 0; wd0 < nwords; wd0 += 64) {
      const int wd = wd0 + lane;
      uint64_t bw = 0;
      if (wd < nwords) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = 4 * wd + q;
          if (t <= rt) bw |= (uint64_t)kmask[row * ntiles + t] << (16 * q);
        }
      }
      const int cnt = __popcll(bw);
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const int total = __shfl(incl, 63);
      int pos = base + incl - cnt;
      while (bw) {
        const int b = __builtin_ctzll(bw);
        out[pos++] = 64 * wd + b;
        bw &= bw - 1;
      }
      base += total;
    }
    if (lane == 0) counts[(int64_t)h * nb + i] = base;
  }
}

}  // namespace

hipError_t fpk_launch_select(const FpDims& dm, const float* q_pool, const float* k_pool,
                             float sm_scale, float ln_tau, float* row_max, int* counts,
                             int* indices, hipStream_t st) {
  const int ntiles = (dm.nb + 15) / 16;
  const size_t lds = ((size_t)16 * ntiles * sizeof(uint16_t) + 3) & ~(size_t)3;
  const int dense = ln_tau == -INFINITY ? 1 : 0;
  dim3 grid((unsigned)(ntiles * dm.Hq));
  if (dm.d == 128)
    hipLaunchKernelGGL(select_kernel<128>, grid, dim3(256), lds, st, q_pool, k_pool, dm.Hq, dm.Hkv,
                       dm.nb, sm_scale, ln_tau, dense, row_max, counts, indices);
  else
    hipLaunchKernelGGL(select_kernel<64>, grid, dim3(256), lds, st, q_pool, k_pool, dm.Hq, dm.Hkv,
                       dm.nb, sm_scale, ln_tau, dense, row_max, counts, indices);
  return hipGetLastError();
}
