// Batches of independent sequences (varlen), with K/V packed like Q or held
// in a cache of block_size-token pages addressed through a block table.
//
// FlashPrefill V2 abstract: the method is deployed for serving (many prompts
// of different lengths prefilled together, K/V in a paged cache).  Each
// sequence is its own causal prefill; only where tokens and pages live
// changes.  The batch's blocks are numbered globally: sequence s owns blocks
// first[s] .. first[s] + nb[s] - 1 (nb[s] = ceil(len[s] / B)).
//
// The kernels here prepare the batch for the same selection and attention
// arithmetic as a single sequence:
//   * varlen_meta_kernel: per block (sequence, block in sequence, first token
//     in q/out, rows), per sequence (first block, blocks, index base), from
//     the device copy of cu_seqlens;
//   * pool_varlen_kernel: the pooled proxies per block, and K gathered per kv
//     head into [Hkv][NB*B][d] (rows past a sequence's end are zero), so the
//     attention reads K tiles at block * B without page indirection;
//   * vtrans_varlen_kernel: V^T [Hkv][d][NB*B] from packed or paged V;
//   * select_varlen_kernel: scores, the single-pass max threshold and the
//     lists of one tile of 16 block rows, whose rows may belong to different
//     sequences: each row sees only its own sequence's blocks, and its list
//     holds block indices local to the sequence.
// Page ids outside [0, num_pages) read as zero pages.
#include "common.h"
#include "varlen.h"

namespace {

using fpk::floatx4;

__global__ __launch_bounds__(256) void varlen_meta_kernel(const int* __restrict__ cu, int S, int B, int Hq,
                                                          int NB, fpk::VlBlock* __restrict__ blk,
                                                          fpk::VlSeq* __restrict__ seq) {
  __shared__ int s_nb[256];
  __shared__ long long s_tri[256];
  __shared__ int carry_nb;
  __shared__ long long carry_tri;
  const int tid = threadIdx.x;
  if (tid == 0) {
    carry_nb = 0;
    carry_tri = 0;
  }
  __syncthreads();
  // sequences in chunks of 256: block counts and index bases by a block-wide scan
  for (int c0 = 0; c0 < S; c0 += 256) {
    const int s = c0 + tid;
    int nbs = 0;
    if (s < S) nbs = (cu[s + 1] - cu[s] + B - 1) / B;
    s_nb[tid] = nbs;
    s_tri[tid] = (long long)Hq * nbs * (nbs + 1) / 2;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int a = tid >= off ? s_nb[tid - off] : 0;
      const long long b = tid >= off ? s_tri[tid - off] : 0;
      __syncthreads();
      s_nb[tid] += a;
      s_tri[tid] += b;
      __syncthreads();
    }
    if (s < S) {
      seq[s].first = carry_nb + s_nb[tid] - nbs;
      seq[s].nb = nbs;
      seq[s].idx_base = carry_tri + s_tri[tid] - (long long)Hq * nbs * (nbs + 1) / 2;
    }
    __syncthreads();
    if (tid == 255) {
      carry_nb += s_nb[255];
      carry_tri += s_tri[255];
    }
    __syncthreads();
  }
  __threadfence_block();
  __syncthreads();
  // blocks: find the sequence by binary search over the first blocks
  for (int b = tid; b < NB; b += 256) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seq[mid].first <= b) lo = mid;
      else hi = mid - 1;
    }
    // (an empty sequence shares its first block with the next one; the
    // search returns the last sequence starting at or before b, which owns it)
    const int jl = b - seq[lo].first;
    const int tok0 = cu[lo] + jl * B;
    blk[b] = fpk::VlBlock{lo, jl, tok0, min(B, cu[lo + 1] - tok0)};
  }
}

struct VlSrc {
  const uint8_t* base;        // packed tensor, or the page cache
  int64_t st_tok, st_head;    // element strides (inside a page for the cache)
  int64_t page_stride;        // elements between pages (paged only)
  const int* table;           // block table [S][max_blocks] or null (packed)
  int max_blocks, num_pages;
};

// Byte offset of row r (< rows) of block b's token rows, head `head`, or -1
// for a page id outside the cache.
template <int ESZ>
__device__ __forceinline__ int64_t row_off(const VlSrc& src, const fpk::VlBlock& m, int r, int head) {
  if (src.table == nullptr) return ((int64_t)(m.tok0 + r) * src.st_tok + (int64_t)head * src.st_head) * ESZ;
  const int pg = src.table[(int64_t)m.seq * src.max_blocks + m.jl];
  if (pg < 0 || pg >= src.num_pages) return -1;
  return ((int64_t)pg * src.page_stride + (int64_t)r * src.st_tok + (int64_t)head * src.st_head) * ESZ;
}

template <int ESZ>
__device__ __forceinline__ void accum(float* acc, const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (ESZ == 2) {
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

// One workgroup per (block, 64 column chunks of the concatenated Q heads or K
// heads), as the single-sequence pooling; the K workgroups also write the
// rows they read to the gathered K, and zeros for the rows past the end.
template <int ESZ>
__global__ __launch_bounds__(256) void pool_varlen_kernel(VlSrc qs, VlSrc ks, const fpk::VlBlock* __restrict__ blk,
                                                          float* __restrict__ q_pool, float* __restrict__ k_pool,
                                                          uint8_t* __restrict__ k_c, int Hq, int Hkv, int d,
                                                          int B, int NB, float q_scale, float k_scale, int wgq,
                                                          int wgk) {
  constexpr int VEC = 16 / ESZ;
  __shared__ float red[3][64 * VEC];
  const int per_block = wgq + wgk;
  const int b = blockIdx.x / per_block;
  const int r = blockIdx.x - b * per_block;
  const bool isq = r < wgq;
  const VlSrc src = isq ? qs : ks;
  const int chunks = (isq ? Hq : Hkv) * d / VEC;
  const int cgrp = isq ? r : r - wgq;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int chunk = cgrp * 64 + lane;
  const bool active = chunk < chunks;
  const int elem = chunk * VEC;
  const int head = active ? elem / d : 0;
  const int col = active ? elem - head * d : 0;
  const fpk::VlBlock m = blk[b];
  const int n = m.rows;
  const int q4 = (B + 3) / 4;
  const int rb = w * q4, re = min(B, rb + q4);  // this wave's rows of the block
  int64_t o0 = active ? row_off<ESZ>(src, m, 0, head) : -1;
  if (o0 >= 0) o0 += (int64_t)col * ESZ;
  const int64_t step = src.st_tok * ESZ;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  uint8_t* kout = (!isq && active) ? k_c + (((int64_t)head * NB * B + (int64_t)b * B) * d + col) * ESZ : nullptr;
#pragma unroll 8
  for (int t = rb; t < re; ++t) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < n && o0 >= 0) v = *reinterpret_cast<const uint4*>(src.base + o0 + (int64_t)t * step);
    if (t < n) accum<ESZ>(acc, v);
    if (kout) *reinterpret_cast<uint4*>(kout + (int64_t)t * d * ESZ) = v;
  }
  if (w > 0) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[w - 1][e * 64 + lane] = acc[e];
  }
  __syncthreads();
  if (w == 0 && active) {
    const float sc = isq ? q_scale : k_scale;
    float res[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float s = acc[e] + red[0][e * 64 + lane];
      s += red[1][e * 64 + lane];
      s += red[2][e * 64 + lane];
      res[e] = (s / (float)n) * sc;
    }
    float* outp = (isq ? q_pool : k_pool) + ((int64_t)head * NB + b) * d + col;
#pragma unroll
    for (int e = 0; e < VEC / 4; ++e)
      reinterpret_cast<float4*>(outp)[e] = make_float4(res[4 * e], res[4 * e + 1], res[4 * e + 2], res[4 * e + 3]);
  }
}

// V^T [Hkv][d][NB*B] bf16 from packed or paged V; tiles of 64 tokens x 64
// dims through LDS, zero past each sequence's end.
template <int ESZ>
__global__ __launch_bounds__(256) void vtrans_varlen_kernel(VlSrc vs, const fpk::VlBlock* __restrict__ blk, int d,
                                                            int B, int Lpad, uint16_t* __restrict__ vt) {
  __shared__ uint16_t tile[64][66];
  const int tt = blockIdx.x, dtile = blockIdx.y, g = blockIdx.z;
  const int b = (tt * 64) / B;
  const int r0 = tt * 64 - b * B;
  const fpk::VlBlock m = blk[b];
  const int tid = threadIdx.x;
  constexpr int VEC = 16 / ESZ;
  constexpr int CPR = 64 / VEC;
  const int64_t o0 = row_off<ESZ>(vs, m, 0, g);
  for (int c = tid; c < 64 * CPR; c += 256) {
    const int tr = c / CPR, cc = c - tr * CPR;
    const int r = r0 + tr;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (r < m.rows && o0 >= 0)
      x = *reinterpret_cast<const uint4*>(vs.base + o0 + ((int64_t)r * vs.st_tok + dtile * 64 + cc * VEC) * ESZ);
    const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (ESZ == 2) {
        tile[tr][cc * VEC + 2 * e] = (uint16_t)(wv[e] & 0xffffu);
        tile[tr][cc * VEC + 2 * e + 1] = (uint16_t)(wv[e] >> 16);
      } else {
        float f[4];
        fpk::e4m3x4_to_f32(wv[e], f);  // every e4m3 value is a bf16 value: truncation is exact
#pragma unroll
        for (int q = 0; q < 4; ++q) tile[tr][cc * VEC + 4 * e + q] = (uint16_t)(__float_as_uint(f[q]) >> 16);
      }
    }
  }
  __syncthreads();
  for (int c = tid; c < 512; c += 256) {
    const int dd = c >> 3, tc = c & 7;
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)tile[tc * 8 + 2 * e][dd] | ((uint32_t)tile[tc * 8 + 2 * e + 1][dd] << 16);
    uint16_t* dst = vt + ((int64_t)g * d + dtile * 64 + dd) * Lpad + tt * 64 + tc * 8;
    *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Max over the 16 lanes of each DPP row.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xb1, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4e, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false)));
  return x;
}

// One workgroup (4 waves) per (q head, tile of 16 block rows).  The score
// tiles use the instruction sequence of the single-sequence selection (same
// bits for the same proxies).  Row i of sequence s sees blocks first[s] .. i.
template <int D>
__global__ __launch_bounds__(256) void select_varlen_kernel(const float* __restrict__ qp, const float* __restrict__ kp,
                                                            const fpk::VlBlock* __restrict__ blk,
                                                            const fpk::VlSeq* __restrict__ seq, int Hq, int Hkv,
                                                            int NB, float scale, float ln_tau,
                                                            float* __restrict__ row_max, int* __restrict__ counts,
                                                            int* __restrict__ indices) {
  extern __shared__ uint16_t kmask[];  // [16][kst], key tiles from tb0
  __shared__ float red[4][16];
  __shared__ float mrow[16];
  __shared__ int first_of[16];
  const int ntiles = (NB + 15) >> 4;
  const int rt = ntiles - 1 - (int)(blockIdx.x / Hq);
  const int h = (int)(blockIdx.x % Hq);
  const int g = h / (Hq / Hkv);
  const int i0 = rt * 16;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int grp = lane >> 4;
  if (threadIdx.x < 16) {
    const int i = min(i0 + (int)threadIdx.x, NB - 1);
    first_of[threadIdx.x] = seq[blk[i].seq].first;
  }
  __syncthreads();
  // first key tile any row of the tile needs, rounded down to a whole
  // 64-column word so that the masks read back with 8-byte loads
  const int tb0 = (first_of[0] >> 4) & ~3;
  const int kst = ((rt - tb0 + 1) + 3) & ~3;
  floatx4 qa[D / 16];
  {
    const int qrow = min(i0 + c16, NB - 1);
    const float* qptr = qp + ((int64_t)h * NB + qrow) * D + 4 * grp;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qa[t] = *reinterpret_cast<const floatx4*>(qptr + 16 * t);
  }
  const float* kbase = kp + (int64_t)g * NB * D + 4 * grp;
  auto tile = [&](int jt) -> floatx4 {
    const int krow = min(jt * 16 + c16, NB - 1);
    const float* kptr = kbase + (int64_t)krow * D;
    floatx4 kb[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) kb[t] = *reinterpret_cast<const floatx4*>(kptr + 16 * t);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[t][c], kb[t][c], acc, 0, 0, 0);
    return acc;
  };
  // ---- pass 1: row maxima over the row's own sequence
  float mr[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int jt = tb0 + w; jt <= rt; jt += 4) {
    const floatx4 acc = tile(jt);
    const int j = jt * 16 + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * grp + r;
      if (j >= first_of[row] && j <= i0 + row) mr[r] = fmaxf(mr[r], acc[r] * scale);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) mr[r] = row16_max(mr[r]);
  if (c16 == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[w][4 * grp + r] = mr[r];
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const int row = threadIdx.x;
    mrow[row] = fmaxf(fmaxf(red[0][row], red[1][row]), fmaxf(red[2][row], red[3][row]));
    if (i0 + row < NB) row_max[(int64_t)h * NB + i0 + row] = mrow[row];
  }
  __syncthreads();
  // ---- pass 2: keep masks (S - m >= ln tau, or the diagonal)
  for (int jt = tb0 + w; jt <= rt; jt += 4) {
    const floatx4 acc = tile(jt);
    const int j = jt * 16 + c16;
    uint64_t bits[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * grp + r;
      const int i = i0 + row;
      const bool keep = (j >= first_of[row] && j <= i && i < NB) &&
                        ((fpk::score_minus_max(acc[r], scale, mrow[row]) >= ln_tau) || j == i);
      bits[r] = __ballot(keep);
    }
    if (lane < 16) {
      const int rr = lane & 3;
      const uint64_t bb = rr == 0 ? bits[0] : rr == 1 ? bits[1] : rr == 2 ? bits[2] : bits[3];
      kmask[lane * kst + (jt - tb0)] = (uint16_t)((bb >> (16 * (lane >> 2))) & 0xffffu);
    }
  }
  __syncthreads();
  // ---- pass 3: compaction; entries are block indices local to the sequence
  for (int row = w; row < 16; row += 4) {
    const int i = i0 + row;
    if (i >= NB) break;
    const fpk::VlBlock m = blk[i];
    const fpk::VlSeq sq = seq[m.seq];
    const int first = sq.first;
    int* out = indices + sq.idx_base + (int64_t)h * sq.nb * (sq.nb + 1) / 2 + (int64_t)m.jl * (m.jl + 1) / 2;
    const int w0 = (first >> 6) - (tb0 >> 2);   // first word (of 64 columns) in mask coordinates
    const int w1 = (i >> 6) - (tb0 >> 2);       // last word
    int base = 0;
    for (int wd0 = w0; wd0 <= w1; wd0 += 64) {
      const int wd = wd0 + lane;
      uint64_t bw = 0;
      if (wd <= w1) {
        const uint2 x = *reinterpret_cast<const uint2*>(kmask + row * kst + 4 * wd);
        const int valid = (i >> 4) - tb0 - 4 * wd + 1;  // tiles up to the row's own
        const uint64_t v = ((uint64_t)x.y << 32) | x.x;
        bw = valid >= 4 ? v : v & ((uint64_t(1) << (16 * valid)) - 1);
      }
      uint64_t nz = __ballot(bw != 0);
      while (nz) {
        const int src = __builtin_ctzll(nz);
        nz &= nz - 1;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bw, src);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bw >> 32), src);
        if ((((uint64_t)hi << 32 | lo) >> lane) & 1)
          out[base + __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0))] =
              64 * (wd0 + src) + 16 * tb0 + lane - first;
        base += __popc(lo) + __popc(hi);
      }
    }
    if (lane == 0) counts[(int64_t)h * NB + i] = base;
  }
}

}  // namespace

hipError_t fpk_launch_varlen_prepare(const fp_problem& p, const fp_varlen& vl, const FpDims& dm, int NB,
                                     fpk::VlBlock* blk, fpk::VlSeq* seq, float* q_pool, float* k_pool,
                                     uint8_t* k_c, hipStream_t st) {
  hipLaunchKernelGGL(varlen_meta_kernel, dim3(1), dim3(256), 0, st, vl.cu_seqlens_dev, vl.num_seqs, dm.B, dm.Hq,
                     NB, blk, seq);
  const bool fp8 = p.dtype == FP_FP8_E4M3;
  const int esz = fp8 ? 1 : 2;
  const int vec = 16 / esz;
  const int* table = vl.block_table_dev;
  VlSrc qs{static_cast<const uint8_t*>(p.q), p.q_stride_tok, p.q_stride_head, 0, nullptr, 0, 0};
  VlSrc ks{static_cast<const uint8_t*>(p.k), p.k_stride_tok, p.k_stride_head, vl.k_page_stride, table,
           vl.max_blocks, vl.num_pages};
  const int wgq = (dm.Hq * dm.d / vec + 63) / 64;
  const int wgk = (dm.Hkv * dm.d / vec + 63) / 64;
  const dim3 gp((unsigned)(NB * (wgq + wgk)));
  const float qsc = fp8 ? p.q_scale : 1.f, ksc = fp8 ? p.k_scale : 1.f;
  if (fp8)
    hipLaunchKernelGGL(pool_varlen_kernel<1>, gp, dim3(256), 0, st, qs, ks, blk, q_pool, k_pool, k_c, dm.Hq, dm.Hkv,
                       dm.d, dm.B, NB, qsc, ksc, wgq, wgk);
  else
    hipLaunchKernelGGL(pool_varlen_kernel<2>, gp, dim3(256), 0, st, qs, ks, blk, q_pool, k_pool, k_c, dm.Hq, dm.Hkv,
                       dm.d, dm.B, NB, qsc, ksc, wgq, wgk);
  return hipGetLastError();
}

hipError_t fpk_launch_vtrans_varlen(const fp_problem& p, const fp_varlen& vl, const FpDims& dm, int NB,
                                    const fpk::VlBlock* blk, uint16_t* v_t, hipStream_t st) {
  VlSrc vs{static_cast<const uint8_t*>(p.v), p.v_stride_tok, p.v_stride_head, vl.v_page_stride, vl.block_table_dev,
           vl.max_blocks, vl.num_pages};
  const int Lpad = NB * dm.B;
  const dim3 gv((unsigned)(Lpad / 64), (unsigned)(dm.d / 64), (unsigned)dm.Hkv);
  if (p.dtype == FP_FP8_E4M3)
    hipLaunchKernelGGL(vtrans_varlen_kernel<1>, gv, dim3(256), 0, st, vs, blk, dm.d, dm.B, Lpad, v_t);
  else
    hipLaunchKernelGGL(vtrans_varlen_kernel<2>, gv, dim3(256), 0, st, vs, blk, dm.d, dm.B, Lpad, v_t);
  return hipGetLastError();
}

hipError_t fpk_launch_select_varlen(const FpDims& dm, int NB, const fpk::VlBlock* blk, const fpk::VlSeq* seq,
                                    const float* q_pool, const float* k_pool, float sm_scale, float ln_tau,
                                    float* row_max, int* counts, int* indices, hipStream_t st) {
  const int ntiles = (NB + 15) / 16;
  const size_t lds = (size_t)16 * (((ntiles + 4) + 3) & ~3) * sizeof(uint16_t);
  const dim3 grid((unsigned)(ntiles * dm.Hq));
  auto launch = [&](auto kern) -> hipError_t {
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, q_pool, k_pool, blk, seq, dm.Hq, dm.Hkv, NB, sm_scale, ln_tau,
                       row_max, counts, indices);
    return hipGetLastError();
  };
  return launch(select_varlen_kernel<128>);
}
