// Sort / cumulative-sum selection baselines on the same block proxies as the
// max threshold: top-k and top-p.
//
// FlashPrefill skill page, "Core Concept", and the FlashPrefill abstract: the
// single-pass max threshold is the pages' answer to the search overhead of
// the selection rules that sort the block scores (top-k) or accumulate their
// probability mass (top-p).  These kernels implement those rules on the GPU so
// that the overhead can be measured next to the threshold kernel:
//   * top-k: the k causal blocks with the largest scores (ties: smaller block
//     index first);
//   * top-p: the shortest prefix of the blocks in descending score order whose
//     block-softmax mass reaches p;
// both plus the diagonal block.
//
// One workgroup (4 waves) owns 16 consecutive query-block rows of one q head
// (heaviest rows first).
//   A. Scores: 16x16 tiles on the fp32 matrix cores with the instruction
//      sequence of the threshold kernel (so the same bits), stored in LDS as
//      order-preserving 32-bit keys, one row of pow2(nb) keys per query block,
//      -inf past the diagonal.
//   B. Each wave sorts four rows, one at a time, in registers (bitonic,
//      descending; the row length rounded up to a power of two, 64 E keys
//      held E per lane) and finds the cut: top-k takes the k-th key; top-p
//      weighs the sorted scores by exp(S - m), sums them (fp32, a contiguous
//      chunk per lane, then a wave scan) and takes the first prefix reaching
//      p times the total.  Blocks equal to the cut key fill the remaining
//      places in ascending block order.
//   C. The tiles are recomputed (same bits) and compared with the cut key:
//      16-bit masks of blocks above it and of blocks equal to it.
//   D. Compaction as in the threshold kernel, after taking the needed number
//      of equal blocks lowest index first and adding the diagonal.
// The rows live in LDS whole, so this baseline takes nb <= 2048.
#include "common.h"

namespace {

using fpk::floatx4;

// fp32 -> uint32, monotone: a < b  <=>  key(a) < key(b) (no NaN here)
__device__ __forceinline__ uint32_t ord_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_val(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
constexpr uint32_t kNegInfKey = 0x007fffffu;  // ord_key(-inf)

__host__ __device__ __forceinline__ int pow2_at_least(int n) {
  int p = 64;
  while (p < n) p <<= 1;
  return p;
}
__host__ __device__ __forceinline__ int mask_stride(int ntiles) { return (ntiles + 3) & ~3; }

// Bitonic sort of n = 64 E keys held E per lane (lane l: elements l E ..
// l E + E - 1), descending.  In the stage (k, j) the element with index x
// meets x ^ j; the lower of the two takes the larger key where bit k of x is
// clear (a descending run), the smaller where it is set.  Strides below E
// stay inside a lane's registers, longer ones swap with lane ^ (j / E).
template <int E>
__device__ __forceinline__ void sort_desc(uint32_t (&v)[E], int lane) {
#pragma unroll
  for (int k = 2; k <= 64 * E; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (e & j) continue;
          const int x = lane * E + e;
          const bool desc = (x & k) == 0;
          const uint32_t a = v[e], b = v[e | j];
          v[e] = desc ? max(a, b) : min(a, b);
          v[e | j] = desc ? min(a, b) : max(a, b);
        }
      } else {
        const int lm = j / E;
        const bool lower = (lane & lm) == 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t y = (uint32_t)__shfl_xor((int)v[e], lm);
          const bool desc = ((lane * E + e) & k) == 0;
          v[e] = (lower == desc) ? max(v[e], y) : min(v[e], y);
        }
      }
    }
  }
}

// Element x of the sorted row (x uniform over the wave): register x % E of
// lane x / E, read with readlane from every register and combined with
// masks, so that no register is indexed at run time.
template <int E>
__device__ __forceinline__ uint32_t element(const uint32_t (&v)[E], int x) {
  const int src = x / E, e = x - src * E;
  uint32_t r = 0;
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const uint32_t vq = (uint32_t)__builtin_amdgcn_readlane((int)v[q], src);
    r |= q == e ? vq : 0u;
  }
  return r;
}

// Sort row i (keys in LDS, n = 64 E entries, -inf past the row), find its
// cut and return (cut key, blocks to take among those equal to it, row max).
template <int E>
__device__ void row_cut(const uint32_t* s, int i, int lane, int rule, float param, uint32_t& ck_out,
                        int& need_out, float& m_out) {
  uint32_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = s[lane * E + e];
  sort_desc<E>(v, lane);
  const float m = key_val((uint32_t)__builtin_amdgcn_readlane((int)v[0], 0));
  int n_keep;
  if (rule == 1) {
    n_keep = min((int)param, i + 1);
  } else {
    // weights exp(S - m) of this lane's contiguous chunk, summed in order,
    // then a wave scan; the lane whose chunk crosses p times the total walks it
    float w[E];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      w[e] = __expf(key_val(v[e]) - m);
      ps += w[e];
    }
    float incl = ps;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const float up = __shfl_up(incl, 1);  // every lane takes part in the exchange
    const float excl = lane == 0 ? 0.f : up;
    const float total = __shfl(incl, 63);
    const float target = param * total;
    const uint64_t hit = __ballot(incl >= target);
    if (hit == 0) {
      n_keep = i + 1;
    } else {
      const int L = __builtin_ctzll(hit);
      int pos = lane * E + E - 1;
      float acc = excl;
      bool found = false;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        acc += w[e];
        if (!found && acc >= target) {
          pos = lane * E + e;
          found = true;
        }
      }
      n_keep = min(__shfl(pos, L) + 1, i + 1);
    }
  }
  const int c = n_keep - 1;
  const uint32_t ck = element<E>(v, c);
  int gt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) gt += v[e] > ck ? 1 : 0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) gt += __shfl_xor(gt, off);
  ck_out = ck;
  need_out = n_keep - gt;
  m_out = m;
}

template <int D>
__global__ __launch_bounds__(256) void select_sorted_kernel(const float* __restrict__ qp,
                                                            const float* __restrict__ kp, int Hq,
                                                            int Hkv, int nb, float scale, int rule,
                                                            float param, float* __restrict__ row_max,
                                                            int* __restrict__ counts,
                                                            int* __restrict__ indices) {
  extern __shared__ uint32_t dyn[];
  __shared__ uint32_t cut_key[16];
  __shared__ int need_eq[16];
  const int ntiles = (nb + 15) >> 4;
  const int rs = pow2_at_least(nb);      // keys per LDS row
  const int kst = mask_stride(ntiles);   // mask words per LDS row
  uint32_t* keys = dyn;                                            // [16][rs]
  uint16_t* gmask = reinterpret_cast<uint16_t*>(dyn + 16 * rs);    // [16][kst] above the cut
  uint16_t* emask = gmask + 16 * kst;                              // [16][kst] equal to the cut

  const int rt = ntiles - 1 - (int)(blockIdx.x / Hq);  // heaviest rows first
  const int h = (int)(blockIdx.x % Hq);
  const int g = h / (Hq / Hkv);
  const int i0 = rt * 16;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int grp = lane >> 4;

  for (int e = threadIdx.x; e < 16 * rs; e += 256) keys[e] = kNegInfKey;

  floatx4 qa[D / 16];
  {
    const int qrow = min(i0 + c16, nb - 1);
    const float* qptr = qp + ((int64_t)h * nb + qrow) * D + 4 * grp;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qa[t] = *reinterpret_cast<const floatx4*>(qptr + 16 * t);
  }
  const float* kbase = kp + (int64_t)g * nb * D + 4 * grp;
  // lane holds S[i0 + 4grp + r][16jt + c16]; same sequence as the threshold kernel
  auto tile = [&](int jt) -> floatx4 {
    const int krow = min(jt * 16 + c16, nb - 1);
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
  __syncthreads();

  // ---- A: scores as keys
  for (int jt = w; jt <= rt; jt += 4) {
    const floatx4 acc = tile(jt);
    const int j = jt * 16 + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * grp + r;
      if (j <= i0 + row && i0 + row < nb) keys[row * rs + j] = ord_key(acc[r] * scale);
    }
  }
  __syncthreads();

  // ---- B: sort each row (descending) and find its cut
  for (int row = w; row < 16; row += 4) {
    const int i = i0 + row;
    if (i >= nb) break;
    const uint32_t* s = keys + row * rs;
    uint32_t ck;
    int need;
    float m;
    switch (pow2_at_least(i + 1) >> 6) {
      case 1: row_cut<1>(s, i, lane, rule, param, ck, need, m); break;
      case 2: row_cut<2>(s, i, lane, rule, param, ck, need, m); break;
      case 4: row_cut<4>(s, i, lane, rule, param, ck, need, m); break;
      case 8: row_cut<8>(s, i, lane, rule, param, ck, need, m); break;
      case 16: row_cut<16>(s, i, lane, rule, param, ck, need, m); break;
      default: row_cut<32>(s, i, lane, rule, param, ck, need, m); break;
    }
    if (lane == 0) {
      cut_key[row] = ck;
      need_eq[row] = need;
      row_max[(int64_t)h * nb + i] = m;
    }
  }
  __syncthreads();

  // ---- C: masks of blocks above and equal to the cut (recomputed tiles)
  for (int jt = w; jt <= rt; jt += 4) {
    const floatx4 acc = tile(jt);
    const int j = jt * 16 + c16;
    uint64_t above[4], equal[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * grp + r;
      const int i = i0 + row;
      const bool valid = j <= i && i < nb;
      const uint32_t kk = ord_key(acc[r] * scale);
      const uint32_t ck = cut_key[row];
      above[r] = __ballot(valid && kk > ck);
      equal[r] = __ballot(valid && kk == ck);
    }
    if (lane < 16) {
      const int rr = lane & 3, sh = 16 * (lane >> 2);
      const uint64_t ba = rr == 0 ? above[0] : rr == 1 ? above[1] : rr == 2 ? above[2] : above[3];
      const uint64_t be = rr == 0 ? equal[0] : rr == 1 ? equal[1] : rr == 2 ? equal[2] : equal[3];
      gmask[lane * kst + jt] = (uint16_t)((ba >> sh) & 0xffffu);
      emask[lane * kst + jt] = (uint16_t)((be >> sh) & 0xffffu);
    }
  }
  __syncthreads();

  // ---- D: compaction; blocks equal to the cut taken lowest index first
  for (int row = w; row < 16; row += 4) {
    const int i = i0 + row;
    if (i >= nb) break;
    const int nwords = (i >> 6) + 1;
    int* out = indices + fpk::tri_offset(h, i, nb);
    int base = 0;
    int eq_left = need_eq[row];
    for (int wd0 = 0; wd0 < nwords; wd0 += 64) {
      const int wd = wd0 + lane;
      uint64_t ga = 0, ge = 0;
      if (wd < nwords) {
        const uint2 xa = *reinterpret_cast<const uint2*>(gmask + row * kst + 4 * wd);
        const uint2 xe = *reinterpret_cast<const uint2*>(emask + row * kst + 4 * wd);
        const int valid = (i >> 4) - 4 * wd + 1;
        const uint64_t lim = valid >= 4 ? ~uint64_t(0) : ((uint64_t(1) << (16 * valid)) - 1);
        ga = (((uint64_t)xa.y << 32) | xa.x) & lim;
        ge = (((uint64_t)xe.y << 32) | xe.x) & lim;
      }
      // equal blocks: this word's share of the remaining places, lowest first
      const int ce = __popcll(ge);
      int incl = ce;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      int take = min(max(eq_left - (incl - ce), 0), ce);
      while (__popcll(ge) > take) ge &= ~(uint64_t(1) << (63 - __builtin_clzll(ge)));
      eq_left -= min(eq_left, __shfl(incl, 63));
      uint64_t bw = ga | ge;
      if (wd == (i >> 6)) bw |= uint64_t(1) << (i & 63);  // the diagonal block
      uint64_t nz = __ballot(bw != 0);
      while (nz) {
        const int src = __builtin_ctzll(nz);
        nz &= nz - 1;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bw, src);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bw >> 32), src);
        if ((((uint64_t)hi << 32 | lo) >> lane) & 1)
          out[base + __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0))] = 64 * (wd0 + src) + lane;
        base += __popc(lo) + __popc(hi);
      }
    }
    if (lane == 0) counts[(int64_t)h * nb + i] = base;
  }
}

}  // namespace

size_t fpk_select_sorted_lds(int nb) {
  const int ntiles = (nb + 15) / 16;
  return (size_t)16 * pow2_at_least(nb) * 4 + (size_t)2 * 16 * mask_stride(ntiles) * 2;
}

hipError_t fpk_launch_select_sorted(const FpDims& dm, const float* q_pool, const float* k_pool,
                                    float sm_scale, int rule, float param, float* row_max,
                                    int* counts, int* indices, hipStream_t st) {
  const int ntiles = (dm.nb + 15) / 16;
  const size_t lds = fpk_select_sorted_lds(dm.nb);
  const dim3 grid((unsigned)(ntiles * dm.Hq));
  auto launch = [&](auto kern) -> hipError_t {
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, q_pool, k_pool, dm.Hq, dm.Hkv, dm.nb, sm_scale,
                       rule, param, row_max, counts, indices);
    return hipGetLastError();
  };
  return dm.d == 128 ? launch(select_sorted_kernel<128>) : launch(select_sorted_kernel<64>);
}
