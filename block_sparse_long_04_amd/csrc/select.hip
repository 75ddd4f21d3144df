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
// Work split.  Row tiles are 16 consecutive query-block rows.  A workgroup
// (4 waves) of one q head owns S row tiles (S = 4, 2 or 1, set by the host
// so that there are enough workgroups to fill the chip).  For S = 4 the tiles
// are taken in pairs (2p, 2p+1), and a workgroup owns pair a and pair
// npairs-1-a: a short pair near the top of the causal triangle and a long one
// near the bottom, so every workgroup scores the same number of block pairs
// and no CU ends up with several long rows.  S = 2 pairs single tiles the
// same way; S = 1 is one tile per workgroup, heaviest first.
// Scores are 16x16 tiles from the fp32 matrix cores (v_mfma_f32_16x16x4f32):
// A = 16 pooled query rows, B = 16 pooled key rows, all of the head
// dimension.  Every wave holds the A operands of all S row tiles (slots
// u = 0..S-1), so a key tile it loads feeds S accumulation chains while all
// need it and the long group's afterwards.  Waves stride over key tiles; the
// next tile's rows load while the current one is multiplied.
// Pass 1 takes the row maxima (lanes of a DPP row, then waves via LDS);
// pass 2 recomputes the identical tiles (same instruction sequence, so the
// same bits) and turns the comparison into 16-bit keep masks per (row, key
// tile) held in LDS; pass 3 compacts each row's mask one nonzero 64-column
// word at a time (a lane per column, positions from the count of set bits
// below the lane) and writes the ascending list with contiguous stores.  Only
// kept entries reach HBM.
#include <type_traits>

#include "common.h"

namespace {

using fpk::floatx4;

// Max over the 16 lanes of each DPP row: quad swaps (xor 1, xor 2), then
// rotations by 4 and 8 within the row.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xb1, 0xf, 0xf, false)));  // quad_perm 1,0,3,2
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4e, 0xf, 0xf, false)));  // quad_perm 2,3,0,1
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false)));  // row_ror 4
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false)));  // row_ror 8
  return x;
}

// Workgroups per q head for S row tiles per workgroup.
__host__ __device__ __forceinline__ int groups_of(int ntiles, int S) {
  const int P = S > 1 ? S / 2 : 1;  // tiles of one group (short or long)
  const int ng = (ntiles + P - 1) / P;
  return S > 1 ? (ng + 1) / 2 : ng;
}

// Mask entries per LDS row: the key tiles, rounded up to whole 64-column
// words so pass 3 reads a word with one 8-byte load.
__host__ __device__ __forceinline__ int mask_stride(int ntiles) { return (ntiles + 3) & ~3; }

// Kept scores (the variant that stores pass 1's scores in LDS): a row of row
// tile rt holds its 16 (rt + 1) causal-range columns plus 4 floats of pad, so
// the four row groups of one MFMA result write to different bank groups.
__host__ __device__ __forceinline__ int score_row(int rt) { return 16 * (rt + 1) + 4; }

// Floats of stored scores a workgroup with S row tiles needs at most: slots
// hold the tiles P a .. P a + P - 1 and P b .. P b + P - 1 with a + b =
// ngroups - 1 (or one group alone), so the sum of their score rows is
// largest for the pair with the most tiles in range.
__host__ __device__ __forceinline__ int score_floats(int ntiles, int S) {
  const int P = S > 1 ? S / 2 : 1;
  const int ng = (ntiles + P - 1) / P;
  int best = 0;
  for (int a = 0; a < (S > 1 ? (ng + 1) / 2 : ng); ++a) {
    const int b = S > 1 ? ng - 1 - a : a;
    int sum = 0;
    for (int u = 0; u < S; ++u) {
      const int rt = u < P ? P * a + u : P * b + u - P;
      if (rt < ntiles && (u < P || b != a)) sum += 16 * score_row(rt);
    }
    best = sum > best ? sum : best;
  }
  return best;
}

template <int D, int kSlots, bool kStore>
__global__ __launch_bounds__(256, 2) void select_kernel(const float* __restrict__ qp,
                                                        const float* __restrict__ kp, int Hq, int Hkv,
                                                        int nb, float scale, float ln_tau, int dense,
                                                        int kmask_off,
                                                        float* __restrict__ row_max,
                                                        int* __restrict__ counts,
                                                        int* __restrict__ indices) {
  // [stored scores (kStore)][16 S local rows][mask_stride] keep masks
  extern __shared__ __align__(16) unsigned char dsm[];
  __shared__ float red[4][16 * kSlots];
  __shared__ __align__(16) float mrow[16 * kSlots];  // row maxima of the local rows

  const int ntiles = (nb + 15) >> 4;
  const int kst = mask_stride(ntiles);
  float* const sc = reinterpret_cast<float*>(dsm);
  uint16_t* const kmask = reinterpret_cast<uint16_t*>(dsm + kmask_off);  // after the scores
  constexpr int P = kSlots > 1 ? kSlots / 2 : 1;  // row tiles per group
  const int ngroups = (ntiles + P - 1) / P;
  // short group (S = 1: the only one, heaviest first)
  const int a = kSlots > 1 ? (int)(blockIdx.x / Hq) : ngroups - 1 - (int)(blockIdx.x / Hq);
  const int b = kSlots > 1 ? ngroups - 1 - a : a;        // long group
  const int h = (int)(blockIdx.x % Hq);
  const int g = h / (Hq / Hkv);
  const bool two = kSlots > 1 && b != a;                 // false: the short group alone
  const int lo_hi = min(P * a + P - 1, ntiles - 1);      // last key tile of the short group
  const int rt_hi = two ? min(P * b + P - 1, ntiles - 1) : lo_hi;  // last key tile of the workgroup
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int grp = lane >> 4;
  // Lane (c16, grp) holds S[i][j] with i = 16 rt_u + 4grp + r, j = 16jt + c16,
  // so j <= i  <=>  dl - r <= 16 (rt_u - jt).
  const int dl = c16 - 4 * grp;
  auto slot_tile = [&](int u) { return u < P ? P * a + u : P * b + u - P; };
  // first stored score of each slot (kStore): slots in order, unused ones
  // empty; uniform, so these stay in scalar registers
  int soff[kSlots];
  {
    int off = 0;
#pragma unroll
    for (int v = 0; v < kSlots; ++v) {
      soff[v] = off;
      if (slot_tile(v) < ntiles && (v < P || two)) off += 16 * score_row(slot_tile(v));
    }
  }

  // A operands: lane supplies Qbar[16 rt_u + c16][16t + 4grp + c] for slot u
  // in MFMA step (t, c).  Without a long group, its slots repeat the short
  // group's (their rows are never used).
  floatx4 qa[kSlots][D / 16];
#pragma unroll
  for (int u = 0; u < kSlots; ++u) {
    const int qrow = min(16 * slot_tile(u) + c16, nb - 1);
    const float* qptr = qp + ((int64_t)h * nb + qrow) * D + 4 * grp;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qa[u][t] = *reinterpret_cast<const floatx4*>(qptr + 16 * t);
  }
  // Pooled keys of kv head g through a buffer resource: the intrinsic loads
  // stay where they are issued, so the read-ahead is really ahead.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(kp + (int64_t)g * nb * D), 0, nb * D * (int)sizeof(float), 0x00020000);

  // B operand of key tile jt: lane supplies Kbar[16jt + c16][16t + 4grp + c].
  // Rows past the last block are clamped to it (their columns are masked).
  struct KRows {
    floatx4 v[D / 16];
  };
  auto load_rows = [&](int jt) -> KRows {
    KRows r;
    const int krow = min(jt * 16 + c16, nb - 1);
    const int off = (krow * D + 4 * grp) * (int)sizeof(float);
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      r.v[t] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 64 * t, 0, 0));
    return r;
  };
  // D layout: lane holds S[16 rt_u + 4grp + r][16jt + c16], r = 0..3.  The
  // slots from U0 (0, or P for the long group alone) to S-1 are independent
  // chains, interleaved; the sequence per (slot, jt) is the same in both
  // passes, so the bits are too.
  auto tiles = [&](const KRows& kr, floatx4 (&acc)[kSlots], auto u0c) {
    constexpr int U0 = decltype(u0c)::value;
#pragma unroll
    for (int u = U0; u < kSlots; ++u) acc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int u = U0; u < kSlots; ++u)
          acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[u][t][c], kr.v[t][c], acc[u], 0, 0, 0);
  };
  using All = std::integral_constant<int, 0>;   // key tile needed by every slot
  using Long = std::integral_constant<int, P>;  // key tile needed by the long group only

  // ---- pass 1: row maxima over j <= i
  float mr[kSlots][4];
#pragma unroll
  for (int u = 0; u < kSlots; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) mr[u][r] = -INFINITY;
  auto max_step = [&](const KRows& kr, int jt, auto u0c) {
    constexpr int U0 = decltype(u0c)::value;
    floatx4 acc[kSlots];
    tiles(kr, acc, u0c);
#pragma unroll
    for (int u = U0; u < kSlots; ++u) {
      const int lim = 16 * (slot_tile(u) - jt);
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = acc[u][r] * scale;
        if (dl - r <= lim) mr[u][r] = fmaxf(mr[u][r], sv[r]);
      }
      // the scores of key tiles up to the slot's own, for pass 2
      if (kStore && lim >= 0 && slot_tile(u) < ntiles && (u < P || two)) {
        const int rl = score_row(slot_tile(u));
        float* dst = sc + soff[u] + 4 * grp * rl + 16 * jt + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r * rl] = sv[r];
      }
    }
  };
  auto max_any = [&](const KRows& kr, int jt) {
    if (jt <= lo_hi) max_step(kr, jt, All{});
    else max_step(kr, jt, Long{});
  };
  // Two register sets in turn: tile jt + 4 loads while tile jt multiplies.
  // The step for jt + 4 runs even past the last tile, which keeps the loads
  // unconditional; there j > i for every row, so the causal test rejects all.
  if (w <= rt_hi) {
    KRows ka = load_rows(w);
    for (int jt = w; jt <= rt_hi; jt += 8) {
      const KRows kb = load_rows(jt + 4);
      __builtin_amdgcn_sched_barrier(0);
      max_any(ka, jt);
      ka = load_rows(jt + 8);
      __builtin_amdgcn_sched_barrier(0);
      max_any(kb, jt + 4);
    }
  }
#pragma unroll
  for (int u = 0; u < kSlots; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) mr[u][r] = row16_max(mr[u][r]);
  if (c16 == 0) {
#pragma unroll
    for (int u = 0; u < kSlots; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[w][16 * u + 4 * grp + r] = mr[u][r];
  }
  __syncthreads();
  if (threadIdx.x < 16 * kSlots) {
    const int row = threadIdx.x;
    mrow[row] = fmaxf(fmaxf(red[0][row], red[1][row]), fmaxf(red[2][row], red[3][row]));
    const int u = row >> 4;
    const int i = 16 * slot_tile(u) + (row & 15);
    if ((u < P || two) && i < nb) row_max[(int64_t)h * nb + i] = mrow[row];
  }
  __syncthreads();

  // ---- pass 2: keep masks of (local row, key tile) for every key tile up
  // to the row's own tile; entries past it are never read
  auto put_masks = [&](int jt, int u, const uint64_t (&bits)[4]) {
    if (lane < 16) {
      const int rr = lane & 3;
      const uint64_t bb = rr == 0 ? bits[0] : rr == 1 ? bits[1] : rr == 2 ? bits[2] : bits[3];
      kmask[(16 * u + lane) * kst + jt] = (uint16_t)((bb >> (16 * (lane >> 2))) & 0xffffu);
    }
  };
  auto mask_step = [&](const KRows& kr, int jt, auto u0c) {  // stores only for jt <= rt_hi
    constexpr int U0 = decltype(u0c)::value;
    floatx4 acc[kSlots];
    tiles(kr, acc, u0c);
    // The row maxima come from LDS after the products are issued (a compiler
    // barrier keeps the reads here): they are not held across the loop.
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int u = U0; u < kSlots; ++u) {
      const int rt = slot_tile(u);
      const int lim = 16 * (rt - jt);
      const int rows_left = nb - 16 * rt;  // i < nb  <=>  4 grp + r < rows_left
      const floatx4 mu = *reinterpret_cast<const floatx4*>(mrow + 16 * u + 4 * grp);
      uint64_t bits[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool keep = (dl - r <= lim && 4 * grp + r < rows_left) &&
                          ((fpk::score_minus_max(acc[u][r], scale, mu[r]) >= ln_tau) || dl - r == lim);
        bits[r] = __ballot(keep);
      }
      if (jt <= rt_hi) put_masks(jt, u, bits);
    }
  };
  auto mask_any = [&](const KRows& kr, int jt) {
    if (jt <= lo_hi) mask_step(kr, jt, All{});
    else mask_step(kr, jt, Long{});
  };
  // pass 2 from the stored scores: the same decision on the same bits
  auto mask_stored = [&](int jt) {
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int rt = slot_tile(u);
      if (jt > rt || rt >= ntiles || !(u < P || two)) continue;
      const int lim = 16 * (rt - jt);
      const int rows_left = nb - 16 * rt;
      const int rl = score_row(rt);
      const float* src = sc + soff[u] + 4 * grp * rl + 16 * jt + c16;
      const floatx4 mu = *reinterpret_cast<const floatx4*>(mrow + 16 * u + 4 * grp);
      uint64_t bits[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float d = src[r * rl] - mu[r];
        const bool keep = (dl - r <= lim && 4 * grp + r < rows_left) && (d >= ln_tau || dl - r == lim);
        bits[r] = __ballot(keep);
      }
      put_masks(jt, u, bits);
    }
  };
  if (w <= rt_hi) {
    if (kStore && !dense) {
      for (int jt = w; jt <= rt_hi; jt += 4) mask_stored(jt);
    } else if (dense) {
      for (int jt = w; jt <= rt_hi; jt += 4) {
#pragma unroll
        for (int u = 0; u < kSlots; ++u) {
          const int rt = slot_tile(u);
          if (jt > rt) continue;
          const int lim = 16 * (rt - jt);
          const int rows_left = nb - 16 * rt;
          uint64_t bits[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) bits[r] = __ballot(dl - r <= lim && 4 * grp + r < rows_left);
          put_masks(jt, u, bits);
        }
      }
    } else {
      KRows ka = load_rows(w);
      for (int jt = w; jt <= rt_hi; jt += 8) {
        const KRows kb = load_rows(jt + 4);
        __builtin_amdgcn_sched_barrier(0);
        mask_any(ka, jt);
        ka = load_rows(jt + 8);
        __builtin_amdgcn_sched_barrier(0);
        mask_any(kb, jt + 4);
      }
    }
  }
  __syncthreads();

  // ---- pass 3: compaction.  Wave w owns local rows w, w+4, w+8, ...: four
  // rows of every slot, so short and long rows are shared evenly.
  constexpr int kRows = 16 * kSlots / 4;
  int base[kRows];
  int row_i[kRows];
  int nwords_max = 0;
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const int lr = w + 4 * k;
    const int u = lr >> 4;
    const int i = 16 * slot_tile(u) + (lr & 15);
    row_i[k] = (u < P || two) && i < nb ? i : -1;
    base[k] = 0;
    if (row_i[k] >= 0) nwords_max = max(nwords_max, (i + 64) >> 6);
  }
  for (int wd0 = 0; wd0 < nwords_max; wd0 += 64) {
    const int wd = wd0 + lane;  // this lane's 64-column word: key tiles 4wd .. 4wd+3
    uint64_t bw[kRows];
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const int i = row_i[k];
      bw[k] = 0;
      if (i >= 0 && wd <= (i >> 6)) {
        const uint2 x = *reinterpret_cast<const uint2*>(kmask + (w + 4 * k) * kst + 4 * wd);
        const int valid = (i >> 4) - 4 * wd + 1;  // entries up to the row's own tile
        const uint64_t v = ((uint64_t)x.y << 32) | x.x;
        bw[k] = valid >= 4 ? v : v & ((uint64_t(1) << (16 * valid)) - 1);
      }
    }
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      if (row_i[k] < 0) continue;
      int* out = indices + fpk::tri_offset(h, row_i[k], nb);
      int bs = base[k];
      uint64_t nz = __ballot(bw[k] != 0);
      while (nz) {
        const int src = __builtin_ctzll(nz);
        nz &= nz - 1;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bw[k], src);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bw[k] >> 32), src);
        if ((((uint64_t)hi << 32 | lo) >> lane) & 1)
          out[bs + __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0))] = 64 * (wd0 + src) + lane;
        bs += __popc(lo) + __popc(hi);
      }
      base[k] = bs;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < kRows; ++k)
      if (row_i[k] >= 0) counts[(int64_t)h * nb + row_i[k]] = base[k];
  }
}

}  // namespace

hipError_t fpk_launch_select(const FpDims& dm, const float* q_pool, const float* k_pool,
                             float sm_scale, float ln_tau, float* row_max, int* counts,
                             int* indices, hipStream_t st) {
  const int ntiles = (dm.nb + 15) / 16;
  // Most row tiles per workgroup that still give a workgroup per CU (256
  // CUs); below that, parallelism matters more than K-tile reuse.  (Measured
  // at 8K / 32K / 128K / 256K: S = 1 / 2 / 4 / 4 is the fastest choice.)
  constexpr int kMinGroups = 256;
  int S = 4;
  if (groups_of(ntiles, 4) * dm.Hq < kMinGroups) S = groups_of(ntiles, 2) * dm.Hq >= kMinGroups ? 2 : 1;
  // Pass 1's scores stay in LDS for pass 2 when they fit two workgroups per
  // CU (the largest S at or below the choice above that fits; at most 2 for
  // D = 128, whose four-slot variant has no registers left for the stores);
  // otherwise pass 2 recomputes them.
  constexpr size_t kStoreLds = 80 * 1024;
  const bool dense_sel = ln_tau == -INFINITY;
  bool store = false;
  for (int s2 = dm.d == 128 ? min(S, 2) : S; s2 >= 1 && !dense_sel; s2 /= 2) {
    const size_t need = (size_t)score_floats(ntiles, s2) * 4 + (size_t)16 * s2 * mask_stride(ntiles) * 2;
    if (need <= kStoreLds) {
      S = s2;
      store = true;
      break;
    }
  }
  const size_t kmask_off = store ? (size_t)score_floats(ntiles, S) * 4 : 0;
  const size_t lds = kmask_off + (size_t)16 * S * mask_stride(ntiles) * sizeof(uint16_t);
  const int dense = dense_sel ? 1 : 0;
  const dim3 grid((unsigned)(groups_of(ntiles, S) * dm.Hq));
  auto launch = [&](auto kern) -> hipError_t {
    // 16 S rows x nb bits of masks (and the stored scores): up to 128 KiB at
    // 16384 blocks, above the default 64 KiB dynamic LDS window, so raise the
    // kernel's limit when needed.
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, q_pool, k_pool, dm.Hq, dm.Hkv, dm.nb, sm_scale,
                       ln_tau, dense, (int)kmask_off, row_max, counts, indices);
    return hipGetLastError();
  };
  if (dm.d == 128) {
    if (store) return S == 2 ? launch(select_kernel<128, 2, true>) : launch(select_kernel<128, 1, true>);
    if (S == 4) return launch(select_kernel<128, 4, false>);
    if (S == 2) return launch(select_kernel<128, 2, false>);
    return launch(select_kernel<128, 1, false>);
  }
  if (store) {
    if (S == 4) return launch(select_kernel<64, 4, true>);
    if (S == 2) return launch(select_kernel<64, 2, true>);
    return launch(select_kernel<64, 1, true>);
  }
  if (S == 4) return launch(select_kernel<64, 4, false>);
  if (S == 2) return launch(select_kernel<64, 2, false>);
  return launch(select_kernel<64, 1, false>);
}
