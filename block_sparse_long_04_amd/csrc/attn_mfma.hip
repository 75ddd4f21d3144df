// Step 5 on the matrix cores: block-sparse causal attention with GQA over the
// kept key blocks, head_dim 128, block 128, bf16 or e4m3fn inputs.
//
// e4m3fn inputs (FlashPrefill V2 abstract: FP8 inference): S^T = K Q^T runs
// on v_mfma_scale_f32_32x32x64_f8f6f4 straight from the e4m3 codes (unit
// block scales; the per-tensor scales q_scale*k_scale are folded into the
// softmax scale), the K tile is staged as 128-byte rows, and P.V stays in
// bf16: V^T is widened exactly from e4m3 to bf16 by the layout pass and
// v_scale is applied to the output, so P is not quantised to 8 bits.
//
// FlashPrefill skill page, "Architecture Overview" (physical index jumping:
// only the listed key blocks are visited) and "Implementation Steps" (the
// last stage is block-sparse attention over the identified blocks); GQA per
// the FlashPrefill V2 abstract.
//
// One workgroup = one (q head h, query block i), 8 waves.  Wave w owns query
// rows 32*(w%4) .. +31 and key half kh = w/4 (keys 64kh .. 64kh+63 of every
// kept block); the two halves keep separate online-softmax states and are
// merged through LDS at the end.  Two waves per SIMD let one wave's softmax
// (VALU) run under the other's matrix-core work.
//
// Per kept key block j (ascending list, the diagonal last):
//   * the K tile [128 keys][128 dims] and the V^T tile [128 dims][128 keys]
//     travel global -> LDS with global_load_lds_dwordx4 (no registers), double
//     buffered: the next block's tiles are in flight while this one computes.
//     Rows are 16 chunks of 16 B stored at chunk ^ f(row), f(r) = (r & 15) ^
//     (((r >> 3) & 1) << 2), so the operand reads below hit distinct banks;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: two 32-key sub-tiles, eight
//     16-wide steps over the head dimension.  A lane column is one query, so
//     a lane holds 32 of its query's logits and lane ^ 32 the rest.  K rows
//     are fed in the order pm(m) (bits 2 and 3 of m swapped), which makes
//     each lane's logits contiguous 8-key runs: the B operand of P.V as is;
//   * online softmax in the exp2 domain with a lazy maximum: the running max
//     is raised (and O, l rescaled) only when a tile's max exceeds it by more
//     than 8 (P <= 2^8 stays exact enough in bf16 and cannot overflow fp32);
//   * O^T += V^T P^T, P packed to bf16 from the S^T registers.
// The causal mask is applied on the diagonal block only.  1/l and the V
// dequantisation scale are applied once, after the merge.
//
// Work order: heavy (late) query blocks first; within every run of 8*G
// consecutive workgroup ids, the G heads of one kv group at one query block
// get ids the hardware deals to the same XCD (ids go round-robin over the 8
// XCDs), so a K/V tile fetched for one head is found in that XCD's L2 by the
// other heads of its group.  The group-to-XCD assignment rotates with the
// query block so that no XCD is left with one group's whole workload.
#include "common.h"

namespace {

using fpk::bf16x8;
using fpk::floatx16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct AttnArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint16_t* vt;
  uint16_t* out;
  const int* counts;
  const int* indices;
  int64_t q_st, q_sh, k_st, k_sh, o_st, o_sh;
  int L, Hq, Hkv, nb, Lpad;
  float scale_log2;  // sm_scale * log2(e) (times q_scale * k_scale for e4m3 inputs)
  float out_scale;
};

constexpr int kTileU4 = 128 * 16;  // one 128 x 256 B tile in uint4
constexpr float kLazy = 8.0f;      // lazy-max slack in log2 units

__device__ __forceinline__ void work_item(int bid, int nb, int Hq, int Hkv, int& h, int& i) {
  const int G = Hq / Hkv;
  const int total = nb * Hq;
  const int chunk = 8 * G;
  const int full = (total / chunk) * chunk;
  int p, slot;
  if (bid < full) {
    // run `sup` of 8*G ids: XCD x (= id % 8) gets (row, group) pair
    // sup*8 + (x + sup) % 8 with its G heads; the rotation spreads every kv
    // group over all XCDs, so per-group differences in kept work even out.
    const int sup = bid / chunk;
    const int r = bid - sup * chunk;
    p = sup * 8 + (((r & 7) + sup) & 7);
    slot = r >> 3;
  } else {
    p = bid / G;
    slot = bid - p * G;
  }
  const int row = p / Hkv;
  i = nb - 1 - row;
  h = (p - row * Hkv) * G + slot;
}

__device__ __forceinline__ int swz(int row) { return (row & 15) ^ (((row >> 3) & 1) << 2); }
// e4m3 K rows are 128 B (8 chunks): the chunk XOR (row >> 1) & 7 sends the 16
// rows one operand read touches to 16 different bank groups.
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

using fpk::intx8;

// Q fragments (B operand of S^T = K Q^T) for one query row: bf16 holds
// Q[16s + 8hh .. +7] for 8 steps s; e4m3 holds Q[64s + 32hh .. +31] for 2.
template <bool kFp8>
struct QFrag;
template <>
struct QFrag<false> {
  bf16x8 f[8];
};
template <>
struct QFrag<true> {
  intx8 f[2];
};

// S^T (32 keys x 32 queries) += K rows `row` of the tile times Q, over the
// whole head dimension.
template <bool kFp8>
__device__ __forceinline__ floatx16 qk_rows(const uint4* sK, const QFrag<kFp8>& q, int row, int hh,
                                            floatx16 acc) {
  if constexpr (!kFp8) {
    const uint4* kr = sK + row * 16;
    const int x = swz(row) ^ hh;
#pragma unroll
    for (int st = 0; st < 8; ++st)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(&kr[(2 * st) ^ x]),
                                                    q.f[st], acc, 0, 0, 0);
  } else {
    const uint4* kr = sK + row * 8;
    const int x = swz8(row);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int c0 = 4 * st + 2 * hh;
      const uint4 lo = kr[c0 ^ x], hi = kr[(c0 + 1) ^ x];
      const intx8 a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, q.f[st], acc, 0, 0, 0, 127, 0, 127);
    }
  }
  return acc;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

struct WaveState {
  floatx16 o[4];
  float m;  // lazy running max (log2 domain)
  float l;  // this lane's partial row sum
};

// Softmax statistics of one tile's logits: causal mask on the diagonal block,
// row max, and the lazy raise of the running max (rescaling O and l).
__device__ __forceinline__ void softmax_stats(floatx16* s, WaveState& ws, float c, bool diag,
                                              int qg, int kh, int qi, int hh) {
  if (diag) {
    const int qrel = 32 * qg + qi;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int krel = 64 * kh + 32 * kt + 16 * (r >> 3) + 8 * hh + (r & 7);
        if (krel > qrel) s[kt][r] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mxs = mx * c;
  if (__any(mxs > ws.m + kLazy)) {
    const float m_new = fmaxf(ws.m, mxs);
    const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(ws.m - m_new);
    ws.m = m_new;
    ws.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) ws.o[dt] *= alpha;
  }
}

// exp2 of one 32-key sub-tile into bf16 P (two 8-key runs); the row sum is
// taken from the bf16 values themselves with v_dot2 against (1, 1), so l
// normalises exactly the weights that enter P.V.
__device__ __forceinline__ void exp_subtile(const floatx16& s, float c, float mu, float& l,
                                            bf16x8& p0, bf16x8& p1) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const __bf16 p = (__bf16)__builtin_amdgcn_exp2f(s[r] * c - mu);
    if (r < 8) p0[r] = p;
    else p1[r - 8] = p;
  }
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    l = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){p0[2 * e], p0[2 * e + 1]}, one, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){p1[2 * e], p1[2 * e + 1]}, one, l, false);
  }
}

// One pipelined step: S(n+1) = K(n+1) Q^T on the matrix cores interleaved
// with the exponentials of tile n, then O += P(n) V(n) interleaved with the
// rest of the exponentials.  sched_group_barrier pins the interleave (MFMA,
// LDS read, a few VALU) so the in-order wave keeps both pipes busy.
template <bool kFp8>
__device__ __forceinline__ void pipelined_step(const uint4* sKn, const uint4* sV,
                                               const QFrag<kFp8>& qf, const floatx16* s_cur,
                                               floatx16* s_nxt, WaveState& ws, float c, int kh,
                                               int qi, int hh, int pm) {
  const float mu = ws.m == -INFINITY ? 0.0f : ws.m;
  bf16x8 pb[4];
  float l = ws.l;
  // -- S(n+1): the two 32-key sub-tiles of this wave's half
  s_nxt[0] = qk_rows<kFp8>(sKn, qf, 64 * kh + pm, hh, (floatx16){0});
  s_nxt[1] = qk_rows<kFp8>(sKn, qf, 64 * kh + 32 + pm, hh, (floatx16){0});
  exp_subtile(s_cur[0], c, mu, l, pb[0], pb[1]);
  if constexpr (!kFp8) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
  } else {
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    }
  }
  // -- O += P V for this half's 64 keys, with the second sub-tile's exps
  exp_subtile(s_cur[1], c, mu, l, pb[2], pb[3]);
  const int xv = (8 * kh) ^ hh;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int drow = 32 * dt + qi;
      const bf16x8 av =
          *reinterpret_cast<const bf16x8*>(&sV[drow * 16 + ((2 * u) ^ xv ^ swz(drow))]);
      ws.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[u], ws.o[dt], 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
  ws.l = l;
}

// S^T sub-tiles of this wave's 64 keys of one K tile (prologue only).
template <bool kFp8>
__device__ __forceinline__ void qk_tile(const uint4* sK, const QFrag<kFp8>& qf, floatx16* s,
                                        int kh, int hh, int pm) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) s[kt] = qk_rows<kFp8>(sK, qf, 64 * kh + 32 * kt + pm, hh, (floatx16){0});
}

// Direct-to-LDS tile loads.  bf16 K and V^T rows are 256 B (16 chunks of
// 16 B): wave w moves row quads 4w .. 4w+3, lane l filling slot l%16 of row
// 16w + 4e + l/16 with the global chunk (l%16) ^ swz(row).  e4m3 K rows are
// 128 B: wave w moves row octets 2w, 2w+1, lane l filling slot l%8 of row
// 16w + 8e + l/8 with chunk (l%8) ^ swz8(row).  The per-lane byte offsets
// are fixed for the whole workgroup; only the uniform tile base moves with
// the key block.
template <bool kFp8>
struct TileLoader {
  static constexpr int kEsz = kFp8 ? 1 : 2;
  static constexpr int kKLoads = kFp8 ? 2 : 4;  // K loads per wave per tile
  const uint8_t* kbase;  // K of kv head g
  const uint8_t* vbase;  // V^T rows of kv head g
  int64_t k_tile;        // bytes between consecutive key blocks of K
  int64_t k_st;
  uint32_t koff[kKLoads], voff[4];
  int krow[kKLoads], kchunk[kKLoads];
  int L;

  __device__ __forceinline__ void init(const AttnArgs& a, int g, int w, int lane) {
    kbase = a.k + (int64_t)g * a.k_sh * kEsz;
    vbase = reinterpret_cast<const uint8_t*>(a.vt) + (int64_t)g * 128 * a.Lpad * 2;
    k_tile = (int64_t)128 * a.k_st * kEsz;
    k_st = a.k_st;
    L = a.L;
#pragma unroll
    for (int e = 0; e < kKLoads; ++e) {
      if constexpr (!kFp8) {
        krow[e] = 16 * w + 4 * e + (lane >> 4);
        kchunk[e] = (lane & 15) ^ swz(krow[e]);
      } else {
        krow[e] = 16 * w + 8 * e + (lane >> 3);
        kchunk[e] = (lane & 7) ^ swz8(krow[e]);
      }
      koff[e] = (uint32_t)(krow[e] * a.k_st * kEsz + kchunk[e] * 16);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * w + 4 * e + (lane >> 4);
      voff[e] = (uint32_t)((int64_t)row * a.Lpad * 2 + ((lane & 15) ^ swz(row)) * 16);
    }
  }
  __device__ __forceinline__ void load_k(uint4* sK, int j, int w) const {
    const uint8_t* base = kbase + (int64_t)j * k_tile;
    if (j * 128 + 128 <= L) {
#pragma unroll
      for (int e = 0; e < kKLoads; ++e)
        __builtin_amdgcn_global_load_lds(base + koff[e], (lds_ptr_t)(sK + (kKLoads * w + e) * 64),
                                         16, 0, 0);
    } else {  // ragged last block: rows past L repeat row L-1 (masked later)
#pragma unroll
      for (int e = 0; e < kKLoads; ++e) {
        const int r = min(krow[e], L - 1 - j * 128);
        __builtin_amdgcn_global_load_lds(base + (int64_t)r * k_st * kEsz + kchunk[e] * 16,
                                         (lds_ptr_t)(sK + (kKLoads * w + e) * 64), 16, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void load_v(uint4* sV, int j, int w) const {
    const uint8_t* base = vbase + (int64_t)j * 256;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      __builtin_amdgcn_global_load_lds(base + voff[e], (lds_ptr_t)(sV + (4 * w + e) * 64), 16, 0, 0);
  }
};

#define FP_WAIT_VMEM() __builtin_amdgcn_s_waitcnt(0x0F70) /* vmcnt(0) */

template <bool kFp8>
__global__ __launch_bounds__(512) void attn_d128_kernel(AttnArgs a) {
  // K tile m lives in sK[m & 1], V^T tile m in sV[m & 1]; K runs one tile
  // ahead of V because S(n+1) = K(n+1) Q^T is issued before P(n) V(n).
  __shared__ uint4 sK0[kTileU4], sK1[kTileU4];
  __shared__ uint4 sV0[kTileU4], sV1[kTileU4];

  int h, i;
  work_item(blockIdx.x, a.nb, a.Hq, a.Hkv, h, i);
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int qg = w & 3;
  const int kh = w >> 2;
  const int qi = lane & 31;
  const int hh = lane >> 5;
  const int tq = i * 128 + 32 * qg + qi;
  const int pm = (qi & 0x13) | ((qi & 4) << 1) | ((qi & 8) >> 1);
  const float c = a.scale_log2;

  const int cnt = a.counts[(int64_t)h * a.nb + i];
  const int* lst = a.indices + fpk::tri_offset(h, i, a.nb);

  // The kept list is read 64 entries at a time into one VGPR (lane e holds
  // entry base + e) and entries are taken with readlane: no per-tile memory
  // wait, so in-flight tile prefetches are never drained for an index.
  int win = lst[min(lane, cnt - 1)];
  int wbase = 0;
  auto entry = [&](int n) -> int {
    if (n - wbase >= 64) {
      wbase += 64;
      win = lst[min(wbase + lane, cnt - 1)];
    }
    return __builtin_amdgcn_readlane(win, n - wbase);
  };

  TileLoader<kFp8> ld;
  ld.init(a, g, w, lane);

  // B operand of S^T = K Q^T for query row tq
  QFrag<kFp8> qf;
  if constexpr (!kFp8) {
    if (tq < a.L) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)tq * a.q_st +
                           (int64_t)h * a.q_sh + 8 * hh;
#pragma unroll
      for (int s = 0; s < 8; ++s) qf.f[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) qf.f[s] = (bf16x8){0, 0, 0, 0, 0, 0, 0, 0};
    }
  } else {
#pragma unroll
    for (int s = 0; s < 2; ++s) qf.f[s] = (intx8){0, 0, 0, 0, 0, 0, 0, 0};
    if (tq < a.L) {
      const uint8_t* qp = a.q + (int64_t)tq * a.q_st + (int64_t)h * a.q_sh + 32 * hh;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint4 lo = *reinterpret_cast<const uint4*>(qp + 64 * s);
        const uint4 hi = *reinterpret_cast<const uint4*>(qp + 64 * s + 16);
        qf.f[s] = (intx8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                          (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
  }

  // prologue: K(0), K(1), V(0), V(1) in; S(0); then K(2) on its way
  int j0 = entry(0);
  int j1 = cnt > 1 ? entry(1) : 0;
  int j2 = cnt > 2 ? entry(2) : 0;
  ld.load_k(sK0, j0, w);
  ld.load_v(sV0, j0, w);
  if (cnt > 1) {
    ld.load_k(sK1, j1, w);
    ld.load_v(sV1, j1, w);
  }
  WaveState ws;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) ws.o[dt] = (floatx16){0};
  ws.m = -INFINITY;
  ws.l = 0.f;
  FP_WAIT_VMEM();
  __syncthreads();
  floatx16 sA[2], sB[2];
  qk_tile<kFp8>(sK0, qf, sA, kh, hh, pm);
  __syncthreads();
  if (cnt > 2) ld.load_k(sK0, j2, w);

  // Step n (tiles n and n+1 live in the S registers and K buffers):
  //   mask/max/rescale of S(n); S(n+1) || exp(S(n)); O += P(n) V(n);
  //   wait + barrier; prefetch K(n+3) into K(n+1)'s buffer, V(n+2) into V(n)'s.
  // Two steps per trip so buffer and register roles are static.
  for (int n = 0; n < cnt; n += 2) {
    softmax_stats(sA, ws, c, j0 == i, qg, kh, qi, hh);
    pipelined_step<kFp8>(sK1, sV0, qf, sA, sB, ws, c, kh, qi, hh, pm);
    FP_WAIT_VMEM();
    __syncthreads();
    {
      const int j3 = n + 3 < cnt ? entry(n + 3) : 0;
      if (n + 3 < cnt) ld.load_k(sK1, j3, w);
      if (n + 2 < cnt) ld.load_v(sV0, j2, w);
      j0 = j1;
      j1 = j2;
      j2 = j3;
    }
    if (n + 1 >= cnt) break;
    softmax_stats(sB, ws, c, j0 == i, qg, kh, qi, hh);
    pipelined_step<kFp8>(sK0, sV1, qf, sB, sA, ws, c, kh, qi, hh, pm);
    FP_WAIT_VMEM();
    __syncthreads();
    {
      const int j3 = n + 4 < cnt ? entry(n + 4) : 0;
      if (n + 4 < cnt) ld.load_k(sK0, j3, w);
      if (n + 3 < cnt) ld.load_v(sV1, j2, w);
      j0 = j1;
      j1 = j2;
      j2 = j3;
    }
  }

  // merge the two key halves of each query group through LDS
  float* mrg = reinterpret_cast<float*>(sK0);  // [qg][66][64] floats over sK0..sV1
  if (kh == 1) {
    float* dst = mrg + qg * 66 * 64;
    dst[lane] = ws.m;
    dst[64 + lane] = ws.l;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(2 + 16 * dt + r) * 64 + lane] = ws.o[dt][r];
  }
  __syncthreads();
  if (kh == 1) return;
  const float* src = mrg + qg * 66 * 64;
  const float m1 = src[lane];
  const float l1 = src[64 + lane] + src[64 + (lane ^ 32)];
  const float l0 = ws.l + __shfl_xor(ws.l, 32);
  const float m = fmaxf(ws.m, m1);
  const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ws.m - m);
  const float a1 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
  const float inv = a.out_scale / (l0 * a0 + l1 * a1);
  if (tq < a.L) {
    uint16_t* op = a.out + (int64_t)tq * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * dt + 8 * q4 + 4 * hh;
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e;
          const float v = (ws.o[dt][r] * a0 + src[(2 + 16 * dt + r) * 64 + lane] * a1) * inv;
          b[e] = fpk::f32_to_bf16_bits(v);
        }
        *reinterpret_cast<uint2*>(op + d0) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
      }
  }
}

}  // namespace

hipError_t fpk_launch_attn_mfma(const fp_problem& p, const FpDims& dm, const int* counts,
                                const int* indices, const uint16_t* v_t, float sm_scale,
                                hipStream_t st) {
  AttnArgs a;
  a.q = static_cast<const uint8_t*>(p.q);
  a.k = static_cast<const uint8_t*>(p.k);
  a.vt = v_t;
  a.out = static_cast<uint16_t*>(p.out);
  a.counts = counts;
  a.indices = indices;
  a.q_st = p.q_stride_tok;
  a.q_sh = p.q_stride_head;
  a.k_st = p.k_stride_tok;
  a.k_sh = p.k_stride_head;
  a.o_st = p.o_stride_tok;
  a.o_sh = p.o_stride_head;
  a.L = dm.L;
  a.Hq = dm.Hq;
  a.Hkv = dm.Hkv;
  a.nb = dm.nb;
  a.Lpad = dm.nb * dm.B;
  const bool fp8 = p.dtype == FP_FP8_E4M3;
  a.scale_log2 = sm_scale * (fp8 ? p.q_scale * p.k_scale : 1.0f) * 1.4426950408889634f;
  a.out_scale = fp8 ? p.v_scale : 1.0f;
  const dim3 grid((unsigned)(dm.nb * dm.Hq));
  if (fp8)
    hipLaunchKernelGGL(attn_d128_kernel<true>, grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL(attn_d128_kernel<false>, grid, dim3(512), 0, st, a);
  return hipGetLastError();
}
