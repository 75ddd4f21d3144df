// Building blocks shared by the matrix-core attention kernels (head_dim 128,
// block 128): argument struct, work order, LDS swizzles, the softmax step
// phases and the global -> LDS tile loader.  Each kernel source includes this
// header once; everything here has internal linkage.
#pragma once

#include "common.h"
#include "varlen.h"

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
  const fpk::VlBlock* blk;  // batch metadata (varlen kernel only)
  const fpk::VlSeq* seq;
  int64_t q_st, q_sh, k_st, k_sh, o_st, o_sh;
  int L, Hq, Hkv, nb, Lpad;
  float scale_log2;  // sm_scale * log2(e) (times q_scale * k_scale for e4m3 inputs)
  float out_scale;
};

constexpr int kHalfU4 = 64 * 16;  // one half tile (64 x 256 B K, or 128 x 128 B V^T) in uint4
constexpr int kStageRow = 272;     // staged bf16 output row (256 B + 16 B pad)
static_assert(4 * 32 * kStageRow <= 4 * kHalfU4 * 16, "output staging fits in the tile buffers");
constexpr float kLazy = 8.0f;      // lazy-max slack in log2 units

// Workgroup id -> (head h, query block i).  Ids are dealt round-robin to the
// 8 XCDs (id % 8), and each XCD holds 64 workgroups at a time (32 CUs x 2).
// With 8 kv heads, XCD x takes kv group (x + t) % 8 for the 16 query blocks
// of period t (its G heads each), so the workgroups an XCD runs together
// share their kv group's K/V tiles in its L2, and the rotation spreads every
// group over all XCDs.  Heavy (late) query blocks first.  Other head layouts,
// and the rows after the last whole period, take plain row-major order.
// Long sequences (nb >= 2048, a multiple of 128) instead take the kv groups
// one after another: all XCDs work on one group (XCD x on a 16-row band of
// every 128 rows, heavy rows first), so the K/V the chip touches at a time is
// one group's, which the Infinity Cache holds (128 MiB at 256K tokens against
// 1 GiB for all eight).  Each group then spans at least 16 rounds of 512
// workgroups, so light rows still end the kernel only within each group.
constexpr int kPeriodRows = 16;
constexpr int kSeqGroupsMinBlocks = 2048;
__device__ __forceinline__ void work_item(int bid, int nb, int Hq, int Hkv, int& h, int& i) {
  const int G = Hq / Hkv;
  if (nb >= kSeqGroupsMinBlocks && nb % 128 == 0) {
    const int x = bid & 7;
    const int n = bid >> 3;
    const int per_g = nb * G / 8;  // ids of one kv group per XCD
    const int g = n / per_g;
    const int m = n - g * per_g;
    const int t = m / (16 * G);
    const int k = m - t * (16 * G);
    i = nb - 1 - (t * 128 + x * 16 + k / G);
    h = g * G + (k - (k / G) * G);
    return;
  }
  const int per = 8 * G * kPeriodRows;
  const int full = Hkv == 8 ? (nb * Hq / per) * per : 0;
  int row, grp, slot;
  if (bid < full) {
    const int x = bid & 7;
    const int n = bid >> 3;
    const int t = n / (G * kPeriodRows);
    const int k = n - t * (G * kPeriodRows);
    grp = (x + t) & 7;
    row = t * kPeriodRows + k / G;
    slot = k - (k / G) * G;
  } else {
    const int p = bid / G;
    slot = bid - p * G;
    row = p / Hkv;
    grp = p - row * Hkv;
  }
  i = nb - 1 - row;
  h = grp * G + slot;
}

__device__ __forceinline__ int swz(int row) { return (row & 15) ^ (((row >> 3) & 1) << 2); }
// 128-byte rows (e4m3 K, V^T half tiles) hold 8 chunks: the chunk XOR
// (row >> 1) & 7 sends the 16 rows one operand read touches to 16 different
// bank slots (row parity picks the 128-byte half of the 256-byte bank cycle).
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

// Lanes l and l ^ 32 hold the two 16-key halves of one query's logits:
// v_permlane32_swap exchanges the half-waves without an LDS round trip.
__device__ __forceinline__ float pair_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// Causal mask of the diagonal block: key 64hf + 32kt + 16(r/8) + 8hh + r%8
// of unit half hf is dropped for query 32qg + qi when it lies later.
__device__ __forceinline__ void mask_diag(floatx16* s, int qg, int kh, int qi, int hh) {
  // key offset 32kt + 16(r/8) + r%8 is dropped when it exceeds lim.  The
  // opaque copy keeps the compiler from hoisting the 32 comparisons out of
  // the loop as lane masks (64 scalar registers for a path taken twice per
  // row).
  int lim = 32 * qg + qi - 64 * kh - 8 * hh;
  asm volatile("" : "+v"(lim));
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int koff = 32 * kt + 16 * (r >> 3) + (r & 7);
      if (koff > lim) s[kt][r] = -INFINITY;
    }
}

__device__ __forceinline__ float tile_max(const floatx16* s) {
  float a = -INFINITY, b = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    a = fmaxf(a, fmaxf(s[0][r], s[0][r + 1]));
    b = fmaxf(b, fmaxf(s[1][r], s[1][r + 1]));
  }
  return fmaxf(a, b);
}

// Lazy raise of the running max: only when some query's tile max (mx, both
// half-waves combined, raw logits) exceeds it by more than kLazy in log2
// units are O and l rescaled.
__device__ __forceinline__ void raise_max(WaveState& ws, float mx, float c) {
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

// exp2 of one logit (scaled to log2 units, shifted by the running max).
__device__ __forceinline__ float exp_one(float v, float c, float mu) {
  return __builtin_amdgcn_exp2f(v * c - mu);
}

// One bf16 pair of P from two exponentials; the row sum takes the bf16
// values themselves (v_dot2 against (1, 1)), so l normalises exactly the
// weights that enter P.V.
__device__ __forceinline__ uint32_t pack_pair(float e0, float e1, float& l) {
  const bf16x2 pp = {(__bf16)e0, (__bf16)e1};
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  l = __builtin_amdgcn_fdot2_f32_bf16(pp, one, l, false);
  return __builtin_bit_cast(uint32_t, pp);
}

// Pins a value to this point of the instruction stream.  P(n) computed in
// phase 1 is only used by phase 2's products, after a barrier and a branch;
// without the pin the optimiser sinks those exponentials into phase 2's
// block, where they run as one long VALU stretch instead of in the gaps of
// phase 1's matrix products.
__device__ __forceinline__ uint32_t pin(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint32_t* w) {
  return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// max(a, b, c) in one v_max3_f32.  (fmaxf on matrix-core results costs an
// extra canonicalising max per operand.)  Used only on logits written by
// products issued at least eight matrix-core slots earlier, far beyond the
// matrix-to-vector read hazard distance.
__device__ __forceinline__ float max3_late(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Per-step softmax context of one wave.
struct StepCtx {
  float c, mu, l;
  uint32_t pw[4][4];  // P(n) in bf16 pairs: pw[u] is the B operand of PV slots 4u .. 4u+3
  float e_hold[2];    // first exponential of a pair whose partner comes a slot later
};

// Phase 1 of step n, in issue order: S(n+1) = K(n+1) Q^T, the two 32-key
// sub-tiles as alternating accumulation chains.  Every slot holds one MFMA
// whose LDS operand was read three slots earlier (a ring of four fragments);
// sched_barrier fences keep the slots in this order, so each LDS wait is for
// the oldest read only.  The VALU gaps carry exponentials of P(n): bf16 does
// all of sub-tile 0 and the first half of sub-tile 1 (1.5 per slot); e4m3,
// whose four products are twice as long, does sub-tile 0 (4 per slot).
template <bool kFp8>
__device__ __forceinline__ void phase1(const uint4* sKn, const QFrag<kFp8>& qf, const floatx16* s_cur,
                                       floatx16* s_nxt, StepCtx& x, int hh, int pm) {
  s_nxt[0] = (floatx16){0};
  s_nxt[1] = (floatx16){0};
  const int r0 = pm;  // sub-tile 1 is rows r0 + 32, same swizzle
  if constexpr (!kFp8) {
    const uint4* k0 = sKn + r0 * 16;
    const int xs = swz(r0) ^ hh;
    auto kread = [&](int m) -> bf16x8 {  // slot m: sub-tile m & 1, head-dim step m >> 1
      return *reinterpret_cast<const bf16x8*>(&k0[(m & 1) * 512 + ((2 * (m >> 1)) ^ xs)]);
    };
    bf16x8 ka[4];
    ka[0] = kread(0);
    ka[1] = kread(1);
    ka[2] = kread(2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m + 3 < 16) ka[(m + 3) & 3] = kread(m + 3);
      s_nxt[m & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[m & 3], qf.f[m >> 1], s_nxt[m & 1], 0, 0, 0);
      const float e = exp_one(s_cur[0][m], x.c, x.mu);
      if (m & 1) x.pw[m >> 3][(m & 7) >> 1] = pin(pack_pair(x.e_hold[0], e, x.l));
      else x.e_hold[0] = e;
      if (!(m & 1)) {
        const int v = m >> 1;  // sub-tile 1, values 0 .. 7
        const float e1 = exp_one(s_cur[1][v], x.c, x.mu);
        if (v & 1) x.pw[2][v >> 1] = pin(pack_pair(x.e_hold[1], e1, x.l));
        else x.e_hold[1] = e1;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    const uint4* k0 = sKn + r0 * 8;
    const int xs = swz8(r0);
    auto kread = [&](int m, int part) -> uint4 {  // slot m: sub-tile m & 1, 64-dim step m >> 1
      return k0[(m & 1) * 256 + ((4 * (m >> 1) + 2 * hh + part) ^ xs)];
    };
    uint4 ka[3][2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      ka[m][0] = kread(m, 0);
      ka[m][1] = kread(m, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m + 2 < 4) {
        ka[(m + 2) % 3][0] = kread(m + 2, 0);
        ka[(m + 2) % 3][1] = kread(m + 2, 1);
      }
      const uint4 lo = ka[m % 3][0], hi = ka[m % 3][1];
      const intx8 f = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      s_nxt[m & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f, qf.f[m >> 1], s_nxt[m & 1], 0, 0,
                                                                     0, 127, 0, 127);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int v = 4 * m + 2 * e;
        x.pw[v >> 3][(v & 7) >> 1] =
            pin(pack_pair(exp_one(s_cur[0][v], x.c, x.mu), exp_one(s_cur[0][v + 1], x.c, x.mu), x.l));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Phase 2 of step n: O += P(n) V(n), slot m = key group u = m >> 2 times
// head dims 32 (m & 3) .. +31.  V^T row 32 dt + qi (eight 16-byte chunks of
// 8 keys) has the same swizzle for every dt, so one address per u serves a
// group.  Slots 0-7 finish P(n)'s
// exponentials (bf16: sub-tile 1 values 8-15, ready before slot 12 reads
// them; e4m3: all of sub-tile 1, two per slot), slots 8-15 take the row max
// of S(n+1) for the next step.  Returns that max (this lane's half).
template <bool kFp8>
__device__ __forceinline__ float phase2(const uint4* sV, const floatx16* s_cur, const floatx16* s_nxt,
                                        WaveState& ws, StepCtx& x, int qi, int hh) {
  const int xv = hh ^ swz8(qi);  // swz8(32 dt + qi) == swz8(qi)
  const uint4* vr = sV + qi * 8;
  auto vread = [&](int m) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(&vr[(m & 3) * 256 + ((2 * (m >> 2)) ^ xv)]);
  };
  bf16x8 va[4];
  va[0] = vread(0);
  va[1] = vread(1);
  va[2] = vread(2);
  float mx0 = -INFINITY, mx1 = -INFINITY;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (m + 3 < 16) va[(m + 3) & 3] = vread(m + 3);
    ws.o[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[m & 3], as_bf16x8(x.pw[m >> 2]), ws.o[m & 3], 0, 0, 0);
    if (m < 8) {
      if constexpr (!kFp8) {
        const float e = exp_one(s_cur[1][8 + m], x.c, x.mu);
        if (m & 1) x.pw[3][m >> 1] = pack_pair(x.e_hold[1], e, x.l);
        else x.e_hold[1] = e;
      } else {
        x.pw[2 + (m >> 2)][m & 3] =
            pack_pair(exp_one(s_cur[1][2 * m], x.c, x.mu), exp_one(s_cur[1][2 * m + 1], x.c, x.mu), x.l);
      }
    } else {
      const int r = 2 * (m - 8);
      mx0 = max3_late(mx0, s_nxt[0][r], s_nxt[0][r + 1]);
      mx1 = max3_late(mx1, s_nxt[1][r], s_nxt[1][r + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  return fmaxf(mx0, mx1);
}

// S^T of one 64-key unit (prologue only).
template <bool kFp8>
__device__ __forceinline__ void qk_unit(const uint4* sK, const QFrag<kFp8>& qf, floatx16* s, int hh,
                                        int pm) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) s[kt] = qk_rows<kFp8>(sK, qf, 32 * kt + pm, hh, (floatx16){0});
}

// Direct-to-LDS loads of 64-key half tiles, each 16 KiB (e4m3 K: 8 KiB),
// moved as 1 KiB loads (64 lanes x 16 B) with buffer_load ... lds.
//   K: 64 rows of 256 B (16 chunks); load e of wave w fills rows
//      16w + 4e + l/16, lane l writing slot l%16 with the global chunk
//      (l%16) ^ swz(row).  e4m3 rows are 128 B (8 chunks): rows
//      16w + 8e + l/8, slot l%8 <- chunk (l%8) ^ swz8(row).
//   V^T: 128 rows (head dims) of 64 keys = 128 B (8 chunks of 8 keys);
//      load e of wave w fills rows 32w + 8e + l/8, slot l%8 <- chunk
//      (l%8) ^ swz8(row).
// The per-lane offsets are fixed for the workgroup and a unit only moves
// scalar values, so a load costs no vector address arithmetic.  K is reached
// through a buffer resource based at its key block (64-bit scalar address,
// extent up to the block's last present row), so offsets stay below one
// block's rows whatever the sequence length; V^T through one resource per kv
// head (at most 2^21 keys of 128 dims: 512 MiB).  (Buffer loads also keep
// LDS-read waits exact: while a flat or global LDS load is in flight the
// compiler can only wait for every LDS read, which would serialise the
// operand prefetch of the matrix products.)
template <bool kFp8>
struct TileLoader {
  static constexpr int kEsz = kFp8 ? 1 : 2;
  static constexpr int kKLoads = kFp8 ? 2 : 4;  // K loads per wave per unit
  const uint8_t* kg;           // K of kv head g
  __amdgpu_buffer_rsrc_t vrs;  // V^T rows of kv head g
  int64_t k_tile;              // bytes between consecutive key blocks of K
  int k_row;                   // bytes between consecutive keys
  uint32_t koff[kKLoads], voff[4];
  int L;

  // key row (of the half tile) and 16-byte chunk that K load e moves
  __device__ __forceinline__ static int krow_of(int w, int e, int lane) {
    return kFp8 ? 16 * w + 8 * e + (lane >> 3) : 16 * w + 4 * e + (lane >> 4);
  }
  __device__ __forceinline__ static int kchunk_of(int row, int lane) {
    return kFp8 ? (lane & 7) ^ swz8(row) : (lane & 15) ^ swz(row);
  }

  __device__ __forceinline__ void init(const AttnArgs& a, int g, int w, int lane) {
    k_row = (int)(a.k_st * kEsz);
    k_tile = 128 * (int64_t)k_row;
    L = a.L;
    kg = a.k + (int64_t)g * a.k_sh * kEsz;
#pragma unroll
    for (int e = 0; e < kKLoads; ++e) {
      const int row = krow_of(w, e, lane);
      koff[e] = (uint32_t)(row * k_row + kchunk_of(row, lane) * 16);
    }
    vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.vt + (int64_t)g * 128 * a.Lpad), 0, 128 * a.Lpad * 2, 0x00020000);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 32 * w + 8 * e + (lane >> 3);
      voff[e] = (uint32_t)(row * a.Lpad * 2 + ((lane & 7) ^ swz8(row)) * 16);
    }
  }
  // K half tile hf of key block j
  __device__ __forceinline__ void load_k(uint4* sK, int j, int hf, int w) const {
    const int rows = min(128, L - j * 128);  // key rows present in block j
    // A list entry outside [0, nb) (a caller-written list that breaks the
    // documented rules) gets an empty resource: its reads return zeros
    // instead of leaving the tensor.
    const int ext = (j >= 0 && rows > 0) ? (rows - 1) * k_row + 128 * kEsz : 0;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kg + j * k_tile), 0, ext, 0x00020000);
    if (64 * hf + 64 <= rows) {
#pragma unroll
      for (int e = 0; e < kKLoads; ++e)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(sK + (kKLoads * w + e) * 64), 16,
                                                 koff[e], hf * 64 * k_row, 0, 0);
    } else {  // ragged last block: rows past L repeat row L-1 (masked later)
      const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
      for (int e = 0; e < kKLoads; ++e) {
        const int row = krow_of(w, e, lane);
        const int r = min(64 * hf + row, rows - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(sK + (kKLoads * w + e) * 64), 16,
                                                 (uint32_t)(r * k_row + kchunk_of(row, lane) * 16), 0, 0,
                                                 0);
      }
    }
  }
  // Load e (0 .. kKLoads-1) of K half tile hf of key block j alone, so a
  // caller can spread one tile's loads over several instruction slots.
  __device__ __forceinline__ void load_k_one(uint4* sK, int j, int hf, int w, int e) const {
    const int rows = min(128, L - j * 128);
    const int ext = (j >= 0 && rows > 0) ? (rows - 1) * k_row + 128 * kEsz : 0;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kg + j * k_tile), 0, ext, 0x00020000);
    if (64 * hf + 64 <= rows) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(sK + (kKLoads * w + e) * 64), 16, koff[e],
                                               hf * 64 * k_row, 0, 0);
    } else {
      const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      const int row = krow_of(w, e, lane);
      const int r = min(64 * hf + row, rows - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(sK + (kKLoads * w + e) * 64), 16,
                                               (uint32_t)(r * k_row + kchunk_of(row, lane) * 16), 0, 0, 0);
    }
  }
  // Load e (0 .. 3) of V^T half tile hf of key block j alone.
  __device__ __forceinline__ void load_v_one(uint4* sV, int j, int hf, int w, int e) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(sV + (4 * w + e) * 64), 16, voff[e],
                                             j * 256 + hf * 128, 0, 0);
  }
  // V^T half tile hf of key block j (V^T is zero past L)
  __device__ __forceinline__ void load_v(uint4* sV, int j, int hf, int w) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) load_v_one(sV, j, hf, w, e);
  }
};

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8]
// | vmcnt[15:14]): wait for vector memory only.
#define FP_WAIT_VMEM() __builtin_amdgcn_s_waitcnt(0x0F70) /* vmcnt(0) */

// Workgroup barrier of the tile pipeline.  Each wave first waits until at
// most n of its own LDS-bound loads are in flight (the older group has
// landed) and all its LDS reads have returned; the barrier then makes the
// landed tile visible to every wave and lets the freed buffer be refilled.
// (__syncthreads would also drain the younger loads: its release fence waits
// for all outstanding vector memory.)  The empty asm statements keep the
// compiler from moving LDS accesses across the barrier.
template <int n>
__device__ __forceinline__ void tile_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0070 | (n & 15) | ((n >> 4) << 14)); /* vmcnt(n) lgkmcnt(0) */
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace
