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
// One workgroup = one (q head h, query block i): 4 waves, wave w owning query
// rows 32w .. 32w+31.  The kept key blocks are walked in 64-key units (two
// per block); per unit every wave computes its 32 x 64 logits and P.V over
// those 64 keys, so a wave keeps one online-softmax state for its queries
// and no cross-wave merge is needed.  A workgroup stages 16 KiB K and V^T
// half tiles (64 KiB of LDS in all), so two workgroups share a compute unit:
// their waves pair up on each SIMD and, having no barrier in common, fill
// each other's waits (barrier skew, row start-up, epilogue).
//
// Per 64-key unit (ascending list, the diagonal block last):
//   * the K half tile [64 keys][128 dims] and the V^T half tile [128 dims]
//     [64 keys] travel global -> LDS with buffer_load ... lds (no
//     registers), double buffered.  K rows are 16 chunks of 16 B stored at
//     chunk ^ f(row), f(r) = (r & 15) ^ (((r >> 3) & 1) << 2); V^T rows are
//     8 chunks stored at chunk ^ ((row >> 1) & 7).  A 16-byte LDS read is
//     served 16 lanes at a time over 64 four-byte banks; the swizzles give
//     the 16 rows such a read touches 16 different 16-byte bank slots;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: two 32-key sub-tiles, eight
//     16-wide steps over the head dimension.  A lane column is one query, so
//     a lane holds 32 of its query's logits and lane ^ 32 the rest.  K rows
//     are fed in the order pm(m) (bits 2 and 3 of m swapped), which makes
//     each lane's logits contiguous 8-key runs: the B operand of P.V as is;
//   * online softmax in the exp2 domain with a lazy maximum: the running max
//     is raised (and O, l rescaled) only when a unit's max exceeds it by more
//     than 8 (P <= 2^8 stays exact enough in bf16 and cannot overflow fp32);
//   * O^T += V^T P^T, P packed to bf16 from the S^T registers.
// The causal mask is applied on the diagonal block only.  1/l and the V
// dequantisation scale are applied once, at the end.
//
// Work order: heavy (late) query blocks first, and the workgroups one XCD
// runs together belong to one kv group (work_item below).
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
    vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.vt + (int64_t)g * 128 * a.Lpad), 0, 128 * a.Lpad * 2, 0x00020000);
#pragma unroll
    for (int e = 0; e < kKLoads; ++e) {
      const int row = krow_of(w, e, lane);
      koff[e] = (uint32_t)(row * k_row + kchunk_of(row, lane) * 16);
    }
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
  // V^T half tile hf of key block j (V^T is zero past L)
  __device__ __forceinline__ void load_v(uint4* sV, int j, int hf, int w) const {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(sV + (4 * w + e) * 64), 16, voff[e],
                                               j * 256 + hf * 128, 0, 0);
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

template <bool kFp8, bool kVarlen>
__global__ __launch_bounds__(256, 2) void attn_d128_kernel(AttnArgs a) {  // 2 waves per SIMD: two workgroups per CU
  // K unit m lives in sK[m & 1], V^T unit m in sV[m & 1]; K runs one unit
  // ahead of V because S(n+1) = K(n+1) Q^T is issued before P(n) V(n).
  __shared__ uint4 smem[4 * kHalfU4];
  uint4* const sK0 = smem;
  uint4* const sK1 = smem + kHalfU4;
  uint4* const sV0 = smem + 2 * kHalfU4;
  uint4* const sV1 = smem + 3 * kHalfU4;

  int h, i;
  work_item(blockIdx.x, a.nb, a.Hq, a.Hkv, h, i);
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // = query group
  const int qi = lane & 31;
  const int hh = lane >> 5;
  // Tokens of block i in q / out, and its list.  One sequence: block i is
  // tokens 128 i .. and row (h, i) of the triangle.  A batch (varlen): block
  // i of the batch is block li of its sequence, which starts at block
  // `first`; list entries are local to the sequence.
  int tok0 = i * 128, rows = min(128, a.L - i * 128), li = i, first = 0;
  const int* lst = a.indices + fpk::tri_offset(h, i, a.nb);
  if constexpr (kVarlen) {
    const fpk::VlBlock m = a.blk[i];
    const fpk::VlSeq sq = a.seq[m.seq];
    tok0 = m.tok0;
    rows = m.rows;
    li = m.jl;
    first = sq.first;
    lst = a.indices + sq.idx_base + (int64_t)h * sq.nb * (sq.nb + 1) / 2 + (int64_t)li * (li + 1) / 2;
  }
  const int tq = tok0 + 32 * w + qi;
  const bool q_valid = 32 * w + qi < rows;
  const int pm = (qi & 0x13) | ((qi & 4) << 1) | ((qi & 8) >> 1);
  const float c = a.scale_log2;

  const int cnt = a.counts[(int64_t)h * a.nb + i];

  // The kept list is read 64 entries at a time into one VGPR (lane e holds
  // entry base + e) and entries are taken with readlane: no per-unit memory
  // wait, so in-flight tile prefetches are never drained for an index.  The
  // window is read through a buffer resource bounded by the row's capacity
  // (i + 1 entries; reads past it return 0), so the first window does not
  // wait for the count: both loads are in flight together.  Entries at or
  // past the count are never selected.
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int*>(lst), 0, (li + 1) * 4, 0x00020000);
  int win = (int)__builtin_amdgcn_raw_buffer_load_b32(lrs, lane * 4, 0, 0);
  int wbase = 0;
  auto entry = [&](int n) -> int {
    if (n - wbase >= 64) {  // rare: wait right here, so no wait sits on the common path
      wbase += 64;
      win = (int)__builtin_amdgcn_raw_buffer_load_b32(lrs, (wbase + lane) * 4, 0, 0);
      FP_WAIT_VMEM();
    }
    return __builtin_amdgcn_readlane(win, n - wbase) + first;
  };

  TileLoader<kFp8> ld;
  ld.init(a, g, w, lane);

  // B operand of S^T = K Q^T for query row tq
  QFrag<kFp8> qf;
  if constexpr (!kFp8) {
    if (q_valid) {
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
    if (q_valid) {
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

  // Units: u = 0 .. 2 cnt - 1, unit u = half u & 1 of block list[u >> 1].
  // Load schedule.  Buffers: K(m) in sK[m & 1], V(m) in sV[m & 1].  Step n
  // computes S(n+1) from K(n+1) (phase 1) and O += P(n) V(n) (phase 2):
  //   after phase 1, a barrier frees K(n+1)'s buffer and K(n+3) is issued;
  //   after phase 2, a barrier frees V(n)'s buffer and V(n+2) is issued.
  // Each load thus has one and a half steps to land.  Loads go out in the
  // order ... K(n+2), V(n+1), K(n+3), V(n+2) ..., so before each barrier
  // the wait leaves the two younger groups in flight (vmcnt(kK + kV)); near
  // the end of the list, where fewer groups are in flight, it waits for all.
  constexpr int kK = TileLoader<kFp8>::kKLoads;
  const int ucnt = 2 * cnt;
  // block of units u, u+1, u+2 (two units per block: units 2b and 2b + 1)
  int j0 = entry(0);  // block of unit 0 and unit 1
  int j2 = cnt > 1 ? entry(1) : 0;  // block of units 2 and 3
  ld.load_k(sK0, j0, 0, w);
  ld.load_v(sV0, j0, 0, w);
  ld.load_k(sK1, j0, 1, w);
  WaveState ws;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) ws.o[dt] = (floatx16){0};
  ws.m = -INFINITY;
  ws.l = 0.f;
  FP_WAIT_VMEM();
  __syncthreads();
  floatx16 sA[2], sB[2];
  qk_unit<kFp8>(sK0, qf, sA, hh, pm);
  __syncthreads();
  if (ucnt > 2) ld.load_k(sK0, j2, 0, w);  // unit 2 (issued as step -1's phase-1 load)
  ld.load_v(sV1, j0, 1, w);                // unit 1 (and as its phase-2 load)
  if (j0 == i) mask_diag(sA, w, 0, qi, hh);
  float mx = pair_max(tile_max(sA));

  // blocks of the units around step t: jb[0] = block of unit t, ...
  // (t even: units t, t+1 share block jc; t+2, t+3 share block jn)
  int jc = j0;   // block of units t and t+1 when t is even
  int jn = j2;   // block of units t+2 and t+3
  StepCtx x;
  x.c = c;
  // Two steps (= one key block) per trip so buffer and register roles are
  // static: half 0 is the block's first unit, half 1 its second.
  for (int n = 0; n < ucnt; n += 2) {
    int jn2 = 0;  // block of units n+4, n+5
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int t = n + half;  // this step's unit
      floatx16* s_cur = half == 0 ? sA : sB;
      floatx16* s_nxt = half == 0 ? sB : sA;
      uint4* sKn = half == 0 ? sK1 : sK0;
      uint4* sVc = half == 0 ? sV0 : sV1;
      raise_max(ws, mx, c);
      x.mu = ws.m == -INFINITY ? 0.0f : ws.m;
      x.l = ws.l;
      phase1<kFp8>(sKn, qf, s_cur, s_nxt, x, hh, pm);
      // V(t) must have landed; K(t+2) and V(t+1) may still be in flight
      if (t + 2 < ucnt) tile_barrier<kK + 4>();
      else tile_barrier<0>();
      // K(t+3): unit t+3 is half (t+3)&1 of block (t+3)>>1
      if (t + 3 < ucnt) {
        if (half == 0) ld.load_k(sKn, jn, 1, w);  // t even: unit t+3 = second half of jn
        else {
          jn2 = entry((t + 3) >> 1);  // t odd: unit t+3 = first half of the block after jn
          ld.load_k(sKn, jn2, 0, w);
        }
      }
      // The two waves sharing a SIMD come from different workgroups; raising
      // the issue priority of the matrix-heavy phase 2 lets the other wave's
      // VALU-heavy phase 1 fill its gaps rather than compete for them.
      __builtin_amdgcn_s_setprio(2);
      mx = phase2<kFp8>(sVc, s_cur, s_nxt, ws, x, qi, hh);
      __builtin_amdgcn_s_setprio(0);
      ws.l = x.l;
      // S(t+1) belongs to unit t+1: block jc (t even) or jn (t odd)
      const int jnext = half == 0 ? jc : jn;
      if (t + 1 < ucnt && jnext == i) {
        mask_diag(s_nxt, w, half == 0 ? 1 : 0, qi, hh);
        mx = tile_max(s_nxt);
      }
      mx = pair_max(mx);
      // K(t+2) must have landed; V(t+1) and K(t+3) may still be in flight
      if (t + 3 < ucnt) tile_barrier<kK + 4>();
      else tile_barrier<0>();
      // V(t+2): unit t+2 is half t&1 of block jn
      if (t + 2 < ucnt) ld.load_v(sVc, jn, half, w);
    }
    jc = jn;
    jn = jn2;
  }

  // Normalise and write out.  A lane holds 4-dim pieces of one token; stored
  // directly, every store instruction would touch 32 tokens one output row
  // apart.  The bf16 rows of this wave's 32 tokens are staged in LDS
  // (272-byte rows: 16-byte aligned, neighbouring rows on different banks,
  // over the tile buffers, which the last barrier has released) and written
  // back as whole 256-byte head slices, four tokens per 1 KiB store.
  const float l = ws.l + __shfl_xor(ws.l, 32);
  const float inv = a.out_scale / l;
  uint8_t* stg = reinterpret_cast<uint8_t*>(smem) + w * 32 * kStageRow;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * hh;
      const int r = 4 * q4;
      // v_cvt_pk_bf16_f32: round to nearest even, branch free
      const bf16x2 p01 = {(__bf16)(ws.o[dt][r] * inv), (__bf16)(ws.o[dt][r + 1] * inv)};
      const bf16x2 p23 = {(__bf16)(ws.o[dt][r + 2] * inv), (__bf16)(ws.o[dt][r + 3] * inv)};
      *reinterpret_cast<uint2*>(stg + qi * kStageRow + 2 * d0) =
          make_uint2(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23));
    }
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int ch = it * 64 + lane;  // 16-byte chunk: token ch / 16, piece ch % 16
    const int tok = ch >> 4;
    const uint4 v = *reinterpret_cast<const uint4*>(stg + tok * kStageRow + (ch & 15) * 16);
    const int t = tok0 + 32 * w + tok;
    if (32 * w + tok < rows)
      *reinterpret_cast<uint4*>(a.out + (int64_t)t * a.o_st + (int64_t)h * a.o_sh + (ch & 15) * 8) = v;
  }
}

// Explicit instantiations: the launchers below name these variants from
// outside the unnamed namespace.
template __global__ void attn_d128_kernel<false, false>(AttnArgs);
template __global__ void attn_d128_kernel<true, false>(AttnArgs);
template __global__ void attn_d128_kernel<false, true>(AttnArgs);
template __global__ void attn_d128_kernel<true, true>(AttnArgs);

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
    hipLaunchKernelGGL((attn_d128_kernel<true, false>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_d128_kernel<false, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t fpk_launch_attn_mfma_varlen(const fp_problem& p, const FpDims& dm, int NB, const fpk::VlBlock* blk,
                                       const fpk::VlSeq* seq, const int* counts, const int* indices,
                                       const uint8_t* k_c, const uint16_t* v_t, float sm_scale, hipStream_t st) {
  // K is read from the gathered copy [Hkv][NB * 128][128]: full blocks, rows
  // past a sequence's end zero (the causal mask of the diagonal block hides
  // them), so the loader never takes its ragged path.
  AttnArgs a{};
  a.q = static_cast<const uint8_t*>(p.q);
  a.k = k_c;
  a.vt = v_t;
  a.out = static_cast<uint16_t*>(p.out);
  a.counts = counts;
  a.indices = indices;
  a.blk = blk;
  a.seq = seq;
  a.q_st = p.q_stride_tok;
  a.q_sh = p.q_stride_head;
  a.k_st = 128;
  a.k_sh = (int64_t)NB * 128 * 128;
  a.o_st = p.o_stride_tok;
  a.o_sh = p.o_stride_head;
  a.L = NB * 128;
  a.Hq = dm.Hq;
  a.Hkv = dm.Hkv;
  a.nb = NB;
  a.Lpad = NB * 128;
  const bool fp8 = p.dtype == FP_FP8_E4M3;
  a.scale_log2 = sm_scale * (fp8 ? p.q_scale * p.k_scale : 1.0f) * 1.4426950408889634f;
  a.out_scale = fp8 ? p.v_scale : 1.0f;
  const dim3 grid((unsigned)(NB * dm.Hq));
  if (fp8)
    hipLaunchKernelGGL((attn_d128_kernel<true, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_d128_kernel<false, true>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
