// Step 5 on the matrix cores with two query heads of one kv group per wave
// (bf16, head_dim 128, block 128, Hq/Hkv even).
//
// FlashPrefill V2 abstract (PackGQA: the query heads of one kv group share
// the K/V tiles they read) on the block-sparse attention of the FlashPrefill
// skill page ("Architecture Overview": only the listed key blocks are
// visited; "Implementation Steps": block-sparse attention over the kept
// blocks).  Every head keeps its own list and its own result: the kernel
// walks the union of the two heads' ascending lists, and a block that only
// one head lists has the other head's logits set to -inf (its weights are
// exactly zero), so each head attends over exactly its own blocks.
//
// One workgroup = (head pair, query block): 4 waves, one per SIMD, wave w
// owning query rows 32w .. 32w+31 of BOTH heads.  Per 64-key unit a wave
// runs 32 products for S^T = K Q^T (two heads x two 32-key sub-tiles x eight
// 16-wide head-dim steps) and 32 for O^T += V^T P^T (two heads x four 32-dim
// tiles x four 16-key steps).  Each K or V^T fragment read from LDS feeds
// both heads' products, so a product costs half the LDS operand bytes of the
// one-head kernel (attn_mfma.hip), and each K/V tile is staged once for 256
// query rows instead of 128.  The price is registers: both heads' Q
// fragments, logits of two units and output accumulators need more than the
// 256 a wave may hold at two waves per SIMD, so this kernel runs one wave per
// SIMD (one workgroup per compute unit) and hides latency inside the wave:
// the products of one phase carry the other phase's exponentials and maxima
// in their gaps, slot by slot, exactly as the one-head kernel does.
//
// The tile pipeline (double-buffered K and V^T half tiles, buffer loads
// straight into LDS, two barriers per unit with partial vmcnt waits), the
// swizzles, the lazy online softmax and the output staging are those of the
// one-head kernel; see attn_mfma.hip and attn_common.h.
#include "attn_common.h"

namespace {

// Register-file placement hints.  An empty asm statement whose operand must
// sit in the accumulation registers ("a") or the vector registers ("v") makes
// the allocator keep the value there: the output accumulators and Q in the
// accumulation file (only matrix products read them), the logits in the
// vector file (the exponentials read them), so no copies between the two
// files sit in the step.
__device__ __forceinline__ void in_agpr(floatx16& v) { asm volatile("" : "+a"(v)); }
__device__ __forceinline__ void in_agpr(bf16x8& v) { asm volatile("" : "+a"(v)); }
__device__ __forceinline__ void in_vgpr(floatx16& v) { asm volatile("" : "+v"(v)); }

// S^T chain steps with the logits kept in the vector registers: acc = K Q^T
// (first step) or acc += K Q^T, K from the vector registers (an LDS
// fragment), Q from the accumulation registers.  Written as asm because the
// allocator otherwise keeps every matrix-product result of this kernel in the
// accumulation file and copies the logits out and back for the softmax (about
// 300 copies per step).  Hazards: the logits are read by vector instructions
// only in the next phase, at least sixteen products later; the products of
// one chain are four products apart and accumulate in place (the
// exactly-overlapping accumulation the matrix cores chain back to back).
__device__ __forceinline__ floatx16 qk_first(const bf16x8& k, const bf16x8& q) {
  floatx16 d;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "a"(q));
  return d;
}
__device__ __forceinline__ void qk_acc(floatx16& d, const bf16x8& k, const bf16x8& q) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
}

// Softmax context of one wave for its two heads.
struct Step2 {
  float c;
  float mu[2];
  float l[2];
  uint32_t pw[2][4][4];  // P(n) of head x in bf16 pairs: pw[x][u] feeds PV slots 4u .. 4u+3
  float e_hold[2][2];
};

// Phase 1 of step n for both heads: S_x(n+1) = K(n+1) Q_x^T.  Slot m reads
// K fragment (sub-tile m & 1, head-dim step m >> 1) three slots ahead and
// issues head a's and head b's products with it; the gaps carry 1.5
// exponentials of P(n) per head (sub-tile 0 whole, sub-tile 1 first half).
__device__ __forceinline__ void phase1_2h(const uint4* sKn, const QFrag<false>& qa, const QFrag<false>& qb,
                                          const floatx16* sa_cur, const floatx16* sb_cur, floatx16* sa_nxt,
                                          floatx16* sb_nxt, Step2& x, int hh, int pm) {
  const uint4* k0 = sKn + pm * 16;
  const int xs = swz(pm) ^ hh;
  auto kread = [&](int m) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(&k0[(m & 1) * 512 + ((2 * (m >> 1)) ^ xs)]);
  };
  auto exps = [&](int hd, const floatx16* s, int m) {
    const float e = exp_one(s[0][m], x.c, x.mu[hd]);
    if (m & 1) x.pw[hd][m >> 3][(m & 7) >> 1] = pin(pack_pair(x.e_hold[hd][0], e, x.l[hd]));
    else x.e_hold[hd][0] = e;
    if (!(m & 1)) {
      const int v = m >> 1;  // sub-tile 1, values 0 .. 7
      const float e1 = exp_one(s[1][v], x.c, x.mu[hd]);
      if (v & 1) x.pw[hd][2][v >> 1] = pin(pack_pair(x.e_hold[hd][1], e1, x.l[hd]));
      else x.e_hold[hd][1] = e1;
    }
  };
  bf16x8 ka[4];
  ka[0] = kread(0);
  ka[1] = kread(1);
  ka[2] = kread(2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (m + 3 < 16) ka[(m + 3) & 3] = kread(m + 3);
    if (m < 2) sa_nxt[m] = qk_first(ka[m & 3], qa.f[0]);
    else qk_acc(sa_nxt[m & 1], ka[m & 3], qa.f[m >> 1]);
    exps(0, sa_cur, m);
    // half slots: each product carries one head's vector work, so the work
    // fits in the product's shadow instead of piling up before the first one
    __builtin_amdgcn_sched_barrier(0);
    if (m < 2) sb_nxt[m] = qk_first(ka[m & 3], qb.f[0]);
    else qk_acc(sb_nxt[m & 1], ka[m & 3], qb.f[m >> 1]);
    exps(1, sb_cur, m);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Phase 2 of step n for both heads: O_x += P_x(n) V(n).  Slot m reads V^T
// fragment (head-dim tile m & 3, key group m >> 2) and issues both heads'
// products with it.  Slots 0-7 finish P(n) (sub-tile 1, values 8-15, needed
// from slot 12 on), slots 8-15 take the row maxima of S_x(n+1).  Returns
// this lane's half of both maxima.
template <class Issue>
__device__ __forceinline__ void phase2_2h(const uint4* sV, const floatx16* sa_cur, const floatx16* sb_cur,
                                          const floatx16* sa_nxt, const floatx16* sb_nxt, floatx16 (*o)[4],
                                          Step2& x, int qi, int hh, float* mx, const Issue& issue) {
  const int xv = hh ^ swz8(qi);
  const uint4* vr = sV + qi * 8;
  auto vread = [&](int m) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(&vr[(m & 3) * 256 + ((2 * (m >> 2)) ^ xv)]);
  };
  bf16x8 va[4];
  va[0] = vread(0);
  va[1] = vread(1);
  va[2] = vread(2);
  float mx0[2] = {-INFINITY, -INFINITY}, mx1[2] = {-INFINITY, -INFINITY};
  auto tail = [&](int hd, const floatx16* s_cur, const floatx16* s_nxt, int m) {
    if (m < 8) {
      const float e = exp_one(s_cur[1][8 + m], x.c, x.mu[hd]);
      if (m & 1) x.pw[hd][3][m >> 1] = pack_pair(x.e_hold[hd][1], e, x.l[hd]);
      else x.e_hold[hd][1] = e;
    } else {
      const int r = 2 * (m - 8);
      mx0[hd] = max3_late(mx0[hd], s_nxt[0][r], s_nxt[0][r + 1]);
      mx1[hd] = max3_late(mx1[hd], s_nxt[1][r], s_nxt[1][r + 1]);
    }
  };
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (m < 8) issue(m);  // the step's tile loads, one per slot
    if (m + 3 < 16) va[(m + 3) & 3] = vread(m + 3);
    o[0][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[m & 3], as_bf16x8(x.pw[0][m >> 2]), o[0][m & 3], 0, 0, 0);
    tail(0, sa_cur, sa_nxt, m);
    __builtin_amdgcn_sched_barrier(0);
    o[1][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[m & 3], as_bf16x8(x.pw[1][m >> 2]), o[1][m & 3], 0, 0, 0);
    tail(1, sb_cur, sb_nxt, m);
    __builtin_amdgcn_sched_barrier(0);
  }
  mx[0] = fmaxf(mx0[0], mx1[0]);
  mx[1] = fmaxf(mx0[1], mx1[1]);
}

// o *= alpha in place in the accumulation registers, one register at a time
// through a vector temporary.  (A plain multiply gives the accumulators a
// vector-register home, and the allocator then copies part of them out and
// back on every step, whether or not the rare rescale runs.)
__device__ __forceinline__ void scale_acc(floatx16& o, float alpha) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float e = o[r];
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %2, %1\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(e), "=&v"(t)
                 : "v"(alpha));
    o[r] = e;
  }
}

// Lazy raise of one head's running max (see raise_max in attn_common.h).
__device__ __forceinline__ void raise_max_h(floatx16* o, float& m, float& l, float mx, float c) {
  const float mxs = mx * c;
  if (__any(mxs > m + kLazy)) {
    // The last products that wrote o were issued in the previous phase 2,
    // possibly only a few instructions ago: 16 wait states before the
    // accumulation registers are read (a matrix-core result needs at most 11
    // before a vector read on this chip).
    asm volatile("s_nop 7\n\ts_nop 7");
    const float m_new = fmaxf(m, mxs);
    const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) scale_acc(o[dt], alpha);
  }
}

// Logits of a head that does not list the unit's block: exactly -inf, so its
// weights are exactly zero.
__device__ __forceinline__ void drop_unit(floatx16* s) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kt][r] = -INFINITY;
}

// Ascending list of one head, read 64 entries at a time into one VGPR (lane
// e holds entry base + e) and taken with readlane, as in the one-head kernel.
struct ListCursor {
  __amdgpu_buffer_rsrc_t rs;
  int win, base, pos, cnt;
};

__device__ __forceinline__ void cursor_init(ListCursor& c, const int* lst, int cap, int cnt, int lane) {
  c.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int*>(lst), 0, cap * 4, 0x00020000);
  c.win = (int)__builtin_amdgcn_raw_buffer_load_b32(c.rs, lane * 4, 0, 0);
  c.base = 0;
  c.pos = 0;
  c.cnt = cnt;
}

// Entry at the cursor, or INT_MAX past the end.
__device__ __forceinline__ int cursor_peek(ListCursor& c, int lane) {
  if (c.pos >= c.cnt) return 0x7fffffff;
  if (c.pos - c.base >= 64) {  // rare: wait right here, so no wait sits on the common path
    c.base += 64;
    c.win = (int)__builtin_amdgcn_raw_buffer_load_b32(c.rs, (c.base + lane) * 4, 0, 0);
    FP_WAIT_VMEM();
  }
  return __builtin_amdgcn_readlane(c.win, c.pos - c.base);
}

// Next block of the union of both lists and which heads list it (bit 0: head
// a, bit 1: head b).  False once both lists are exhausted.
__device__ __forceinline__ bool union_next(ListCursor& A, ListCursor& B, int lane, int& j, int& fl) {
  const int ea = cursor_peek(A, lane);
  const int eb = cursor_peek(B, lane);
  j = min(ea, eb);
  if (j == 0x7fffffff) return false;
  fl = (ea == j ? 1 : 0) | (eb == j ? 2 : 0);
  A.pos += ea == j ? 1 : 0;
  B.pos += eb == j ? 1 : 0;
  return true;
}

__global__ __launch_bounds__(256, 1) void attn_pack_kernel(AttnArgs a) {  // 1 wave per SIMD
  // Three K and three V^T half-tile buffers: unit t's K lives in sK[t % 3],
  // its V^T in sV[t % 3] (96 KiB; one workgroup per compute unit).
  __shared__ uint4 smem[6 * kHalfU4];
  uint4* const sK = smem;
  uint4* const sV = smem + 3 * kHalfU4;

  int hp, i;
  work_item(blockIdx.x, a.nb, a.Hq / 2, a.Hkv, hp, i);  // head pairs take the place of heads
  const int ha = 2 * hp;
  const int g = ha / (a.Hq / a.Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = lane & 31;
  const int hh = lane >> 5;
  const int tok0 = i * 128;
  const int rows = min(128, a.L - tok0);
  const int tq = tok0 + 32 * w + qi;
  const bool q_valid = 32 * w + qi < rows;
  const int pm = (qi & 0x13) | ((qi & 4) << 1) | ((qi & 8) >> 1);
  const float c = a.scale_log2;

  ListCursor A, B;
  cursor_init(A, a.indices + fpk::tri_offset(ha, i, a.nb), i + 1, a.counts[(int64_t)ha * a.nb + i], lane);
  cursor_init(B, a.indices + fpk::tri_offset(ha + 1, i, a.nb), i + 1, a.counts[(int64_t)(ha + 1) * a.nb + i],
              lane);

  TileLoader<false> ld;
  ld.init(a, g, w, lane);

  QFrag<false> qf[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    if (q_valid) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)tq * a.q_st +
                           (int64_t)(ha + x) * a.q_sh + 8 * hh;
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[x].f[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[x].f[s] = (bf16x8){0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) in_agpr(qf[x].f[s]);
  }

  // Units t = 0 .. 2U-1, two per union block (U blocks).  Step t computes
  // S(t+1) (phase 1, K(t+1)) and O += P(t) V(t) (phase 2, V(t)), with one
  // workgroup barrier B_t between the phases.  Before B_t each wave waits
  // for its share of V(t) and K(t+2); after B_t every wave has finished
  // phase 1 of step t (so K(t+1)'s buffer is free) and phase 2 of step t-1
  // (so V(t-1)'s buffer is free): K(t+4) and V(t+2) are issued into them.
  // Each load thus has two steps to land.  Issue order ... K(t+3), V(t+1),
  // K(t+4), V(t+2) ...: at B_t the loads younger than K(t+2) and V(t) are
  // K(t+3) and V(t+1), so the wait is vmcnt(kK + kV) while both exist, and
  // a full drain near the end of the list.
  constexpr int kK = TileLoader<false>::kKLoads;
  int jc, fc;
  union_next(A, B, lane, jc, fc);  // never empty: both lists end with the diagonal
  int jn = 0, fn = 0;
  bool hn = union_next(A, B, lane, jn, fn);
  // prologue loads, in this order: K(0), K(1), K(2), V(0), V(1)
  ld.load_k(sK, jc, 0, w);
  ld.load_k(sK + kHalfU4, jc, 1, w);
  if (hn) ld.load_k(sK + 2 * kHalfU4, jn, 0, w);
  ld.load_v(sV, jc, 0, w);
  ld.load_v(sV + kHalfU4, jc, 1, w);
  floatx16 o[2][4];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      o[x][dt] = (floatx16){0};
      in_agpr(o[x][dt]);
    }
  float m_run[2] = {-INFINITY, -INFINITY};
  Step2 x;
  x.c = c;
  x.l[0] = 0.f;
  x.l[1] = 0.f;
  // K(0) and K(1) landed (K(2), V(0), V(1) may be in flight)
  if (hn) tile_barrier<kK + 8>();
  else tile_barrier<8>();
  floatx16 sA[2][2], sB[2][2];  // [head][sub-tile]
#pragma unroll
  for (int hd = 0; hd < 2; ++hd)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const uint4* kr = sK + (32 * kt + pm) * 16;
      const int xk = swz(32 * kt + pm) ^ hh;
      sA[hd][kt] = qk_first(*reinterpret_cast<const bf16x8*>(&kr[0 ^ xk]), qf[hd].f[0]);
#pragma unroll
      for (int st = 1; st < 8; ++st)
        qk_acc(sA[hd][kt], *reinterpret_cast<const bf16x8*>(&kr[(2 * st) ^ xk]), qf[hd].f[st]);
    }
  float mx[2];
#pragma unroll
  for (int hd = 0; hd < 2; ++hd) {
    if (!(fc & (1 << hd))) drop_unit(sA[hd]);
    else if (jc == i) mask_diag(sA[hd], w, 0, qi, hh);
    mx[hd] = pair_max(tile_max(sA[hd]));
  }

  int r0 = 0;  // t % 3 of the trip's first unit
  bool first = true;
  for (;;) {
    int jn2 = 0, fn2 = 0;
    const bool hn2 = hn && union_next(A, B, lane, jn2, fn2);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      floatx16(*s_cur)[2] = half == 0 ? sA : sB;
      floatx16(*s_nxt)[2] = half == 0 ? sB : sA;
      const int rt = half == 0 ? r0 : (r0 == 2 ? 0 : r0 + 1);  // t % 3
      const int rt1 = rt == 2 ? 0 : rt + 1;                    // (t+1) % 3
      const int rt2 = rt1 == 2 ? 0 : rt1 + 1;                  // (t+2) % 3
#pragma unroll
      for (int hd = 0; hd < 2; ++hd) {
        raise_max_h(o[hd], m_run[hd], x.l[hd], mx[hd], c);
        x.mu[hd] = m_run[hd] == -INFINITY ? 0.0f : m_run[hd];
      }
      phase1_2h(sK + rt1 * kHalfU4, qf[0], qf[1], s_cur[0], s_cur[1], s_nxt[0], s_nxt[1], x, hh, pm);
      // B_t: V(t) and K(t+2) landed; K(t+3) and V(t+1) may be in flight
      if (half == 0 && first) tile_barrier<4>();  // t = 0: only V(1) is younger
      else if (half == 0 ? hn : hn2) tile_barrier<kK + 4>();
      else tile_barrier<0>();
      // After B_t: K(t+4) into K(t+1)'s buffer, V(t+2) into V(t-1)'s buffer
      // (t = 0 also issues K(3), into K(0)'s buffer, first).  With one wave
      // per SIMD nothing covers a burst of loads, so phase 2 issues them one
      // per slot, in the shadow of its products.
      if (half == 0 && first && hn) ld.load_k(sK + rt * kHalfU4, jn, 1, w);
      uint4* const k_dst = sK + rt1 * kHalfU4;
      uint4* const v_dst = sV + rt2 * kHalfU4;
      auto issue = [&](int m) {
        if (m < kK) {
          if (hn2) ld.load_k_one(k_dst, jn2, half, w, m);
        } else if (m < kK + 4) {
          if (hn) ld.load_v_one(v_dst, jn, half, w, m - kK);
        }
      };
      phase2_2h(sV + rt * kHalfU4, s_cur[0], s_cur[1], s_nxt[0], s_nxt[1], o, x, qi, hh, mx, issue);
      // S(t+1) belongs to the second half of jc (half 0) or the first of jn (half 1)
      const bool nxt_exists = half == 0 || hn;
      const int jb = half == 0 ? jc : jn;
      const int fb = half == 0 ? fc : fn;
      if (nxt_exists) {
#pragma unroll
        for (int hd = 0; hd < 2; ++hd) {
          if (!(fb & (1 << hd))) {
            drop_unit(s_nxt[hd]);
            mx[hd] = -INFINITY;
          } else if (jb == i) {
            mask_diag(s_nxt[hd], w, half == 0 ? 1 : 0, qi, hh);
            mx[hd] = tile_max(s_nxt[hd]);
          }
        }
      }
      mx[0] = pair_max(mx[0]);
      mx[1] = pair_max(mx[1]);
    }
    if (!hn) break;
    first = false;
    r0 = r0 == 0 ? 2 : r0 - 1;  // (t + 2) % 3
    jc = jn;
    fc = fn;
    jn = jn2;
    fn = fn2;
    hn = hn2;
  }
  // every wave has finished reading the tile buffers before they are reused
  // for the output staging
  __syncthreads();

  // Normalise and write out, one head after the other, through the LDS
  // staging rows of the one-head kernel (the last barrier released the tile
  // buffers; each wave only touches its own 32 rows).
#pragma unroll
  for (int hd = 0; hd < 2; ++hd) {
    const float l = x.l[hd] + __shfl_xor(x.l[hd], 32);
    const float inv = a.out_scale / l;
    uint8_t* stg = reinterpret_cast<uint8_t*>(smem) + w * 32 * kStageRow;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * dt + 8 * q4 + 4 * hh;
        const int r = 4 * q4;
        const bf16x2 p01 = {(__bf16)(o[hd][dt][r] * inv), (__bf16)(o[hd][dt][r + 1] * inv)};
        const bf16x2 p23 = {(__bf16)(o[hd][dt][r + 2] * inv), (__bf16)(o[hd][dt][r + 3] * inv)};
        *reinterpret_cast<uint2*>(stg + qi * kStageRow + 2 * d0) =
            make_uint2(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23));
      }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int ch = it * 64 + lane;
      const int tok = ch >> 4;
      const uint4 v = *reinterpret_cast<const uint4*>(stg + tok * kStageRow + (ch & 15) * 16);
      const int t = tok0 + 32 * w + tok;
      if (32 * w + tok < rows)
        *reinterpret_cast<uint4*>(a.out + (int64_t)t * a.o_st + (int64_t)(ha + hd) * a.o_sh + (ch & 15) * 8) = v;
    }
  }
}

}  // namespace

hipError_t fpk_launch_attn_pack(const fp_problem& p, const FpDims& dm, const int* counts, const int* indices,
                                const uint16_t* v_t, float sm_scale, hipStream_t st) {
  AttnArgs a{};
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
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.out_scale = 1.0f;
  const dim3 grid((unsigned)(dm.nb * (dm.Hq / 2)));
  hipLaunchKernelGGL(attn_pack_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
