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
#include "attn_common.h"

namespace {

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
