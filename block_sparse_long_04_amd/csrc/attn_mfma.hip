// Step 5 on the matrix cores: block-sparse causal attention with GQA over the
// kept key blocks, bf16 inputs (e4m3fn variant in attn_fp8.hip), head_dim 128,
// block 128.
//
// FlashPrefill skill page, "Architecture Overview" (physical index jumping:
// only the listed key blocks are visited) and "Implementation Steps" (the
// final stage is block-sparse attention over the identified blocks); GQA per
// the FlashPrefill V2 abstract.
//
// One workgroup = one (q head h, query block i), four waves of 32 query rows.
// Per kept key block j (ascending list, the diagonal last):
//   * the K tile [128 keys][128 dims] and the V^T tile [128 dims][128 keys]
//     are staged in LDS (16-byte chunks, chunk index XOR (row & 15) so the
//     matrix-core operand reads are bank-conflict free);
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (four 32-key sub-tiles, eight
//     16-wide steps over the head dimension).  Computing the transpose puts
//     one query per lane column, so each lane owns 64 of its query's 128
//     logits and the other half sits in lane ^ 32: softmax statistics need a
//     single cross-lane exchange.  The K rows are fed in the permuted order
//     that makes those 64 logits come out as contiguous 8-key runs, which are
//     exactly the B operand of the next product;
//   * online softmax in the exp2 domain (running max and sum per query);
//   * O^T += V^T P^T, P packed to bf16 straight from the S^T registers.
// The causal mask is applied only on the diagonal block.  The final 1/l and
// the V dequantisation scale are applied once at the end.
//
// Work order: heavy (late) query blocks first; within every run of 8*G
// consecutive workgroup ids, the G heads of one kv group at one query block
// get ids that the hardware dispatches to the same XCD (ids are dealt to the
// 8 XCDs round-robin), so a K/V tile fetched for one head is found in that
// XCD's L2 by the other heads of its group.
#include "common.h"

namespace {

using fpk::bf16x8;
using fpk::floatx16;

struct AttnArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint16_t* vt;
  uint16_t* out;
  const int* counts;
  const int* indices;
  int64_t q_st, q_sh, k_st, k_sh, o_st, o_sh;
  int L, Hq, Hkv, nb, Lpad;
  float scale_log2;  // sm_scale * log2(e)
  float out_scale;
};

__device__ __forceinline__ void work_item(int bid, int nb, int Hq, int Hkv, int& h, int& i) {
  const int G = Hq / Hkv;
  const int total = nb * Hq;
  const int chunk = 8 * G;
  const int full = (total / chunk) * chunk;
  int p, slot;
  if (bid < full) {
    const int sup = bid / chunk;
    const int r = bid - sup * chunk;
    p = sup * 8 + (r & 7);
    slot = r >> 3;
  } else {
    p = bid / G;
    slot = bid - p * G;
  }
  const int row = p / Hkv;
  i = nb - 1 - row;
  h = (p - row * Hkv) * G + slot;
}

__global__ __launch_bounds__(256) void attn_bf16_d128_kernel(AttnArgs a) {
  __shared__ uint4 sK[128 * 16];  // [key][16 chunks], swizzled
  __shared__ uint4 sV[128 * 16];  // [dim][16 chunks of 8 keys], swizzled

  int h, i;
  work_item(blockIdx.x, a.nb, a.Hq, a.Hkv, h, i);
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int qi = lane & 31;
  const int hh = lane >> 5;
  const int tq = i * 128 + w * 32 + qi;

  // B operand of S^T = K Q^T: lane holds Q[tq][16s + 8hh .. +7] for step s.
  bf16x8 qf[8];
  if (tq < a.L) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + tq * a.q_st + h * a.q_sh + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = (bf16x8){0, 0, 0, 0, 0, 0, 0, 0};
  }

  floatx16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = (floatx16){0};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int cnt = a.counts[(int64_t)h * a.nb + i];
  const int* lst = a.indices + fpk::tri_offset(h, i, a.nb);
  // Output row m of the 32x32 tile sits in register 4*(m/8) + m%4 of lane
  // half (m/4)&1; feeding key pm(m) = m with bits 2 and 3 swapped as row m
  // makes register r of half hh hold key 16*(r/8) + 8*hh + r%8.
  const int pm = (qi & 0x13) | ((qi & 4) << 1) | ((qi & 8) >> 1);
  const int lc = tid & 15;   // tile-load chunk
  const int lr = tid >> 4;   // tile-load row base

  for (int n = 0; n < cnt; ++n) {
    const int j = lst[n];
    __syncthreads();
    {
      uint4 kv[8], vv[8];
      const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k) + g * a.k_sh + lc * 8;
      const uint16_t* vb = a.vt + ((int64_t)g * 128) * a.Lpad + (int64_t)j * 128 + lc * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = lr + 16 * e;
        const int key = j * 128 + row;
        kv[e] = key < a.L ? *reinterpret_cast<const uint4*>(kb + (int64_t)key * a.k_st)
                          : make_uint4(0, 0, 0, 0);
        vv[e] = *reinterpret_cast<const uint4*>(vb + (int64_t)row * a.Lpad);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = lr + 16 * e;
        sK[row * 16 + (lc ^ (row & 15))] = kv[e];
        sV[row * 16 + (lc ^ (row & 15))] = vv[e];
      }
    }
    __syncthreads();

    floatx16 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = (floatx16){0};
      const int row = kt * 32 + pm;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sK[row * 16 + ((2 * st + hh) ^ (row & 15))]);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[st], s[kt], 0, 0, 0);
      }
    }
    if (j == i) {
      const int qrel = w * 32 + qi;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int krel = kt * 32 + 16 * (r >> 3) + 8 * hh + (r & 7);
          if (krel > qrel) s[kt][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[kt][r] * a.scale_log2 - m_new);
        s[kt][r] = p;
        l_run += p;
      }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;

    bf16x8 pb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[u][e] = (__bf16)s[u >> 1][8 * (u & 1) + e];

#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int drow = dt * 32 + qi;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sV[drow * 16 + ((2 * u + hh) ^ (drow & 15))]);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[u], o[dt], 0, 0, 0);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = a.out_scale / l_tot;
  if (tq < a.L) {
    uint16_t* op = a.out + tq * a.o_st + h * a.o_sh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = dt * 32 + 8 * q4 + 4 * hh;
        const uint32_t b0 = fpk::f32_to_bf16_bits(o[dt][4 * q4 + 0] * inv);
        const uint32_t b1 = fpk::f32_to_bf16_bits(o[dt][4 * q4 + 1] * inv);
        const uint32_t b2 = fpk::f32_to_bf16_bits(o[dt][4 * q4 + 2] * inv);
        const uint32_t b3 = fpk::f32_to_bf16_bits(o[dt][4 * q4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + d0) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
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
  dim3 grid((unsigned)(dm.nb * dm.Hq));
  if (fp8) return hipErrorInvalidValue;  // e4m3fn inputs take the generic kernel for now
  hipLaunchKernelGGL(attn_bf16_d128_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
