// Step 5 on the vector ALUs: block-sparse causal attention for the shapes
// the matrix-core kernel does not take (fp32 inputs, head_dim 64, block 64,
// token strides too large for its 32-bit tile offsets).
//
// FlashPrefill skill page, "Architecture Overview" (physical index jumping
// over the kept block indices).  One workgroup = one (q head, query block):
// KS threads per query row, each taking every KS-th key of the listed blocks.
// For each listed key block the K and V tiles are widened to fp32 in LDS;
// every thread runs an exact per-key online softmax (running max, rescaled
// sum and accumulator) in fp32 with expf over its keys, and at the end the
// KS partial states of a row are merged (max, rescale, sum).
#include "common.h"

namespace {

struct GenArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  void* out;
  const int* counts;
  const int* indices;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;
  int L, Hq, Hkv, nb;
  float logit_scale;  // sm_scale * q_scale * k_scale
  float out_scale;    // v_scale
  int out_f32;
};

template <int ESZ>
__device__ __forceinline__ float load_elem(const uint8_t* p, int64_t idx) {
  if constexpr (ESZ == 4) return reinterpret_cast<const float*>(p)[idx];
  else if constexpr (ESZ == 2) return fpk::bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[idx]);
  else return fpk::e4m3_to_f32(p[idx]);
}

template <int D, int BS, int ESZ>
__global__ __launch_bounds__(256) void attn_generic_kernel(GenArgs a) {
  constexpr int KS = 256 / BS;  // threads per query row: 4 for B = 64, 2 for B = 128
  __shared__ float sK[BS][D];
  __shared__ float sV[BS][D];
  __shared__ float sML[BS][2];
  const int h = blockIdx.x % a.Hq;
  const int i = a.nb - 1 - (int)(blockIdx.x / a.Hq);
  const int g = h / (a.Hq / a.Hkv);
  const int t = threadIdx.x % BS;   // query row of the block
  const int part = threadIdx.x / BS;  // this thread takes keys s with s % KS == part
  const int tq = i * BS + t;
  const bool valid = tq < a.L;

  float qv[D];
  float o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = valid ? load_elem<ESZ>(a.q, (int64_t)tq * a.q_st + h * a.q_sh + c) : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int cnt = a.counts[(int64_t)h * a.nb + i];
  const int* lst = a.indices + fpk::tri_offset(h, i, a.nb);

  for (int n = 0; n < cnt; ++n) {
    const int j = lst[n];
    __syncthreads();
    for (int e = threadIdx.x; e < BS * D; e += BS * KS) {
      const int r = e / D;
      const int c = e - r * D;
      const int key = j * BS + r;
      float kx = 0.f, vx = 0.f;
      if (key >= 0 && key < a.L) {  // (j outside the sequence: zeros, never a stray read)
        kx = load_elem<ESZ>(a.k, (int64_t)key * a.k_st + g * a.k_sh + c);
        vx = load_elem<ESZ>(a.v, (int64_t)key * a.v_st + g * a.v_sh + c);
      }
      sK[r][c] = kx;
      sV[r][c] = vx;
    }
    __syncthreads();
    int kend = (j == i) ? t : BS - 1;       // causal inside the diagonal block
    kend = min(kend, a.L - 1 - j * BS);     // keys past L do not exist
    if (!valid) kend = -1;
    for (int s = part; s <= kend; s += KS) {
      float x = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) x = fmaf(qv[c], sK[s][c], x);
      x *= a.logit_scale;
      if (x > m) {
        const float alpha = expf(m - x);
        l *= alpha;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] *= alpha;
        m = x;
      }
      const float p = expf(x - m);
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(p, sV[s][c], o[c]);
    }
  }
  // merge the KS partial states of each row into part 0, one part at a
  // time through sK (a part with no keys has m = -inf and l = 0)
  for (int p = 1; p < KS; ++p) {
    __syncthreads();
    if (part == p) {
#pragma unroll
      for (int c = 0; c < D; ++c) sK[t][c] = o[c];
      sML[t][0] = m;
      sML[t][1] = l;
    }
    __syncthreads();
    if (part == 0) {
      const float m2 = sML[t][0], l2 = sML[t][1];
      const float mn = fmaxf(m, m2);
      const float a1 = mn == -INFINITY ? 0.f : expf(m - mn);
      const float a2 = mn == -INFINITY ? 0.f : expf(m2 - mn);
      l = l * a1 + l2 * a2;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = o[c] * a1 + sK[t][c] * a2;
      m = mn;
    }
  }
  if (!valid || part != 0) return;
  const float inv = a.out_scale / l;
  if (a.out_f32) {
    float* op = static_cast<float*>(a.out) + (int64_t)tq * a.o_st + h * a.o_sh;
#pragma unroll
    for (int c = 0; c < D; ++c) op[c] = o[c] * inv;
  } else {
    uint16_t* op = static_cast<uint16_t*>(a.out) + (int64_t)tq * a.o_st + h * a.o_sh;
#pragma unroll
    for (int c = 0; c < D; ++c) op[c] = (uint16_t)fpk::f32_to_bf16_bits(o[c] * inv);
  }
}

template <int D, int BS>
hipError_t launch_db(const GenArgs& a, int esz, unsigned grid, hipStream_t st) {
  static_assert(256 % BS == 0, "block size divides the workgroup");
  if (esz == 4) hipLaunchKernelGGL((attn_generic_kernel<D, BS, 4>), dim3(grid), dim3(256), 0, st, a);
  else if (esz == 2) hipLaunchKernelGGL((attn_generic_kernel<D, BS, 2>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((attn_generic_kernel<D, BS, 1>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t fpk_launch_attn_generic(const fp_problem& p, const FpDims& dm, const int* counts,
                                   const int* indices, float sm_scale, hipStream_t st) {
  GenArgs a;
  a.q = static_cast<const uint8_t*>(p.q);
  a.k = static_cast<const uint8_t*>(p.k);
  a.v = static_cast<const uint8_t*>(p.v);
  a.out = p.out;
  a.counts = counts;
  a.indices = indices;
  a.q_st = p.q_stride_tok;
  a.q_sh = p.q_stride_head;
  a.k_st = p.k_stride_tok;
  a.k_sh = p.k_stride_head;
  a.v_st = p.v_stride_tok;
  a.v_sh = p.v_stride_head;
  a.o_st = p.o_stride_tok;
  a.o_sh = p.o_stride_head;
  a.L = dm.L;
  a.Hq = dm.Hq;
  a.Hkv = dm.Hkv;
  a.nb = dm.nb;
  const bool fp8 = p.dtype == FP_FP8_E4M3;
  a.logit_scale = sm_scale * (fp8 ? p.q_scale * p.k_scale : 1.0f);
  a.out_scale = fp8 ? p.v_scale : 1.0f;
  a.out_f32 = p.dtype == FP_F32 ? 1 : 0;
  const int esz = p.dtype == FP_F32 ? 4 : (p.dtype == FP_BF16 ? 2 : 1);
  const unsigned grid = (unsigned)(dm.nb * dm.Hq);
  if (dm.d == 64 && dm.B == 64) return launch_db<64, 64>(a, esz, grid, st);
  if (dm.d == 64 && dm.B == 128) return launch_db<64, 128>(a, esz, grid, st);
  if (dm.d == 128 && dm.B == 64) return launch_db<128, 64>(a, esz, grid, st);
  return launch_db<128, 128>(a, esz, grid, st);
}
