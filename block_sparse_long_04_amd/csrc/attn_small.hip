// Step 5 on the matrix cores for bf16 layers whose head dimension or block
// is 64 (D, B in {64, 128}, not both 128: those take attn_mfma.hip).
//
// FlashPrefill skill page, "Architecture Overview" (only the listed key
// blocks are visited) and "Implementation Steps" (block-sparse attention over
// the identified blocks); GQA per the FlashPrefill V2 abstract.
//
// One workgroup = one (q head h, query block i): B / 32 waves, wave w owning
// query rows 32w .. 32w+31.  Per listed key block:
//   * the K tile [B keys][D dims] and the V^T tile [D dims][B keys] (V^T
//     written by this call's layout pass) travel global -> LDS with
//     buffer_load ... lds into a ring of three stages: block n + 2 is
//     requested while block n is computed, one barrier per block;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16, one 32-key sub-tile at a
//     time, D / 16 steps; K rows are fed in the order pm(m) (bits 2 and 3
//     swapped) so each lane holds runs of 8 consecutive keys, the B operand
//     of P.V as is (the same conventions as attn_mfma.hip);
//   * online softmax in the exp2 domain with the lazy maximum of
//     attn_mfma.hip; the causal mask on the diagonal block only;
//   * O^T += V^T P^T, D / 32 head-dim tiles by B / 16 key groups.
// LDS rows of 128 B (K with D = 64, V^T with B = 64) hold their eight 16-byte
// chunks at chunk ^ ((row >> 1) & 7), rows of 256 B at chunk ^ (row & 15):
// the 16 rows a 16-byte operand read touches land on distinct bank slots.
#include "attn_common.h"

namespace {

struct SmallArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* vt;
  uint16_t* out;
  const int* counts;
  const int* indices;
  int64_t q_st, q_sh, k_st, k_sh, o_st, o_sh;
  int L, Hq, Hkv, nb, Lpad;
  float scale_log2;
};

// slot of 16-byte chunk c in an LDS row r of kRowBytes bytes (an XOR, so
// the chunk stored in slot s is slot_of(r, s) too)
template <int kRowBytes>
__device__ __forceinline__ int slot_of(int r, int c) {
  return kRowBytes == 128 ? (c ^ ((r >> 1) & 7)) : (c ^ (r & 15));
}

// Maximum of the NKT sub-tiles' 16 values per lane, with v_max3_f32 written
// out: fmaxf would first canonicalise each operand (one more instruction per
// value), which scores fresh from the matrix cores do not need.
template <int NKT>
__device__ __forceinline__ float block_max(const floatx16* s) {
  float acc[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    acc[kt] = max3_late(s[kt][0], s[kt][1], s[kt][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) acc[kt] = max3_late(acc[kt], s[kt][r], s[kt][r + 1]);
    acc[kt] = max3_late(acc[kt], s[kt][15], s[kt][15]);
  }
  float m = acc[0];
#pragma unroll
  for (int kt = 1; kt < NKT; kt += 2)
    m = kt + 1 < NKT ? max3_late(m, acc[kt], acc[kt + 1]) : max3_late(m, acc[kt], acc[kt]);
  return m;
}

// Issues one key block's K and V^T tiles into ring stage stg: LPW 1 KiB
// buffer_load ... lds per tile for this wave (its chunks of the tile).
template <int D, int BS>
struct SmallLoader {
  static constexpr int KRB = D * 2;
  static constexpr int TCH = BS * D / 8;
  static constexpr int LPW = TCH / (64 * (BS / 32));
  const uint8_t* kg;   // K of this kv head
  const uint16_t* vg;  // V^T of this kv head
  int k_row, L, v_bytes;
  int wave_off;  // this wave's first chunk of a tile
  uint32_t koff[LPW], voff[LPW];
  int krow[LPW];

  __device__ __forceinline__ void load(int j, uint4* dk, uint4* dv) const {
    const int present = min(BS, L - j * BS);
    const int ext = (j >= 0 && present > 0) ? (present - 1) * k_row + KRB : 0;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kg + (int64_t)j * BS * k_row), 0, ext, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vg), 0, v_bytes, 0x00020000);
#pragma unroll
    for (int e = 0; e < LPW; ++e) {
      uint32_t ko = koff[e];
      if (krow[e] >= present)  // ragged last block: repeat row L - 1
        ko = (uint32_t)((present - 1) * k_row) + (koff[e] - (uint32_t)(krow[e] * k_row));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(dk + wave_off + 64 * e), 16, ko, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < LPW; ++e)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(dv + wave_off + 64 * e), 16, voff[e],
                                               j * BS * 2, 0, 0);
  }
};

template <int D, int BS, int kWaves>
__global__ __launch_bounds__(BS * 2) __attribute__((amdgpu_waves_per_eu(kWaves))) void attn_small_kernel(SmallArgs a) {
  constexpr int NKT = BS / 32;       // 32-key sub-tiles per block
  constexpr int KST = D / 16;        // head-dim steps of S^T
  constexpr int NDT = D / 32;        // head-dim tiles of O^T
  constexpr int NU = BS / 16;        // 16-key groups of P.V
  constexpr int KRB = D * 2;         // K row bytes in LDS
  constexpr int VRB = BS * 2;        // V^T row bytes in LDS
  constexpr int TCH = BS * D / 8;    // 16-byte chunks of a K tile (= of a V^T tile)
  constexpr int NW = BS / 32;        // waves
  constexpr int LPW = TCH / (64 * NW);  // 1 KiB loads per wave per tile
  static_assert(TCH % (64 * NW) == 0, "tile loads split evenly over the waves");
  __shared__ uint4 smem[4 * TCH];  // K stage 0, K stage 1, V^T stage 0, V^T stage 1

  const int h = blockIdx.x % a.Hq;
  const int i = a.nb - 1 - (int)(blockIdx.x / a.Hq);  // late (heavy) query blocks first
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = lane & 31;
  const int hh = lane >> 5;
  const int tok0 = i * BS;
  const int rows = min(BS, a.L - tok0);
  const int tq = tok0 + 32 * w + qi;
  const bool q_valid = 32 * w + qi < rows;
  const int pm = (qi & 0x13) | ((qi & 4) << 1) | ((qi & 8) >> 1);
  const float c = a.scale_log2;
  const int cnt = a.counts[(int64_t)h * a.nb + i];
  const int* lst = a.indices + fpk::tri_offset(h, i, a.nb);

  // the list, 64 entries at a time in one VGPR, taken with readlane
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int*>(lst), 0, (i + 1) * 4, 0x00020000);
  int win = (int)__builtin_amdgcn_raw_buffer_load_b32(lrs, lane * 4, 0, 0);
  int wbase = 0;
  auto entry = [&](int n) -> int {
    if (n - wbase >= 64) {
      wbase += 64;
      win = (int)__builtin_amdgcn_raw_buffer_load_b32(lrs, (wbase + lane) * 4, 0, 0);
      FP_WAIT_VMEM();
    }
    return __builtin_amdgcn_readlane(win, n - wbase);
  };

  bf16x8 qf[KST];
#pragma unroll
  for (int s = 0; s < KST; ++s) {
    qf[s] = (bf16x8){0, 0, 0, 0, 0, 0, 0, 0};
    if (q_valid)
      qf[s] = *reinterpret_cast<const bf16x8*>(a.q + (int64_t)tq * a.q_st + (int64_t)h * a.q_sh + 16 * s + 8 * hh);
  }

  // Direct-to-LDS tile loads.  Load e of wave w moves 1 KiB: lane l writes
  // 16-byte chunk (64 (LPW w + e) + l) of the tile, i.e. row r = that / (row
  // chunks), slot = that % (row chunks), fetching the row's global chunk
  // slot_of(r, .) maps there (an involution).  K rows come through a buffer
  // resource per key block (extent up to the block's last present row; rows
  // past L repeat row L - 1, masked later), V^T rows through one resource
  // per kv head (zero past L).
  SmallLoader<D, BS> ld;
  ld.kg = reinterpret_cast<const uint8_t*>(a.k + (int64_t)g * a.k_sh);
  ld.vg = a.vt + (int64_t)g * D * a.Lpad;
  ld.k_row = (int)(a.k_st * 2);
  ld.L = a.L;
  ld.v_bytes = D * a.Lpad * 2;
  ld.wave_off = 64 * LPW * w;
#pragma unroll
  for (int e = 0; e < LPW; ++e) {
    const int ch = 64 * (LPW * w + e) + lane;
    const int kr = ch / (KRB / 16), ks = ch % (KRB / 16);
    ld.krow[e] = kr;
    ld.koff[e] = (uint32_t)(kr * ld.k_row + slot_of<KRB>(kr, ks) * 16);
    const int vr = ch / (VRB / 16), vs = ch % (VRB / 16);
    ld.voff[e] = (uint32_t)(vr * a.Lpad * 2 + slot_of<VRB>(vr, vs) * 16);
  }

  floatx16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = (floatx16){0};
  float m_run = -INFINITY, l = 0.f;

  // One key block j from the tiles sKc (K) and sVc (V^T).
  auto block_step = [&](int j, const uint4* sKc, const uint4* sVc) {
    // S^T = K Q^T, sub-tile by sub-tile
    floatx16 s[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const int r = 32 * kt + pm;
      s[kt] = (floatx16){0};
#pragma unroll
      for (int st = 0; st < KST; ++st)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(&sKc[r * (KRB / 16) + slot_of<KRB>(r, 2 * st + hh)]), qf[st],
            s[kt], 0, 0, 0);
    }
    if (j == i) {  // causal mask of the diagonal block
#pragma unroll
      for (int kh = 0; kh < NKT / 2; ++kh) mask_diag(s + 2 * kh, w, kh, qi, hh);
    }
    const float mx = pair_max(block_max<NKT>(s));
    const float mxs = mx * c;
    if (__any(mxs > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mxs);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    }
    const float mu = m_run == -INFINITY ? 0.0f : m_run;
    // P in bf16 pairs: group u = keys 16 u .. 16 u + 15 (sub-tile u / 2, registers 8 (u % 2) ..)
    uint32_t pw[NU][4];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * (u & 1) + 2 * e;
        pw[u][e] = pack_pair(exp_one(s[u >> 1][r], c, mu), exp_one(s[u >> 1][r + 1], c, mu), l);
      }
    // O^T += V^T P^T
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int r = 32 * dt + qi;
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(&sVc[r * (VRB / 16) + slot_of<VRB>(r, 2 * u + hh)]),
            as_bf16x8(pw[u]), o[dt], 0, 0, 0);
      }
  };

  // Two stages; two list positions per trip so each stage's role is static
  // (the loads into one stage and the reads of the other then carry
  // distinct addresses the compiler can tell apart, and no wait for the
  // loads in flight is placed before the reads).  entry() is called once
  // per list position, in order: its window only moves forward.
  uint4* const sK0 = smem;
  uint4* const sK1 = smem + TCH;
  uint4* const sV0 = smem + 2 * TCH;
  uint4* const sV1 = smem + 3 * TCH;
  int j_cur = entry(0);
  ld.load(j_cur, sK0, sV0);
  for (int n = 0; n < cnt; n += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int t = n + half;
      if (half == 1 && t >= cnt) break;
      const uint4* sKc = half == 0 ? sK0 : sK1;
      const uint4* sVc = half == 0 ? sV0 : sV1;
      uint4* sKn = half == 0 ? sK1 : sK0;
      uint4* sVn = half == 0 ? sV1 : sV0;
      const int j = j_cur;
      // block t has landed; after the barrier every wave is done with block
      // t - 1, whose stage takes block t + 1
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + 1 < cnt) {
        j_cur = entry(t + 1);
        ld.load(j_cur, sKn, sVn);
      }
      block_step(j, sKc, sVc);
    }
  }

  // Normalise and write out: lane holds dims 32 dt + 8 q4 + 4 hh + 0..3 of token qi.
  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.0f / lt;
  if (q_valid) {
    uint16_t* op = a.out + (int64_t)tq * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r = 4 * q4;
        const bf16x2 p01 = {(__bf16)(o[dt][r] * inv), (__bf16)(o[dt][r + 1] * inv)};
        const bf16x2 p23 = {(__bf16)(o[dt][r + 2] * inv), (__bf16)(o[dt][r + 3] * inv)};
        *reinterpret_cast<uint2*>(op + 32 * dt + 8 * q4 + 4 * hh) =
            make_uint2(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23));
      }
  }
}

// The waves per SIMD each variant's registers are sized for (LDS: two
// stages of K and V^T, 4 B D 2 bytes per workgroup, of 160 KiB per CU).
constexpr int kWv6464 = 3, kWv64128 = 2, kWv12864 = 1;
template __global__ void attn_small_kernel<64, 64, kWv6464>(SmallArgs);
template __global__ void attn_small_kernel<64, 128, kWv64128>(SmallArgs);
template __global__ void attn_small_kernel<128, 64, kWv12864>(SmallArgs);

}  // namespace

hipError_t fpk_launch_attn_small(const fp_problem& p, const FpDims& dm, const int* counts, const int* indices,
                                 const uint16_t* v_t, float sm_scale, hipStream_t st) {
  SmallArgs a{};
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
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
  const dim3 grid((unsigned)(dm.nb * dm.Hq));
  if (dm.d == 64 && dm.B == 64)
    hipLaunchKernelGGL((attn_small_kernel<64, 64, kWv6464>), grid, dim3(128), 0, st, a);
  else if (dm.d == 64)
    hipLaunchKernelGGL((attn_small_kernel<64, 128, kWv64128>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_small_kernel<128, 64, kWv12864>), grid, dim3(128), 0, st, a);
  return hipGetLastError();
}
