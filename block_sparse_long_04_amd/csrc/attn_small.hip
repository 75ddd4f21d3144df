// Step 5 on the matrix cores for bf16 layers whose head dimension or block
// is 64 (D, B in {64, 128}, not both 128: those take attn_mfma.hip).
//
// FlashPrefill skill page, "Architecture Overview" (only the listed key
// blocks are visited) and "Implementation Steps" (block-sparse attention over
// the identified blocks); GQA per the FlashPrefill V2 abstract.
//
// One workgroup = one (q head h, query block i): B / 32 waves, wave w owning
// query rows 32w .. 32w+31.  The listed key blocks are walked in units of 64
// keys (B / 64 units per block).  Per unit:
//   * the K tile [64 keys][D dims] and the V^T tile [D dims][64 keys] (V^T
//     written by this call's layout pass) travel global -> LDS with
//     buffer_load ... lds into a ring of NS stages: unit t + NS - 1 is
//     requested while unit t is computed, one barrier per unit;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16, two 32-key sub-tiles, D / 16
//     steps each; K rows are fed in the order pm(m) (bits 2 and 3 swapped) so
//     each lane holds runs of 8 consecutive keys, the B operand of P.V as is
//     (the same conventions as attn_mfma.hip);
//   * online softmax in the exp2 domain with the lazy maximum of
//     attn_mfma.hip; the causal mask on the diagonal block only;
//   * O^T += V^T P^T, D / 32 head-dim tiles by 4 key groups of 16.
// LDS rows of 128 B (K with D = 64, every V^T unit row) hold their eight
// 16-byte chunks at chunk ^ ((row >> 1) & 7), rows of 256 B (K with D = 128)
// at chunk ^ (row & 15): the 16 rows a 16-byte operand read touches land on
// distinct bank slots.
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

// Issues one 64-key unit's K and V^T tiles (key block j, keys 64 hf ..
// 64 hf + 63 of it) into the stage at dk / dv: LPW 1 KiB buffer_load ... lds
// per tile for this wave (its chunks of the tile).  K rows come through a
// buffer resource per unit (extent up to the unit's last present row; rows
// past L repeat row L - 1 and a unit wholly past L reads zeros, masked
// later), V^T rows through one resource per kv head (zero past L).
template <int D, int BS>
struct UnitLoader {
  static constexpr int KRB = D * 2;
  static constexpr int TCH = 64 * D / 8;
  static constexpr int LPW = TCH / (64 * (BS / 32));
  const uint8_t* kg;   // K of this kv head
  const uint16_t* vg;  // V^T of this kv head
  int k_row, L, v_bytes;
  int wave_off;  // this wave's first chunk of a tile
  uint32_t koff[LPW], voff[LPW];
  int krow[LPW];

  __device__ __forceinline__ void load(int j, int hf, uint4* dk, uint4* dv) const {
    const int key0 = j * BS + 64 * hf;
    const int present = min(64, L - key0);
    const int ext = present > 0 ? (present - 1) * k_row + KRB : 0;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kg + (int64_t)key0 * k_row), 0, ext, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vg), 0, v_bytes, 0x00020000);
#pragma unroll
    for (int e = 0; e < LPW; ++e) {
      uint32_t ko = koff[e];
      if (krow[e] >= present)  // ragged last unit: repeat row L - 1
        ko = (uint32_t)((present - 1) * k_row) + (koff[e] - (uint32_t)(krow[e] * k_row));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(dk + wave_off + 64 * e), 16, ko, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < LPW; ++e)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(dv + wave_off + 64 * e), 16, voff[e], key0 * 2,
                                               0, 0);
  }
};

template <int D, int BS, int NS, int kWaves>
__global__ __launch_bounds__(BS * 2) __attribute__((amdgpu_waves_per_eu(kWaves))) void attn_small_kernel(SmallArgs a) {
  constexpr int UPB = BS / 64;       // 64-key units per key block
  constexpr int KST = D / 16;        // head-dim steps of S^T
  constexpr int NDT = D / 32;        // head-dim tiles of O^T
  constexpr int KRB = D * 2;         // K row bytes in LDS
  constexpr int TCH = 64 * D / 8;    // 16-byte chunks of a K unit tile (= of a V^T unit tile)
  constexpr int NW = BS / 32;        // waves
  constexpr int LPW = TCH / (64 * NW);  // 1 KiB loads per wave per tile
  static_assert(NS == 2 || NS == 3, "ring stages");
  static_assert(TCH % (64 * NW) == 0, "tile loads split evenly over the waves");
  __shared__ uint4 smem[2 * NS * TCH];  // K stages 0 .. NS-1, then V^T stages 0 .. NS-1

  int h, i;  // XCD-aware order: the workgroups an XCD runs together share a kv group
  work_item(blockIdx.x, a.nb, a.Hq, a.Hkv, h, i);
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

  // Load e of wave w moves 1 KiB: lane l writes 16-byte chunk
  // (64 (LPW w + e) + l) of the tile, i.e. row r = that / (row chunks),
  // slot = that % (row chunks), fetching the row's global chunk slot_of(r, .)
  // maps there (an involution).
  UnitLoader<D, BS> ld;
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
    const int vr = ch / 8, vs = ch % 8;
    ld.voff[e] = (uint32_t)(vr * a.Lpad * 2 + slot_of<128>(vr, vs) * 16);
  }

  floatx16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = (floatx16){0};
  float m_run = -INFINITY, l = 0.f;

  // One unit: keys 64 hf .. 64 hf + 63 of key block j, from the tiles sKc
  // (K) and sVc (V^T).
  auto unit_step = [&](int j, int hf, const uint4* sKc, const uint4* sVc) {
    // S^T = K Q^T, two 32-key sub-tiles
    floatx16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int r = 32 * kt + pm;
      s[kt] = (floatx16){0};
#pragma unroll
      for (int st = 0; st < KST; ++st)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(&sKc[r * (KRB / 16) + slot_of<KRB>(r, 2 * st + hh)]), qf[st],
            s[kt], 0, 0, 0);
    }
    if (j == i) mask_diag(s, w, hf, qi, hh);  // causal mask of the diagonal block
    const float mx = pair_max(block_max<2>(s));
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
    uint32_t pw[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * (u & 1) + 2 * e;
        pw[u][e] = pack_pair(exp_one(s[u >> 1][r], c, mu), exp_one(s[u >> 1][r + 1], c, mu), l);
      }
    // O^T += V^T P^T
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int r = 32 * dt + qi;
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(&sVc[r * 8 + slot_of<128>(r, 2 * u + hh)]), as_bf16x8(pw[u]),
            o[dt], 0, 0, 0);
      }
  };

  // NS stages; NS units per trip so each stage's role is static (the loads
  // into one stage and the reads of another then carry addresses the
  // compiler can tell apart, and no wait for the loads in flight is placed
  // before the reads).  entry() is called once per list position, in order:
  // its window only moves forward.
  const int U = cnt * UPB;
  int jst[NS];     // key block of the unit each stage holds
  int j_last = 0;  // key block of the last unit issued
  auto issue = [&](int t, int p) {
    const int hf = UPB == 1 ? 0 : t % UPB;
    if (hf == 0) j_last = entry(t / UPB);
    jst[p] = j_last;
    ld.load(j_last, hf, smem + p * TCH, smem + (NS + p) * TCH);
  };
  // Q and the first list window have landed before the first unit's loads
  // are issued: otherwise the first uses of their registers, inside the
  // loop, would wait for every load in flight on each trip.
  FP_WAIT_VMEM();
#pragma unroll
  for (int p = 0; p + 1 < NS; ++p)
    if (p < U) issue(p, p);
  for (int t0 = 0; t0 < U; t0 += NS) {
#pragma unroll
    for (int p = 0; p < NS; ++p) {
      const int t = t0 + p;
      if (p > 0 && t >= U) break;
      // unit t has landed (with three stages unit t + 1 may still be in
      // flight); after the barrier every wave is done with unit t - 1, whose
      // stage takes unit t + NS - 1
      constexpr int kYoung = 2 * LPW;  // one unit's loads of this wave
      static_assert(kYoung < 64, "vmcnt range");
      if (NS == 3 && t + 1 < U) __builtin_amdgcn_s_waitcnt(0x0070 | (kYoung & 15) | ((kYoung >> 4) << 14));
      else __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int j = jst[p];
      if (t + NS - 1 < U) issue(t + NS - 1, (p + NS - 1) % NS);
      unit_step(j, UPB == 1 ? 0 : t % UPB, smem + p * TCH, smem + (NS + p) * TCH);
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

// Ring stages and the waves per SIMD the registers are sized for, per
// variant (LDS: 2 NS 64 D 2 bytes per workgroup, of 160 KiB per CU).
constexpr int kNs6464 = 2, kWv6464 = 3;
constexpr int kNs64128 = 3, kWv64128 = 3;
constexpr int kNs12864 = 2, kWv12864 = 1;
template __global__ void attn_small_kernel<64, 64, kNs6464, kWv6464>(SmallArgs);
template __global__ void attn_small_kernel<64, 128, kNs64128, kWv64128>(SmallArgs);
template __global__ void attn_small_kernel<128, 64, kNs12864, kWv12864>(SmallArgs);

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
    hipLaunchKernelGGL((attn_small_kernel<64, 64, kNs6464, kWv6464>), grid, dim3(128), 0, st, a);
  else if (dm.d == 64 && dm.B == 128)
    hipLaunchKernelGGL((attn_small_kernel<64, 128, kNs64128, kWv64128>), grid, dim3(256), 0, st, a);
  else if (dm.d == 128 && dm.B == 64)
    hipLaunchKernelGGL((attn_small_kernel<128, 64, kNs12864, kWv12864>), grid, dim3(128), 0, st, a);
  else
    return hipErrorInvalidValue;  // no variant for this shape
  return hipGetLastError();
}
