// C ABI of the block-sparse prefill library: argument checks, workspace
// carving and stream-ordered launches.  Declarations and the meaning of every
// argument are in include/flashprefill.h.
#include <math.h>
#include <string.h>

#include <mutex>

#include "common.h"
#include "varlen.h"

// group.hip: union of the G heads' lists of each (kv group, query block),
// written back as the list of every head of the group (in place).
hipError_t fpk_launch_group_union(const FpDims& dm, int* counts, int* indices, hipStream_t st);

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxBlocks = 16384;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

int elem_size(int dtype) { return dtype == FP_F32 ? 4 : (dtype == FP_BF16 ? 2 : 1); }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Non-overlap of an output [L][H][d] view with element strides (st, sh).
bool out_view_ok(int64_t st, int64_t sh, int L, int H, int d) {
  if (st <= 0 || sh <= 0) return false;
  const bool tok_major = sh >= d && (L == 1 || st >= (int64_t)H * sh);
  const bool head_major = st >= d && (H == 1 || sh >= (int64_t)L * st);
  return tok_major || head_major;
}

// Shape/scalar checks common to every entry point (pointers are checked by
// each entry point for the tensors it touches).
int check_problem(const fp_problem* p, FpDims* dm) {
  if (!p) return FP_ERR_INVALID;
  if (p->seq_len < 0 || p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0 ||
      p->block_size <= 0)
    return FP_ERR_INVALID;
  if (p->num_q_heads % p->num_kv_heads != 0) return FP_ERR_INVALID;
  if (p->dtype != FP_F32 && p->dtype != FP_BF16 && p->dtype != FP_FP8_E4M3) return FP_ERR_INVALID;
  if (isnan(p->threshold) || p->threshold < 0.f || p->threshold > 1.f) return FP_ERR_INVALID;
  if (isnan(p->sm_scale) || isinf(p->sm_scale)) return FP_ERR_INVALID;
  if (p->dtype == FP_FP8_E4M3) {
    const float sc[3] = {p->q_scale, p->k_scale, p->v_scale};
    for (float s : sc)
      if (!(s > 0.f) || isinf(s)) return FP_ERR_INVALID;
  }
  if (p->causal != 1) return FP_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return FP_ERR_UNSUPPORTED;
  if (p->block_size != 64 && p->block_size != 128) return FP_ERR_UNSUPPORTED;
  const int64_t nb = ((int64_t)p->seq_len + p->block_size - 1) / p->block_size;
  if (nb > kMaxBlocks) return FP_ERR_UNSUPPORTED;
  const int es = elem_size(p->dtype);
  const int64_t st[6] = {p->q_stride_tok, p->q_stride_head, p->k_stride_tok,
                         p->k_stride_head, p->v_stride_tok, p->v_stride_head};
  for (int64_t s : st)
    if (s <= 0 || (s * es) % 16 != 0) return FP_ERR_INVALID;
  const int oes = p->dtype == FP_F32 ? 4 : 2;
  if (!out_view_ok(p->o_stride_tok, p->o_stride_head, p->seq_len, p->num_q_heads, p->head_dim) ||
      (p->o_stride_tok * oes) % 16 != 0 || (p->o_stride_head * oes) % 16 != 0)
    return FP_ERR_INVALID;
  dm->L = p->seq_len;
  dm->Hq = p->num_q_heads;
  dm->Hkv = p->num_kv_heads;
  dm->d = p->head_dim;
  dm->B = p->block_size;
  dm->nb = (int)nb;
  return FP_OK;
}

// The matrix-core attention serves bf16 and e4m3 inputs with d = B = 128.
// It addresses K one key block at a time through 32-bit buffer offsets, so
// the 128 rows of a block must span less than 2^31 bytes; token strides
// beyond that (16 MiB per token) go to the generic kernel.
bool use_mfma(const fp_problem* p, const FpDims& dm) {
  if (p->dtype == FP_F32 || dm.d != 128 || dm.B != 128) return false;
  const int64_t esz = p->dtype == FP_BF16 ? 2 : 1;
  return (int64_t)dm.B * p->k_stride_tok * esz + dm.d * esz < (int64_t(1) << 31);
}

// bf16 layers with head_dim or block_size 64 (d, B in {64, 128}, not both
// 128: that shape takes attn_mfma.hip) take the matrix-core kernel of
// attn_small.hip.  Its K buffer resources span one 64-key unit, so the same
// 31-bit extent limit applies to 64 rows.
bool use_small(const fp_problem* p, const FpDims& dm) {
  if (p->dtype != FP_BF16 || (dm.d == 128 && dm.B == 128)) return false;
  if (!((dm.d == 64 || dm.d == 128) && (dm.B == 64 || dm.B == 128))) return false;
  return (int64_t)64 * p->k_stride_tok * 2 + dm.d * 2 < (int64_t(1) << 31);
}

void layout_of(const fp_problem* p, const FpDims& dm, fp_ws_layout* w) {
  const size_t nb = (size_t)dm.nb;
  size_t off = 0;
  w->q_pool = off;
  off = align_up(off + (size_t)dm.Hq * nb * dm.d * sizeof(float));
  w->k_pool = off;
  off = align_up(off + (size_t)dm.Hkv * nb * dm.d * sizeof(float));
  w->row_max = off;
  off = align_up(off + (size_t)dm.Hq * nb * sizeof(float));
  w->counts = off;
  off = align_up(off + (size_t)dm.Hq * nb * sizeof(int));
  w->indices = off;
  off = align_up(off + (size_t)dm.Hq * (nb * (nb + 1) / 2) * sizeof(int));
  w->v_t = off;
  if (use_mfma(p, dm) || use_small(p, dm))
    off = align_up(off + (size_t)dm.Hkv * dm.d * nb * dm.B * sizeof(uint16_t));
  w->total = off;
}


int check_ws(const fp_problem* p, const FpDims& dm, void* ws, size_t bytes, fp_ws_layout* w) {
  layout_of(p, dm, w);
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0 || bytes < w->total)
    return FP_ERR_WORKSPACE;
  return FP_OK;
}

float eff_sm_scale(const fp_problem* p) {
  return p->sm_scale > 0.f ? p->sm_scale : (float)(1.0 / sqrt((double)p->head_dim));
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}


// ---- batches (varlen) ------------------------------------------------------

struct VlInfo {
  int NB;             // blocks of the batch
  int64_t idx_total;  // int32 entries of all index lists
};

// Checks of *vl against *p (host side: cu_seqlens is read here).
int check_varlen(const fp_problem* p, const fp_varlen* vl, const FpDims& dm, VlInfo* vi) {
  if (!vl || vl->num_seqs < 1 || !vl->cu_seqlens) return FP_ERR_INVALID;
  if (p->dtype == FP_F32 || dm.d != 128 || dm.B != 128) return FP_ERR_UNSUPPORTED;
  const int32_t* cu = vl->cu_seqlens;
  if (cu[0] != 0 || cu[vl->num_seqs] != p->seq_len) return FP_ERR_INVALID;
  int64_t nb_all = 0, tri = 0, nb_max = 0;
  for (int s = 0; s < vl->num_seqs; ++s) {
    if (cu[s + 1] < cu[s]) return FP_ERR_INVALID;
    const int64_t nbs = ((int64_t)cu[s + 1] - cu[s] + dm.B - 1) / dm.B;
    nb_all += nbs;
    tri += nbs * (nbs + 1) / 2;
    nb_max = nbs > nb_max ? nbs : nb_max;
  }
  if (nb_all > kMaxBlocks) return FP_ERR_UNSUPPORTED;
  if (vl->block_table_dev) {
    const int es = elem_size(p->dtype);
    if (vl->max_blocks < nb_max || vl->num_pages < 1 || vl->k_page_stride <= 0 || vl->v_page_stride <= 0 ||
        (vl->k_page_stride * es) % 16 != 0 || (vl->v_page_stride * es) % 16 != 0)
      return FP_ERR_INVALID;
  }
  vi->NB = (int)nb_all;
  vi->idx_total = tri * dm.Hq;
  return FP_OK;
}

void layout_varlen(const fp_problem* p, const FpDims& dm, const VlInfo& vi, int S, fp_ws_layout_varlen* w) {
  const size_t NB = (size_t)vi.NB;
  size_t off = 0;
  w->q_pool = off;
  off = align_up(off + (size_t)dm.Hq * NB * dm.d * sizeof(float));
  w->k_pool = off;
  off = align_up(off + (size_t)dm.Hkv * NB * dm.d * sizeof(float));
  w->row_max = off;
  off = align_up(off + (size_t)dm.Hq * NB * sizeof(float));
  w->counts = off;
  off = align_up(off + (size_t)dm.Hq * NB * sizeof(int));
  w->indices = off;
  off = align_up(off + (size_t)vi.idx_total * sizeof(int));
  w->v_t = off;
  off = align_up(off + (size_t)dm.Hkv * dm.d * NB * dm.B * sizeof(uint16_t));
  w->k_c = off;
  off = align_up(off + (size_t)dm.Hkv * NB * dm.B * dm.d * elem_size(p->dtype));
  w->meta = off;
  off = align_up(off + NB * sizeof(fpk::VlBlock) + (size_t)S * sizeof(fpk::VlSeq));
  w->total = NB == 0 ? 0 : off;
}

int check_ws_varlen(const fp_problem* p, const fp_varlen* vl, FpDims* dm, VlInfo* vi, void* ws, size_t bytes,
                    fp_ws_layout_varlen* w) {
  int rc = check_problem(p, dm);
  if (rc != FP_OK) return rc;
  rc = check_varlen(p, vl, *dm, vi);
  if (rc != FP_OK) return rc;
  layout_varlen(p, *dm, *vi, vl->num_seqs, w);
  if (vi->NB == 0) return FP_OK;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0 || bytes < w->total)
    return FP_ERR_WORKSPACE;
  return FP_OK;
}

}  // namespace

// ---- fixed scratch buffer of fp_prefill_noalloc -----------------------------
// The workspace of callers that cannot allocate.  Each GPU the library's code
// is loaded on holds its own copy at its own address; host code never uses
// the array's name as an address (it names a host-side stand-in), only the
// per-device address from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[FP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, queried once per device
// with that device current.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FP_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FP_OK;
}

}  // namespace

extern "C" {

int fp_prefill_noalloc(const fp_problem* p, void* stream) {
  FpDims dm;
  int rc = check_problem(p, &dm);
  if (rc != FP_OK) return rc;
  if (dm.L == 0) return FP_OK;
  if (!p->q || !p->k || !p->v || !p->out || !aligned16(p->q) || !aligned16(p->k) ||
      !aligned16(p->v) || !aligned16(p->out))
    return FP_ERR_INVALID;
  fp_ws_layout w;
  layout_of(p, dm, &w);
  if (w.total > FP_NOALLOC_SCRATCH_BYTES) return FP_ERR_SCRATCH;
  void* ws = nullptr;
  rc = scratch_on_current_device(&ws);
  if (rc != FP_OK) return rc;
  rc = fp_block_pool(p, ws, FP_NOALLOC_SCRATCH_BYTES, stream);
  if (rc == FP_OK) rc = fp_block_select(p, ws, FP_NOALLOC_SCRATCH_BYTES, stream);
  if (rc == FP_OK) rc = fp_sparse_prefill(p, ws, FP_NOALLOC_SCRATCH_BYTES, stream);
  return rc;
}

int fp_workspace_layout(const fp_problem* p, fp_ws_layout* layout) {
  FpDims dm;
  const int rc = check_problem(p, &dm);
  if (rc != FP_OK) return rc;
  if (!layout) return FP_ERR_INVALID;
  layout_of(p, dm, layout);
  return FP_OK;
}

int fp_block_pool(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream) {
  FpDims dm;
  int rc = check_problem(p, &dm);
  if (rc != FP_OK) return rc;
  if (dm.L == 0) return FP_OK;
  if (!p->q || !p->k || !aligned16(p->q) || !aligned16(p->k)) return FP_ERR_INVALID;
  fp_ws_layout w;
  rc = check_ws(p, dm, workspace, workspace_bytes, &w);
  if (rc != FP_OK) return rc;
  const hipError_t e = fpk_launch_pool(*p, dm, at<float>(workspace, w.q_pool), at<float>(workspace, w.k_pool),
                                       (hipStream_t)stream);
  return e == hipSuccess ? FP_OK : FP_ERR_HIP;
}

int fp_block_select(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream) {
  FpDims dm;
  int rc = check_problem(p, &dm);
  if (rc != FP_OK) return rc;
  if (dm.L == 0) return FP_OK;
  fp_ws_layout w;
  rc = check_ws(p, dm, workspace, workspace_bytes, &w);
  if (rc != FP_OK) return rc;
  const float lt = p->threshold == 0.f ? -INFINITY : (float)log((double)p->threshold);
  const hipError_t e =
      fpk_launch_select(dm, at<float>(workspace, w.q_pool), at<float>(workspace, w.k_pool),
                        eff_sm_scale(p), lt, at<float>(workspace, w.row_max),
                        at<int>(workspace, w.counts), at<int>(workspace, w.indices),
                        (hipStream_t)stream);
  return e == hipSuccess ? FP_OK : FP_ERR_HIP;
}

int fp_block_select_group(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream) {
  FpDims dm;
  int rc = check_problem(p, &dm);
  if (rc != FP_OK) return rc;
  if (dm.L == 0) return FP_OK;
  fp_ws_layout w;
  rc = check_ws(p, dm, workspace, workspace_bytes, &w);
  if (rc != FP_OK) return rc;
  const float lt = p->threshold == 0.f ? -INFINITY : (float)log((double)p->threshold);
  hipError_t e =
      fpk_launch_select(dm, at<float>(workspace, w.q_pool), at<float>(workspace, w.k_pool),
                        eff_sm_scale(p), lt, at<float>(workspace, w.row_max),
                        at<int>(workspace, w.counts), at<int>(workspace, w.indices),
                        (hipStream_t)stream);
  if (e == hipSuccess && dm.Hq > dm.Hkv)
    e = fpk_launch_group_union(dm, at<int>(workspace, w.counts), at<int>(workspace, w.indices),
                               (hipStream_t)stream);
  return e == hipSuccess ? FP_OK : FP_ERR_HIP;
}

int fp_block_select_sorted(const fp_problem* p, int rule, float param, void* workspace,
                           size_t workspace_bytes, void* stream) {
  FpDims dm;
  int rc = check_problem(p, &dm);
  if (rc != FP_OK) return rc;
  if (rule == FP_SELECT_TOPK) {
    if (!(param >= 1.0f && param <= 16777216.0f && param == floorf(param))) return FP_ERR_INVALID;
  } else if (rule == FP_SELECT_TOPP) {
    if (!(param > 0.0f && param <= 1.0f)) return FP_ERR_INVALID;
  } else {
    return FP_ERR_INVALID;
  }
  if (dm.nb > 2048) return FP_ERR_UNSUPPORTED;
  if (dm.L == 0) return FP_OK;
  fp_ws_layout w;
  rc = check_ws(p, dm, workspace, workspace_bytes, &w);
  if (rc != FP_OK) return rc;
  const hipError_t e = fpk_launch_select_sorted(
      dm, at<float>(workspace, w.q_pool), at<float>(workspace, w.k_pool), eff_sm_scale(p), rule, param,
      at<float>(workspace, w.row_max), at<int>(workspace, w.counts), at<int>(workspace, w.indices),
      (hipStream_t)stream);
  return e == hipSuccess ? FP_OK : FP_ERR_HIP;
}

int fp_block_select_probe(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream) {
  FpDims dm;
  int rc = check_problem(p, &dm);
  if (rc != FP_OK) return rc;
  if (p->dtype == FP_F32 || dm.d != 128 || dm.B != 128 || dm.nb > 1024) return FP_ERR_UNSUPPORTED;
  if (dm.L == 0) return FP_OK;
  if (!p->k || !aligned16(p->k)) return FP_ERR_INVALID;
  fp_ws_layout w;
  rc = check_ws(p, dm, workspace, workspace_bytes, &w);
  if (rc != FP_OK) return rc;
  const float lt = p->threshold == 0.f ? -INFINITY : (float)log((double)p->threshold);
  const hipError_t e = fpk_launch_probe_select(*p, dm, at<float>(workspace, w.q_pool), eff_sm_scale(p), lt,
                                               at<float>(workspace, w.row_max), at<int>(workspace, w.counts),
                                               at<int>(workspace, w.indices), (hipStream_t)stream);
  return e == hipSuccess ? FP_OK : FP_ERR_HIP;
}

int fp_sparse_prefill(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream) {
  FpDims dm;
  int rc = check_problem(p, &dm);
  if (rc != FP_OK) return rc;
  if (dm.L == 0) return FP_OK;
  if (!p->q || !p->k || !p->v || !p->out || !aligned16(p->q) || !aligned16(p->k) ||
      !aligned16(p->v) || !aligned16(p->out))
    return FP_ERR_INVALID;
  fp_ws_layout w;
  rc = check_ws(p, dm, workspace, workspace_bytes, &w);
  if (rc != FP_OK) return rc;
  const hipStream_t st = (hipStream_t)stream;
  const float sc = eff_sm_scale(p);
  const int* counts = at<int>(workspace, w.counts);
  const int* indices = at<int>(workspace, w.indices);
  hipError_t e;
  if (use_mfma(p, dm)) {
    // V^T is this call's own scratch: written here from v, then read by the
    // attention (key-contiguous rows for the P.V operands)
    uint16_t* v_t = at<uint16_t>(workspace, w.v_t);
    e = fpk_launch_vtrans(*p, dm, v_t, st);
    if (e == hipSuccess) e = fpk_launch_attn_mfma(*p, dm, counts, indices, v_t, sc, st);
  } else if (use_small(p, dm)) {
    uint16_t* v_t = at<uint16_t>(workspace, w.v_t);
    e = fpk_launch_vtrans(*p, dm, v_t, st);
    if (e == hipSuccess) e = fpk_launch_attn_small(*p, dm, counts, indices, v_t, sc, st);
  } else {
    e = fpk_launch_attn_generic(*p, dm, counts, indices, sc, st);
  }
  return e == hipSuccess ? FP_OK : FP_ERR_HIP;
}

int fp_sparse_prefill_pack(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream) {
  FpDims dm;
  int rc = check_problem(p, &dm);
  if (rc != FP_OK) return rc;
  if (p->dtype != FP_BF16 || !use_mfma(p, dm) || (dm.Hq / dm.Hkv) % 2 != 0) return FP_ERR_UNSUPPORTED;
  if (dm.L == 0) return FP_OK;
  if (!p->q || !p->k || !p->v || !p->out || !aligned16(p->q) || !aligned16(p->k) ||
      !aligned16(p->v) || !aligned16(p->out))
    return FP_ERR_INVALID;
  fp_ws_layout w;
  rc = check_ws(p, dm, workspace, workspace_bytes, &w);
  if (rc != FP_OK) return rc;
  const hipStream_t st = (hipStream_t)stream;
  uint16_t* v_t = at<uint16_t>(workspace, w.v_t);
  hipError_t e = fpk_launch_vtrans(*p, dm, v_t, st);
  if (e == hipSuccess)
    e = fpk_launch_attn_pack(*p, dm, at<int>(workspace, w.counts), at<int>(workspace, w.indices), v_t,
                             eff_sm_scale(p), st);
  return e == hipSuccess ? FP_OK : FP_ERR_HIP;
}

int fp_workspace_layout_varlen(const fp_problem* p, const fp_varlen* vl, fp_ws_layout_varlen* layout) {
  FpDims dm;
  int rc = check_problem(p, &dm);
  if (rc != FP_OK) return rc;
  VlInfo vi;
  rc = check_varlen(p, vl, dm, &vi);
  if (rc != FP_OK) return rc;
  if (!layout) return FP_ERR_INVALID;
  layout_varlen(p, dm, vi, vl->num_seqs, layout);
  return FP_OK;
}

int fp_block_pool_varlen(const fp_problem* p, const fp_varlen* vl, void* workspace, size_t workspace_bytes,
                         void* stream) {
  FpDims dm;
  VlInfo vi;
  fp_ws_layout_varlen w;
  int rc = check_ws_varlen(p, vl, &dm, &vi, workspace, workspace_bytes, &w);
  if (rc != FP_OK) return rc;
  if (vi.NB == 0) return FP_OK;
  if (!p->q || !p->k || !aligned16(p->q) || !aligned16(p->k) || !vl->cu_seqlens_dev) return FP_ERR_INVALID;
  const hipError_t e = fpk_launch_varlen_prepare(
      *p, *vl, dm, vi.NB, at<fpk::VlBlock>(workspace, w.meta),
      reinterpret_cast<fpk::VlSeq*>(at<fpk::VlBlock>(workspace, w.meta) + vi.NB), at<float>(workspace, w.q_pool),
      at<float>(workspace, w.k_pool), at<uint8_t>(workspace, w.k_c), (hipStream_t)stream);
  return e == hipSuccess ? FP_OK : FP_ERR_HIP;
}

int fp_block_select_varlen(const fp_problem* p, const fp_varlen* vl, void* workspace, size_t workspace_bytes,
                           void* stream) {
  FpDims dm;
  VlInfo vi;
  fp_ws_layout_varlen w;
  int rc = check_ws_varlen(p, vl, &dm, &vi, workspace, workspace_bytes, &w);
  if (rc != FP_OK) return rc;
  if (vi.NB == 0) return FP_OK;
  const float lt = p->threshold == 0.f ? -INFINITY : (float)log((double)p->threshold);
  const fpk::VlBlock* blk = at<fpk::VlBlock>(workspace, w.meta);
  const hipError_t e = fpk_launch_select_varlen(
      dm, vi.NB, blk, reinterpret_cast<const fpk::VlSeq*>(blk + vi.NB), at<float>(workspace, w.q_pool),
      at<float>(workspace, w.k_pool), eff_sm_scale(p), lt, at<float>(workspace, w.row_max),
      at<int>(workspace, w.counts), at<int>(workspace, w.indices), (hipStream_t)stream);
  return e == hipSuccess ? FP_OK : FP_ERR_HIP;
}

int fp_sparse_prefill_varlen(const fp_problem* p, const fp_varlen* vl, void* workspace, size_t workspace_bytes,
                             void* stream) {
  FpDims dm;
  VlInfo vi;
  fp_ws_layout_varlen w;
  int rc = check_ws_varlen(p, vl, &dm, &vi, workspace, workspace_bytes, &w);
  if (rc != FP_OK) return rc;
  if (vi.NB == 0) return FP_OK;
  if (!p->q || !p->v || !p->out || !aligned16(p->q) || !aligned16(p->v) || !aligned16(p->out))
    return FP_ERR_INVALID;
  const fpk::VlBlock* blk = at<fpk::VlBlock>(workspace, w.meta);
  // V^T of the batch (this call's own scratch), from packed or paged v
  hipError_t e = fpk_launch_vtrans_varlen(*p, *vl, dm, vi.NB, blk, at<uint16_t>(workspace, w.v_t),
                                          (hipStream_t)stream);
  if (e == hipSuccess) e = fpk_launch_attn_mfma_varlen(
      *p, dm, vi.NB, blk, reinterpret_cast<const fpk::VlSeq*>(blk + vi.NB), at<int>(workspace, w.counts),
      at<int>(workspace, w.indices), at<uint8_t>(workspace, w.k_c), at<uint16_t>(workspace, w.v_t),
      eff_sm_scale(p), (hipStream_t)stream);
  return e == hipSuccess ? FP_OK : FP_ERR_HIP;
}

const char* fp_strerror(int code) {
  switch (code) {
    case FP_OK: return "ok";
    case FP_ERR_INVALID: return "invalid argument (pointer, shape, stride, alignment, scale or threshold)";
    case FP_ERR_UNSUPPORTED: return "unsupported configuration (head_dim, block_size, causal or block count)";
    case FP_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case FP_ERR_HIP: return "HIP launch failed";
    case FP_ERR_SCRATCH: return "problem too large for the library's fixed scratch buffer (fp_prefill_noalloc)";
    default: return "unknown error code";
  }
}

}  // extern "C"
