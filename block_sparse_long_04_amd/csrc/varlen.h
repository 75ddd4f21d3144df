// Batch (varlen) metadata shared by the batch kernels and the attention.
#pragma once

#include "common.h"

namespace fpk {

// One block of the batch: its sequence, its index in the sequence, the first
// token of the block in the packed q / out, and its rows (< B only at the end
// of a sequence).
struct VlBlock {
  int seq, jl, tok0, rows;
};

// One sequence: its first block in the batch numbering, its block count, and
// the start of its index lists: row (h, i) of the sequence starts at
// idx_base + h * nb * (nb + 1) / 2 + i * (i + 1) / 2.
struct VlSeq {
  int first, nb;
  long long idx_base;
};

}  // namespace fpk

hipError_t fpk_launch_varlen_prepare(const fp_problem& p, const fp_varlen& vl, const FpDims& dm, int NB,
                                     fpk::VlBlock* blk, fpk::VlSeq* seq, float* q_pool, float* k_pool,
                                     uint8_t* k_c, hipStream_t st);

// V^T [Hkv][d][NB * B] (bf16; e4m3 codes widened) of the batch, zero past
// each sequence's end, from packed or paged v.
hipError_t fpk_launch_vtrans_varlen(const fp_problem& p, const fp_varlen& vl, const FpDims& dm, int NB,
                                    const fpk::VlBlock* blk, uint16_t* v_t, hipStream_t st);

hipError_t fpk_launch_select_varlen(const FpDims& dm, int NB, const fpk::VlBlock* blk, const fpk::VlSeq* seq,
                                    const float* q_pool, const float* k_pool, float sm_scale, float ln_tau,
                                    float* row_max, int* counts, int* indices, hipStream_t st);

hipError_t fpk_launch_attn_mfma_varlen(const fp_problem& p, const FpDims& dm, int NB, const fpk::VlBlock* blk,
                                       const fpk::VlSeq* seq, const int* counts, const int* indices,
                                       const uint8_t* k_c, const uint16_t* v_t, float sm_scale, hipStream_t st);
