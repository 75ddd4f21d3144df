/*
 * flashprefill.h -- C ABI of the block-sparse causal prefill library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the FlashPrefill prefill attention of one layer:
 *   1. mean-pool Q and K into one proxy vector per block of B tokens
 *      ("FlashPrefill: Instantaneous Pattern Discovery for Ultra-Fast
 *      Long-Context Prefilling", skill page: "Architecture Overview",
 *      block-level proxy computation, and the Stage 1 code of
 *      "Implementation Steps");
 *   2. score every causal proxy block pair, S[h,i,j] = Qbar[h,i].Kbar[g,j] *
 *      sm_scale (same Stage 1 code; "Core Concept" item 2);
 *   3. keep key block j of query block i when exp(S[h,i,j] - m[h,i]) >= tau,
 *      m being the single-pass row maximum; the diagonal block is always kept
 *      ("Core Concept" item 3; the FlashPrefill abstract: dynamic thresholding
 *      without sorting or accumulation);
 *   4. compact the kept key blocks of each (head, query block) into an
 *      ascending index list ("Architecture Overview": physical index jumping);
 *   5. exact softmax attention of every query over the keys of its listed
 *      blocks, causal inside the diagonal block, with grouped-query heads
 *      (kv head = q head / (Hq/Hkv)); FP8 inputs as in the FlashPrefill V2
 *      abstract ("FlashPrefill V2: Block-Sparse Prefill Attention for
 *      Long-Context LLM Serving").
 *
 * Conventions shared by every entry point
 *   - Pointers named q, k, v, out and the workspace are DEVICE pointers,
 *     allocated and owned by the caller.  The library never allocates, frees
 *     or keeps them.  The fp_problem struct itself is host memory, read during
 *     the call only.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream).  No call synchronises the host.  A kernel fault surfaces at the
 *     caller's next synchronisation.
 *   - All argument checks run on the host before any launch.  A call that
 *     returns an error has launched nothing and written nothing.
 *   - Tensors are [token, head, dim] views given by element strides; the
 *     last (dim) axis must be contiguous.  Every base pointer must be 16-byte
 *     aligned and every stride a multiple of 16 bytes.
 *   - Functions are re-entrant; the library holds no per-call global state.
 *     Two calls that share a workspace must be ordered on one stream.
 *   - seq_len == 0 is an empty problem: every call returns FP_OK and launches
 *     nothing.
 */
#ifndef FLASHPREFILL_H
#define FLASHPREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k and v.  out is fp32 for FP_F32 and bf16 otherwise.
 * FP_FP8_E4M3 is the OCP e4m3fn format (bias 7, no infinities, max 448),
 * dequantised as code * scale with one scale per tensor. */
typedef enum fp_dtype { FP_F32 = 0, FP_BF16 = 1, FP_FP8_E4M3 = 2 } fp_dtype;

/* Return codes. */
enum {
  FP_OK = 0,
  FP_ERR_INVALID = -1,     /* null pointer, bad shape/stride/alignment, tau outside [0,1] or NaN,
                              non-finite or non-positive scale, Hq not a multiple of Hkv */
  FP_ERR_UNSUPPORTED = -2, /* head_dim not 64/128, block_size not 64/128, causal != 1,
                              more than 16384 blocks */
  FP_ERR_WORKSPACE = -3,   /* workspace null, misaligned (256 B) or smaller than fp_workspace_layout().total */
  FP_ERR_HIP = -4,         /* the HIP runtime refused a launch */
  FP_ERR_SCRATCH = -5      /* fp_prefill_noalloc: the problem's workspace exceeds FP_NOALLOC_SCRATCH_BYTES */
};

/* One layer's prefill problem (batch 1). */
typedef struct fp_problem {
  const void* q;   /* [seq_len, num_q_heads, head_dim] */
  const void* k;   /* [seq_len, num_kv_heads, head_dim] */
  const void* v;   /* [seq_len, num_kv_heads, head_dim] */
  void* out;       /* [seq_len, num_q_heads, head_dim], written by fp_sparse_prefill only */
  int32_t seq_len;
  int32_t num_q_heads;
  int32_t num_kv_heads; /* num_q_heads % num_kv_heads == 0 (grouped-query attention) */
  int32_t head_dim;     /* 64 or 128 */
  int32_t block_size;   /* B: 64 or 128 tokens per block (pooling, selection and attention tile) */
  int64_t q_stride_tok, q_stride_head; /* element strides */
  int64_t k_stride_tok, k_stride_head;
  int64_t v_stride_tok, v_stride_head;
  int64_t o_stride_tok, o_stride_head; /* out must not overlap itself */
  int32_t dtype;        /* fp_dtype */
  float q_scale, k_scale, v_scale; /* fp8 dequantisation scales; ignored (taken as 1) otherwise */
  float sm_scale;       /* softmax / proxy-score scale; <= 0 selects 1/sqrt(head_dim) */
  float threshold;      /* tau in [0, 1]: keep block j iff exp(S_ij - m_i) >= tau; 0 keeps every causal block */
  int32_t causal;       /* must be 1: causal prefill */
} fp_problem;

/* Byte offsets of the workspace sections (each 256-byte aligned) and the
 * total size.  nb = ceil(seq_len / block_size).
 *   q_pool  float [num_q_heads][nb][head_dim]   pooled query proxies (scaled by q_scale)
 *   k_pool  float [num_kv_heads][nb][head_dim]  pooled key proxies (scaled by k_scale)
 *   row_max float [num_q_heads][nb]             m[h,i] = max_{j<=i} S[h,i,j]
 *   counts  int32 [num_q_heads][nb]             kept blocks of row (h,i)
 *   indices int32, triangular: row (h,i) starts at h*nb*(nb+1)/2 + i*(i+1)/2, holds
 *           counts[h][i] ascending key-block indices (capacity i+1)
 *   v_t     bf16 [num_kv_heads][head_dim][nb*block_size]  scratch of fp_sparse_prefill: V
 *           transposed per kv head (the key-contiguous rows its P.V products read), zero past
 *           seq_len; e4m3 codes widened to bf16 exactly, v_scale applied at the output
 *           (zero-length unless the attention runs on the matrix cores: bf16 or e4m3 with
 *           head_dim 128 and block_size 128, or bf16 with head_dim and block_size in {64, 128})
 * The layout is part of the ABI: a caller may read the selection, or write
 * its own counts/indices (ascending, each list ending with its diagonal
 * block i) before fp_sparse_prefill to run attention on a given mask. */
typedef struct fp_ws_layout {
  size_t q_pool, k_pool, row_max, counts, indices, v_t, total;
} fp_ws_layout;

/* Host only, launches nothing: validates *p (pointers may be NULL here) and
 * fills *layout.  Returns FP_OK or an error code. */
int fp_workspace_layout(const fp_problem* p, fp_ws_layout* layout);

/* Step 1.  Reads q and k and writes the q_pool and k_pool sections. */
int fp_block_pool(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream);

/* Steps 2-4.  Reads q_pool, k_pool; writes row_max, counts and indices.  The
 * block score matrix is never stored. */
int fp_block_select(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream);

/* Group-shared selection: one list per kv group, shared by its G = Hq/Hkv
 * query heads (FlashPrefill V2 abstract: PackGQA, the heads of a group read
 * the same K/V tiles; VSPrefill, Figure 3: heads of one kv group select
 * closely similar blocks).  Each head first selects with its own threshold
 * exactly as fp_block_select (row_max keeps each head's own maximum); then
 * the union of the G heads' kept blocks of each (group, query block) is
 * written as the list and count of every head of the group (ascending, ending
 * with the diagonal).  Every head thus attends over a superset of its own
 * selection, and the G workgroups of one (group, query block) walk identical
 * lists, so each K/V tile they read is fetched once into L2 for all of them.
 * fp_sparse_prefill runs on the result unchanged.  With G = 1 this is
 * fp_block_select.  Same sections, arguments and errors as fp_block_select. */
int fp_block_select_group(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream);

/* Selection rules that sort the block scores or accumulate their mass: the
 * baselines the single-pass threshold avoids (FlashPrefill skill page, "Core
 * Concept"; FlashPrefill abstract).  Same sections as fp_block_select: reads
 * q_pool and k_pool, writes row_max, counts and indices (so fp_sparse_prefill
 * runs on the result), with another keep rule per row (h, i) over the causal
 * blocks j <= i of the same scores S:
 *   FP_SELECT_TOPK: the k (= param, a whole number >= 1) largest scores;
 *   FP_SELECT_TOPP: the shortest prefix in descending score order whose block
 *                   softmax mass exp(S - m) / sum exp(S - m) reaches p
 *                   (= param, in (0, 1]);
 * among equal scores the smaller block index first; the diagonal block is
 * kept as well.  p->threshold is not used.  Rows are sorted whole in LDS, so
 * nb <= 2048 (FP_ERR_UNSUPPORTED beyond); a bad rule or param is
 * FP_ERR_INVALID. */
typedef enum { FP_SELECT_TOPK = 1, FP_SELECT_TOPP = 2 } fp_select_rule;
int fp_block_select_sorted(const fp_problem* p, int rule, float param, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Query-probe reading of stage 1 (FlashPrefill skill page, "Core Concept":
 * query probes, search cost O(L^2/B) against O((L/B)^2)): the pooled probe of
 * query block i scored against every key token t of block j, reduced by the
 * max, S'[h,i,j] = max_t (Qbar[h,i] . k[t]) * sm_scale, then the same
 * threshold, diagonal and lists as fp_block_select.  Reads q_pool (from
 * fp_block_pool) and k; writes row_max (of S'), counts and indices.  For bf16
 * and e4m3 inputs with head_dim 128 and block_size 128, nb <= 1024
 * (FP_ERR_UNSUPPORTED otherwise). */
int fp_block_select_probe(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream);

/* Step 5.  Reads q, k, v, counts and indices; writes out.  On the matrix
 * cores (bf16 or e4m3 with head_dim 128 and block_size 128; bf16 with
 * head_dim and block_size in {64, 128}) it first writes the v_t section from
 * v, which its attention kernel then reads; other layers (fp32 inputs, e4m3
 * with head_dim or block_size 64) run on the vector ALUs. */
int fp_sparse_prefill(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream);

/* Step 5 with the two query heads of a pair (2p, 2p+1) of one kv group served
 * by one workgroup (FlashPrefill V2 abstract: PackGQA, the query heads of a kv
 * group share the K/V tiles they read): each K and V tile is staged into LDS
 * once for both heads, and every operand fragment read from LDS feeds both
 * heads' matrix products.  Each head still attends over exactly its own list:
 * the kernel walks the union of the pair's lists and gives a head zero weight
 * on a block its own list lacks.  Same inputs, workspace and result as
 * fp_sparse_prefill (any lists, per-head or group-shared); bf16 inputs with
 * head_dim 128, block_size 128 and an even num_q_heads / num_kv_heads only
 * (FP_ERR_UNSUPPORTED otherwise).  It halves the LDS operand reads and the
 * tile loads of fp_sparse_prefill per product but runs one wave per SIMD
 * (its registers allow no second), and on MI355X it is slower than
 * fp_sparse_prefill, which remains the default. */
int fp_sparse_prefill_pack(const fp_problem* p, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Batches of independent sequences (varlen), K/V packed or paged.
 *
 * FlashPrefill V2 abstract: the method serves many prompts prefilled together
 * with K/V in a paged cache.  Each sequence is its own causal prefill (the
 * steps above on its own tokens and blocks); only where the tokens live
 * changes.  p->seq_len is the total token count T of q / out, which are packed
 * token-major: sequence s owns rows cu_seqlens[s] .. cu_seqlens[s+1]-1.  k / v
 * are packed the same way when block_table_dev is NULL; otherwise p->k / p->v
 * point at page caches whose page of block_size tokens starts every
 * k_page_stride / v_page_stride elements, token r of a page at
 * r * k_stride_tok + head * k_stride_head inside it, and block j of sequence s
 * is page block_table_dev[s * max_blocks + j] (ids outside [0, num_pages) read
 * as zero pages).  Supported for bf16 and e4m3 inputs with head_dim 128 and
 * block_size 128 (FP_ERR_UNSUPPORTED otherwise); at most 16384 blocks in all.
 * --------------------------------------------------------------------------- */
typedef struct fp_varlen {
  int32_t num_seqs;                /* S >= 1 */
  const int32_t* cu_seqlens;       /* host [S + 1]: 0 = cu[0] <= cu[1] <= ... <= cu[S] = p->seq_len */
  const int32_t* cu_seqlens_dev;   /* the same S + 1 values in device memory */
  const int32_t* block_table_dev;  /* NULL (packed k / v) or device [S][max_blocks] page ids */
  int32_t max_blocks;              /* row stride of the block table (>= every sequence's block count) */
  int32_t num_pages;               /* pages in each cache */
  int64_t k_page_stride, v_page_stride;  /* elements between pages */
} fp_varlen;

/* Workspace of a batch, NB = sum over s of ceil(len_s / block_size) blocks.
 *   q_pool, k_pool, row_max, counts, v_t: as for one sequence over the NB
 *           blocks of the batch in order (sequence s's blocks first[s] ..
 *           first[s] + nb[s] - 1, first[s] = sum of the earlier nb);
 *   indices: sequence s's lists start at idx_base[s] = num_q_heads * (sum of
 *           nb[s'] (nb[s'] + 1) / 2 over s' < s); within it row (h, i) at
 *           h * nb[s] (nb[s] + 1) / 2 + i * (i + 1) / 2; entries are block
 *           indices local to the sequence (0 = its first block);
 *   k_c     K gathered per kv head [num_kv_heads][NB * block_size][head_dim]
 *           (input dtype, zero past each sequence's end);
 *   meta    per block int32 x4 (sequence, block in sequence, first token in q / out,
 *           rows), then per sequence int32 first, int32 nb, int64 idx_base. */
typedef struct fp_ws_layout_varlen {
  size_t q_pool, k_pool, row_max, counts, indices, v_t, k_c, meta, total;
} fp_ws_layout_varlen;

/* Host only: validates *p and *vl (vl->cu_seqlens is read; device pointers
 * may be NULL here) and fills *layout. */
int fp_workspace_layout_varlen(const fp_problem* p, const fp_varlen* vl, fp_ws_layout_varlen* layout);

/* Step 1 of every sequence: block metadata, pooled proxies and gathered K
 * (reads q, k and cu_seqlens_dev / block_table_dev). */
int fp_block_pool_varlen(const fp_problem* p, const fp_varlen* vl, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Steps 2-4 of every sequence (rows see only their own sequence's blocks). */
int fp_block_select_varlen(const fp_problem* p, const fp_varlen* vl, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Step 5 of every sequence: V^T of the batch into the v_t section (from v,
 * packed or paged), then the attention; writes out.  Must follow
 * fp_block_pool_varlen (block metadata, gathered K) and a selection on the
 * same workspace. */
int fp_sparse_prefill_varlen(const fp_problem* p, const fp_varlen* vl, void* workspace, size_t workspace_bytes,
                             void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): steps 1-5
 * of one layer -- fp_block_pool, fp_block_select and fp_sparse_prefill, the
 * same kernels and results -- with the workspace held in a buffer of
 * FP_NOALLOC_SCRATCH_BYTES that the library itself keeps in device memory (one
 * per GPU, created when the library's code is loaded on that GPU and held until
 * the process ends).  The caller passes q, k, v and out as for the three
 * calls; nothing is allocated or freed, and the selection stays inside the
 * library (it cannot be read or injected).  Problems whose
 * fp_workspace_layout().total exceeds FP_NOALLOC_SCRATCH_BYTES are rejected
 * with FP_ERR_SCRATCH before any launch (at 32 query / 8 kv heads, head_dim
 * and block_size 128, that allows sequences up to 28672 tokens).  Every call on
 * one GPU uses that GPU's one buffer: calls that overlap in time on a GPU
 * (other streams, other host threads) race and must be ordered by the caller.
 * No part of the buffer needs to start at zero: each call writes every section
 * before it reads it. */
#define FP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fp_prefill_noalloc(const fp_problem* p, void* stream);

/* Static, human-readable text of a return code. */
const char* fp_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* FLASHPREFILL_H */
