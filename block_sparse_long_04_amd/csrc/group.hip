// Group-shared selection: the kept-block lists of the G = Hq / Hkv query
// heads of one kv group are merged into their union, and the union becomes
// the list of every head of the group.
//
// FlashPrefill V2 abstract (PackGQA: the query heads of a kv group share the
// K/V tiles they read) and VSPrefill, Figure 3 (heads of one kv group have
// closely similar sparsity patterns).  The pages do not say how the group
// mask is formed; the union of the heads' own threshold selections keeps,
// for every head, every block its own rule keeps.
//
// One wave per (kv group g, query block i), heaviest rows first.  The G
// heads' lists (ascending, each within 0..i) are marked in an LDS bitmap of
// i + 1 bits; then the bitmap is compacted 64 blocks at a time (a lane per
// block, positions from the set bits below the lane) and the ascending union
// is written over each head's list, with its count.  A row reads all its
// heads' lists before it writes any of them, and no other wave touches the
// slots of (g, i), so the merge works in place.
#include "common.h"

namespace {

constexpr int kMaxWords = 16384 / 32;  // bitmap words for the largest block count

__global__ __launch_bounds__(64) void group_union_kernel(int Hq, int Hkv, int nb, int* __restrict__ counts,
                                                         int* __restrict__ indices) {
  __shared__ uint32_t bits[kMaxWords];
  const int G = Hq / Hkv;
  const int i = nb - 1 - (int)(blockIdx.x / Hkv);
  const int g = (int)(blockIdx.x % Hkv);
  const int lane = threadIdx.x;
  const int nw = (i >> 5) + 1;
  for (int w = lane; w < nw; w += 64) bits[w] = 0u;
  __syncthreads();
  for (int u = 0; u < G; ++u) {
    const int h = g * G + u;
    const int c = min(counts[(int64_t)h * nb + i], i + 1);  // a row holds at most i + 1 entries
    const int* lst = indices + fpk::tri_offset(h, i, nb);
    for (int e = lane; e < c; e += 64) {
      const int j = lst[e];
      if (j >= 0 && j <= i) atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
  }
  __syncthreads();
  int base = 0;
  for (int j0 = 0; j0 <= i; j0 += 64) {
    const int j = j0 + lane;
    const bool keep = j <= i && ((bits[j >> 5] >> (j & 31)) & 1u);
    const uint64_t b = __ballot(keep);
    if (keep) {
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
      for (int u = 0; u < G; ++u) indices[fpk::tri_offset(g * G + u, i, nb) + pos] = j;
    }
    base += __popcll(b);
  }
  for (int u = lane; u < G; u += 64) counts[(int64_t)(g * G + u) * nb + i] = base;
}

}  // namespace

hipError_t fpk_launch_group_union(const FpDims& dm, int* counts, int* indices, hipStream_t st) {
  if (dm.nb > 16384) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(dm.nb * dm.Hkv));
  hipLaunchKernelGGL(group_union_kernel, grid, dim3(64), 0, st, dm.Hq, dm.Hkv, dm.nb, counts, indices);
  return hipGetLastError();
}
