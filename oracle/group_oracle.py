"""CPU oracle for group-shared selection: one kept-block list per kv group,
shared by the G query heads that read that kv head.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may use it; it imports
nothing from the GPU library.

What the pages say.  [V2] (FlashPrefill V2 abstract) lists PackGQA among the
kernel features: the query heads of one kv group are packed so that a K/V
tile is brought in once for all of them.  That needs one mask per group.
[VS] ("VSPrefill: Vertical-Slash Sparse Attention with Lightweight Indexing
for Long-Context Prefilling", Figure 3) shows that the heads of one kv group
have closely similar sparsity patterns, while different groups do not.  The
pages do not say how a group mask is formed.  The reading taken here is the
union of the heads' own selections:

    keep_g[g, i, j] = OR over heads h of group g of keep[h, i, j]

where keep[h] is the main method's per-head rule (single-pass row max,
S - m >= ln tau, diagonal forced; flashprefill_oracle.select).  Every head
then attends over a superset of its own blocks, so no head loses a block its
own rule keeps; the extra blocks only add exact attention terms.  Lists are
ascending and end with the diagonal, as for one head.

Pins (tests/test_oracle_group.py): with G = 1 the group lists are the
per-head lists; when the G heads of a group carry the same queries the union
equals each head's own selection; hand-built per-head patterns (keys on
basis vectors) give a union that is exactly the union of the patterns; the
union contains every head's set and is contained in the causal triangle;
brute force over tiny inputs; at tau = 0 the group attention equals the dense
textbook attention.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import flashprefill_oracle as O


def group_union(keep: np.ndarray, num_kv_heads: int) -> np.ndarray:
    """keep [Hq, nb, nb] (per head) -> [Hkv, nb, nb], the OR over each group's
    G = Hq / Hkv consecutive heads (head h belongs to group h // G)."""
    Hq, nb, _ = keep.shape
    G = Hq // num_kv_heads
    return keep.reshape(num_kv_heads, G, nb, nb).any(axis=1)


def group_ambiguous(keep: np.ndarray, amb: np.ndarray, num_kv_heads: int) -> np.ndarray:
    """Where the union is decided by rounding: no head keeps the block outside
    its own tie zone, and at least one head has it inside its tie zone.
    Elsewhere the union is fixed whatever the rounding."""
    Hq, nb, _ = keep.shape
    G = Hq // num_kv_heads
    sure = (keep & ~amb).reshape(num_kv_heads, G, nb, nb).any(axis=1)
    some_amb = amb.reshape(num_kv_heads, G, nb, nb).any(axis=1)
    return some_amb & ~sure


def select_group(S: np.ndarray, tau: float, num_kv_heads: int):
    """Per-head threshold (the main rule) then the union per group.
    Returns dict(keep_head, row_max, keep_group [Hkv, nb, nb],
    lists_group [Hkv][nb], lists [Hq][nb] (each head its group's list),
    amb_group)."""
    keep, m = O.select(S, tau)
    amb = O.ambiguous(S, m, tau)
    kg = group_union(keep, num_kv_heads)
    lg = O.block_lists(kg)
    G = S.shape[0] // num_kv_heads
    lists = [lg[h // G] for h in range(S.shape[0])]
    return dict(keep_head=keep, row_max=m, keep_group=kg, lists_group=lg, lists=lists,
                amb_group=group_ambiguous(keep, amb, num_kv_heads))


def prefill_group(q: np.ndarray, k: np.ndarray, v: np.ndarray, block_size: int, tau: float,
                  sm_scale: float = None, attention: bool = True):
    """Pool -> score -> per-head threshold -> group union -> attention of
    every head over its group's list.  Returns the select_group dict plus
    qbar, kbar, S and out."""
    d = q.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    qbar = O.pool(q, block_size)
    kbar = O.pool(k, block_size)
    S = O.block_scores(qbar, kbar, sm_scale)
    r = select_group(S, tau, k.shape[1])
    r.update(qbar=qbar, kbar=kbar, S=S)
    r["out"] = O.sparse_attention(q, k, v, r["lists"], block_size, sm_scale) if attention else None
    return r
