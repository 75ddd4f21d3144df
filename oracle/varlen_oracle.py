"""CPU oracle for batches of independent sequences (varlen) with K/V packed
or in a paged cache.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may use it; it imports
nothing from the GPU library.

[V2] (FlashPrefill V2 abstract) names serving as the setting: many prompts
of different lengths prefilled together, with K/V in a paged cache.  The
pages give no formula beyond the single-sequence method, so the plainest
reading is taken: each sequence is its own causal prefill, exactly as in
flashprefill_oracle (pooling, scores, threshold, lists and attention over its
own blocks only); a batch changes only where the tokens and pages live.
  * q and out are packed token-major: sequence s owns rows
    cu_seqlens[s] .. cu_seqlens[s+1] - 1.
  * k and v are packed the same way, or held in a cache of pages of
    block_size tokens: block j of sequence s is page block_table[s][j], and
    its first min(block_size, remaining) rows are the sequence's tokens.
  * block lists are local to their sequence (block 0 is the sequence's first).

Pins (tests/test_oracle_varlen.py): at tau = 0 the batch equals one textbook
attention over the packed tokens with the mask "same sequence and not later"
(a formulation that never splits the batch), also cross-checked against torch
CPU scaled_dot_product_attention with that mask; the page gather inverts the
scatter; sequences do not see each other (changing one leaves the others'
lists and outputs unchanged).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np

from oracle import flashprefill_oracle as O


def gather_pages(cache: np.ndarray, table_row: Sequence[int], seq_len: int, block_size: int) -> np.ndarray:
    """The seq_len rows of one sequence from a page cache [pages, B, H, d]."""
    nb = O.num_blocks(seq_len, block_size)
    rows = [cache[int(table_row[j]), : min(block_size, seq_len - j * block_size)] for j in range(nb)]
    return np.concatenate(rows) if rows else cache[:0, 0]


def sequence_kv(k, v, cu_seqlens, s: int, block_size: int, k_cache=None, v_cache=None, table=None):
    """K and V of sequence s, from the packed tensors or the page cache."""
    c0, c1 = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
    if k_cache is None:
        return k[c0:c1], v[c0:c1]
    return (gather_pages(k_cache, table[s], c1 - c0, block_size),
            gather_pages(v_cache, table[s], c1 - c0, block_size))


def prefill_varlen(q: np.ndarray, k: Optional[np.ndarray], v: Optional[np.ndarray],
                   cu_seqlens: Sequence[int], block_size: int, tau: float, sm_scale: float = None,
                   attention: bool = True, k_cache=None, v_cache=None, table=None):
    """Every sequence through flashprefill_oracle.prefill on its own.
    Returns dict(seqs=[per-sequence result dicts], out=packed float64 output)."""
    d = q.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    S = len(cu_seqlens) - 1
    out = np.full(q.shape, np.nan, dtype=np.float64) if attention else None
    seqs = []
    for s in range(S):
        c0, c1 = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        if c1 == c0:  # an empty sequence has no blocks and no output rows
            seqs.append(dict(lists=[], empty=True))
            continue
        ks, vs = sequence_kv(k, v, cu_seqlens, s, block_size, k_cache, v_cache, table)
        r = O.prefill(q[c0:c1], ks, vs, block_size, tau, sm_scale, attention=attention)
        r["k"], r["v"] = ks, vs
        seqs.append(r)
        if attention:
            out[c0:c1] = r["out"]
    return dict(seqs=seqs, out=out)


def dense_varlen_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens: Sequence[int],
                           sm_scale: float) -> np.ndarray:
    """Textbook attention over the packed tokens in float64, with the mask
    "key in the same sequence and not later than the query"; K/V heads are
    repeated for GQA."""
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    seg = np.zeros(T, dtype=np.int64)
    for s in range(len(cu_seqlens) - 1):
        seg[int(cu_seqlens[s]): int(cu_seqlens[s + 1])] = s
    pos = np.arange(T)
    allowed = (seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None])
    out = np.empty((T, Hq, d), dtype=np.float64)
    for h in range(Hq):
        Q = q[:, h].astype(np.float64)
        K = k[:, h // G].astype(np.float64)
        V = v[:, h // G].astype(np.float64)
        lg = np.where(allowed, (Q @ K.T) * sm_scale, -np.inf)
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        out[:, h] = (p / p.sum(axis=1, keepdims=True)) @ V
    return out
