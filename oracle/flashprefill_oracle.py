"""CPU oracle for FlashPrefill-style block-sparse causal prefill attention.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously-correct
definition the GPU library is checked against.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the GPU library never
does, and this module imports nothing from the GPU library (numpy only).

Sources (the pages on FlashPrefill):
  [SKILL]  "FlashPrefill: Instantaneous Pattern Discovery for Ultra-Fast
           Long-Context Prefilling" (skillsmp skill page): sections "Core
           Concept", "Architecture Overview", "Implementation Steps" and the
           Stage 1 code "Block-Level Attention Approximation".
  [ABS]    "FlashPrefill: Instantaneous Pattern Discovery and Thresholding for
           Ultra-Fast Long-Context Prefilling" (chatpaper abstract, English).
  [V2]     "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context
           LLM Serving" (fugumt abstract): GQA / FP8 inference.

Precision.  Pooling, block scores and the threshold decision are taken in
fp32, the precision the GPU library decides them in, so both sides take the
integer keep/drop decision in the same precision.  Attention is computed in
float64.  The separate dense textbook attention is float64 as well.

Readings of the pages where they are silent or garbled (each is the plainest
reading the rest supports):
  * block count is ceil(L/B); block b covers rows [bB, min((b+1)B, L)); the
    pooled proxy is the arithmetic mean over the rows actually present.
  * block scores are (Qbar . Kbar) / sqrt(d) (an explicit sm_scale may replace
    1/sqrt(d)); only causal candidates j <= i exist.
  * threshold: keep (i, j) iff exp(S_ij - m_i) >= tau, i.e.
    S_ij - m_i >= ln(tau), with m_i the single-pass row max over j <= i; the
    diagonal block is always kept; tau = 0 keeps every causal block.
  * selection is per query head against the key/value head of its group.
  * attention is exact softmax attention restricted to the kept key blocks,
    with the token-level causal mask inside the diagonal block.

Parity status: every function here is pinned by CPU tests against closed
forms, brute force, a float64 textbook/library attention or invariants; the
comparison with the paper authors' own implementation is parity unpinned (the
pages print no code output or worked example).
"""
from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np


# ---------------------------------------------------------------------------
# Stage 1 of [SKILL] "Implementation Steps": block-level approximation.
# ---------------------------------------------------------------------------

def num_blocks(seq_len: int, block_size: int) -> int:
    """ceil(L / B): the block count of the Stage 1 code in [SKILL]."""
    return (seq_len + block_size - 1) // block_size


def pool(x: np.ndarray, block_size: int) -> np.ndarray:
    """Mean-pool token rows into one proxy per block ([SKILL] Stage 1 code,
    "Architecture Overview": average-pooled queries/keys per block).

    x: [L, H, d] fp32.  Returns [H, nb, d] fp32; block b averages rows
    [bB, min((b+1)B, L)) (a partial last block is averaged over its own rows).
    """
    x = np.asarray(x, dtype=np.float32)
    L, H, d = x.shape
    nb = num_blocks(L, block_size)
    out = np.empty((H, nb, d), dtype=np.float32)
    for b in range(nb):
        s, e = b * block_size, min((b + 1) * block_size, L)
        acc = np.zeros((H, d), dtype=np.float32)
        for t in range(s, e):  # sequential fp32 summation over the block's rows
            acc += x[t]
        out[:, b, :] = acc / np.float32(e - s)
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray, sm_scale: float) -> np.ndarray:
    """Proxy block-pair scores S[h,i,j] = (Qbar[h,i] . Kbar[g(h),j]) * sm_scale
    for j <= i; -inf above the diagonal ([SKILL] Stage 1 code: pooled Q times
    pooled K transposed over sqrt(d); causal candidates only).

    qbar: [Hq, nb, d] fp32, kbar: [Hkv, nb, d] fp32, g(h) = h // (Hq/Hkv).
    Returns [Hq, nb, nb] fp32.
    """
    Hq, nb, d = qbar.shape
    Hkv = kbar.shape[0]
    G = Hq // Hkv
    scale = np.float32(sm_scale)
    S = np.full((Hq, nb, nb), -np.inf, dtype=np.float32)
    causal = np.tril(np.ones((nb, nb), dtype=bool))
    for h in range(Hq):
        full = (qbar[h].astype(np.float32) @ kbar[h // G].astype(np.float32).T) * scale
        S[h][causal] = full[causal]
    return S


def ln_tau(tau: float) -> np.float32:
    """ln(tau) rounded to fp32 (computed in float64); -inf for tau == 0."""
    if tau == 0.0:
        return np.float32(-np.inf)
    return np.float32(math.log(float(tau)))


def select(S: np.ndarray, tau: float):
    """Single-pass max-based dynamic threshold ([SKILL] "Core Concept" item 3,
    [ABS]): per row, m = max_{j<=i} S[i,j]; keep j iff S[i,j] - m >= ln(tau),
    or j == i.  No sort, no cumulative sum.

    Returns (keep bool [Hq, nb, nb], row_max fp32 [Hq, nb]).
    """
    if not (0.0 <= tau <= 1.0) or math.isnan(tau):
        raise ValueError("tau must lie in [0, 1]")
    Hq, nb, _ = S.shape
    lt = ln_tau(tau)
    m = S.max(axis=2)  # -inf entries above the diagonal never win
    causal = np.tril(np.ones((nb, nb), dtype=bool))
    diff = (S - m[:, :, None]).astype(np.float32)
    keep = (diff >= lt) & causal[None]
    idx = np.arange(nb)
    keep[:, idx, idx] = True
    return keep, m.astype(np.float32)


def block_lists(keep: np.ndarray) -> List[List[np.ndarray]]:
    """Compact kept flags into ascending key-block lists per (head, row)
    ([SKILL] "Architecture Overview": physical index jumping over the kept
    block indices)."""
    Hq, nb, _ = keep.shape
    return [[np.flatnonzero(keep[h, i, : i + 1]).astype(np.int32) for i in range(nb)]
            for h in range(Hq)]


def ambiguous(S: np.ndarray, row_max: np.ndarray, tau: float, rel: float = 1e-5) -> np.ndarray:
    """Blocks whose score lies within `rel` (relative) of the threshold
    T = m + ln(tau): |S - T| <= rel * max(1, |T|, |m|).  Selection there is
    rounding-order sensitive, so either decision is accepted.  Empty for tau=0.
    """
    lt = ln_tau(tau)
    if not np.isfinite(lt):
        return np.zeros(S.shape, dtype=bool)
    m = row_max.astype(np.float64)[:, :, None]
    T = m + float(lt)
    tol = rel * np.maximum(1.0, np.maximum(np.abs(T), np.abs(m)))
    Sd = S.astype(np.float64)
    with np.errstate(invalid="ignore"):
        amb = np.abs(Sd - T) <= tol
    amb &= np.isfinite(Sd)
    nb = S.shape[1]
    idx = np.arange(nb)
    amb[:, idx, idx] = False  # the diagonal is forced, never ambiguous
    return amb


# ---------------------------------------------------------------------------
# Stage 3: block-sparse attention over the kept blocks (float64).
# ---------------------------------------------------------------------------

def attend_row_block(q: np.ndarray, k: np.ndarray, v: np.ndarray, h: int, i: int,
                     kept: Sequence[int], block_size: int, sm_scale: float,
                     group: int, return_probs: bool = False):
    """Exact softmax attention of query block i of head h over the listed key
    blocks, causal inside the diagonal block; kv head = h // group ([SKILL]
    "Physical Index Jumping"; GQA per [V2]).

    q: [L, Hq, d], k/v: [L, Hkv, d] (fp32 values).  Two-pass softmax in
    float64: max, exponentials, sum, divide, then P @ V.
    Returns out [rows, d] float64 (and P [rows, keys] if asked).
    """
    L = q.shape[0]
    g = h // group
    s, e = i * block_size, min((i + 1) * block_size, L)
    key_pos = np.concatenate([np.arange(j * block_size, min((j + 1) * block_size, L))
                              for j in kept]).astype(np.int64)
    Q = q[s:e, h, :].astype(np.float64)
    K = k[key_pos, g, :].astype(np.float64)
    V = v[key_pos, g, :].astype(np.float64)
    logits = (Q @ K.T) * float(sm_scale)
    qpos = np.arange(s, e)[:, None]
    logits = np.where(key_pos[None, :] > qpos, -np.inf, logits)
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    p = p / p.sum(axis=1, keepdims=True)
    out = p @ V
    if return_probs:
        return out, p, key_pos
    return out


def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, lists, block_size: int,
                     sm_scale: float, rows=None) -> np.ndarray:
    """Block-sparse causal attention for all (h, i) (or only the (h, i) pairs in
    ``rows``).  lists[h][i] = ascending kept key blocks.  Returns float64
    [L, Hq, d]; rows not computed are left NaN."""
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nb = num_blocks(L, block_size)
    out = np.full((L, Hq, d), np.nan, dtype=np.float64)
    pairs = rows if rows is not None else [(h, i) for h in range(Hq) for i in range(nb)]
    for h, i in pairs:
        s, e = i * block_size, min((i + 1) * block_size, L)
        out[s:e, h, :] = attend_row_block(q, k, v, h, i, lists[h][i], block_size, sm_scale, G)
    return out


def dense_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float) -> np.ndarray:
    """Textbook causal attention in float64 over all keys:
    softmax(Q K^T * scale + causal mask) V, with K/V heads repeated G times."""
    L, Hq, d = q.shape
    G = Hq // k.shape[1]
    out = np.empty((L, Hq, d), dtype=np.float64)
    mask = np.triu(np.ones((L, L), dtype=bool), 1)
    for h in range(Hq):
        Q = q[:, h, :].astype(np.float64)
        K = k[:, h // G, :].astype(np.float64)
        V = v[:, h // G, :].astype(np.float64)
        a = (Q @ K.T) * float(sm_scale)
        a[mask] = -np.inf
        a = np.exp(a - a.max(axis=1, keepdims=True))
        a /= a.sum(axis=1, keepdims=True)
        out[:, h, :] = a @ V
    return out


# ---------------------------------------------------------------------------
# Whole-layer pipeline.
# ---------------------------------------------------------------------------

def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, block_size: int, tau: float,
            sm_scale: float = None, attention: bool = True):
    """Pool -> score -> threshold -> lists -> sparse attention for one layer.

    q/k/v are fp32 arrays holding the exact values the GPU receives (bf16
    upcast, or fp8 codes times their per-tensor scale).
    Returns dict(qbar, kbar, S, keep, row_max, lists, out).
    """
    d = q.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    qbar = pool(q, block_size)
    kbar = pool(k, block_size)
    S = block_scores(qbar, kbar, sm_scale)
    keep, m = select(S, tau)
    lists = block_lists(keep)
    out = sparse_attention(q, k, v, lists, block_size, sm_scale) if attention else None
    return dict(qbar=qbar, kbar=kbar, S=S, keep=keep, row_max=m, lists=lists, out=out)


def select_rows(qbar_rows: np.ndarray, kbar: np.ndarray, rows, tau: float, sm_scale: float,
                group: int):
    """Selection for a sample of (h, i) rows only (for layers too large to score
    whole).  qbar_rows[n] is Qbar[h_n, i_n, :]; kbar is the full [Hkv, nb, d].
    Returns a list of (kept ascending int32, row_max fp32, S row fp32,
    ambiguous bool row) in the order of ``rows``.  Same arithmetic as
    block_scores + select restricted to one row."""
    lt = ln_tau(tau)
    scale = np.float32(sm_scale)
    res = []
    for n, (h, i) in enumerate(rows):
        kb = kbar[h // group, : i + 1].astype(np.float32)
        srow = (kb @ qbar_rows[n].astype(np.float32)) * scale
        srow = srow.astype(np.float32)
        m = srow.max()
        keep = (srow - m).astype(np.float32) >= lt
        keep[i] = True
        if np.isfinite(lt):
            T = float(m) + float(lt)
            tol = 1e-5 * max(1.0, abs(T), abs(float(m)))
            amb = np.abs(srow.astype(np.float64) - T) <= tol
            amb[i] = False
        else:
            amb = np.zeros(i + 1, dtype=bool)
        res.append((np.flatnonzero(keep).astype(np.int32), np.float32(m), srow, amb))
    return res

