"""CPU oracle for the query-probe variant of stage 1: pooled query probes
scored against every key token, reduced per key block.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may use it; it imports
nothing from the GPU library.

What the pages say.  [SKILL] "Core Concept" describes the pattern search with
uniformly distributed query probes and states the cost dropping from O(L^2/B)
to O((L/B)^2).  The main reading (flashprefill_oracle) takes the probe of a
query block to be its pooled proxy and scores it against pooled key proxies:
O((L/B)^2) scores.  The alternative reading taken here keeps the pooled
query probe but scores it against every key token, O(L^2/B) dot products,
and reduces the tokens of each key block to one score:

    S'[h, i, j] = max over tokens t of block j of (Qbar[h, i] . k[t, g(h)]) * sm_scale

for j <= i; then the same single-pass max threshold, diagonal and lists as
the main method.  The pages do not give the reduction.  The mean would give
back the pooled score exactly (the dot product is linear in k), so the max is
the one that differs: a single key token aligned with the probe lifts its
whole block, which the pooled mean dilutes by 1/B.  The last, partial block
of a sequence reduces over the tokens it has.  Scores are fp32 (BLAS sgemm);
the threshold is the main method's.

Pins (tests/test_oracle_probe.py): with the mean the scores equal the pooled
block scores (closed form, to fp32 rounding); brute force over tokens in
float64 on tiny inputs; max >= mean for every block pair; a single-token
spike is kept by the probe rule and dropped by the pooled rule.
"""
from __future__ import annotations

import numpy as np

from oracle import flashprefill_oracle as O


def probe_scores(qbar: np.ndarray, k: np.ndarray, block_size: int, sm_scale: float,
                 reduce: str = "max") -> np.ndarray:
    """S' [Hq, nb, nb] fp32 (-inf above the diagonal).  qbar [Hq, nb, d] fp32
    pooled query probes, k [L, Hkv, d] fp32 key tokens."""
    Hq, nb, d = qbar.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    S = np.full((Hq, nb, nb), -np.inf, dtype=np.float32)
    scale = np.float32(sm_scale)
    for h in range(Hq):
        tok = (qbar[h].astype(np.float32) @ k[:, h // G].astype(np.float32).T) * scale  # [nb, L]
        tok = tok.astype(np.float32)
        for j in range(nb):
            seg = tok[:, j * block_size: min((j + 1) * block_size, L)]
            red = seg.max(axis=1) if reduce == "max" else seg.astype(np.float64).mean(axis=1).astype(np.float32)
            S[h, j:, j] = red[j:]
    return S


def select_probe(q: np.ndarray, k: np.ndarray, block_size: int, tau: float, sm_scale: float):
    """Pool the queries, probe-score every key token, threshold (the main
    method's rule).  Returns dict(qbar, S, keep, row_max, lists, amb)."""
    qbar = O.pool(q, block_size)
    S = probe_scores(qbar, k, block_size, sm_scale, "max")
    keep, m = O.select(S, tau)
    return dict(qbar=qbar, S=S, keep=keep, row_max=m, lists=O.block_lists(keep),
                amb=O.ambiguous(S, m, tau))


def probe_select_rows(qbar_rows: np.ndarray, k: np.ndarray, rows, block_size: int, tau: float,
                      sm_scale: float, group: int):
    """The probe selection of sampled (h, i) rows only (layers too large to
    score whole).  qbar_rows[n] is Qbar[h_n, i_n, :]; k the [L, Hkv, d] key
    tokens.  Each row's scores S'[h, i, :i+1] are taken as in probe_scores;
    the row is then placed as the last row of an otherwise empty causal
    triangle, so the main method's own select and ambiguous decide it.
    Returns (kept ascending int32, row_max fp32, S' row fp32, ambiguous row)
    in the order of ``rows``."""
    L = k.shape[0]
    scale = np.float32(sm_scale)
    res = []
    for n, (h, i) in enumerate(rows):
        end = min((i + 1) * block_size, L)
        tok = (k[:end, h // group].astype(np.float32) @ qbar_rows[n].astype(np.float32)) * scale
        tok = tok.astype(np.float32)
        srow = np.array([tok[j * block_size: min((j + 1) * block_size, end)].max() for j in range(i + 1)],
                        dtype=np.float32)
        S = np.full((1, i + 1, i + 1), -np.inf, dtype=np.float32)
        S[0, i] = srow
        keep, m = O.select(S, tau)
        amb = O.ambiguous(S, m, tau)
        res.append((np.flatnonzero(keep[0, i]).astype(np.int32), m[0, i], srow, amb[0, i]))
    return res
