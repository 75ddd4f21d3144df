"""CPU oracle for the sort / cumulative-sum selection baselines (top-k, top-p)
on the same pooled block proxies as the max-threshold selection.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may use it; it imports
nothing from the GPU library.

What the pages say.  [SKILL] "Core Concept" and [ABS] present the single-pass
max threshold as the way to avoid the search overhead of the selection rules
earlier block-sparse methods use, which sort the block scores or accumulate
their probability mass.  The pages name those rules but give no formula.  The
plainest readings, taken here on the same block scores S[h, i, j] (j <= i)
that the threshold method uses:

  * top-k: keep the k causal blocks of row (h, i) with the largest scores;
    among equal scores the smaller block index comes first.
  * top-p: with pi_j = exp(S_j - m) / sum_{j' <= i} exp(S_j' - m) the row's
    block softmax, keep the shortest prefix of the blocks in descending-score
    order (ties: smaller index first) whose mass reaches p.  If rounding keeps
    every prefix below p (p = 1), every causal block is kept.

  In both the diagonal block is kept as well, as in the threshold method.
  Scores are fp32 as in the threshold method; the softmax mass and its prefix
  sums are float64.

Pins (tests/test_oracle_sorted_select.py): brute force over all subsets on
tiny rows, the special cases k >= i+1 and p = 1 (every causal block), k = 1
and p -> 0 (the argmax), nesting in k and p, a hand-built score pattern that
must come back exactly, and agreement with the threshold method where the two
rules coincide (top-p against the threshold on a row of two distinct values).
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

TOPK, TOPP = 1, 2


def _order(srow: np.ndarray) -> np.ndarray:
    """Block indices of one row in descending score order, ties by index."""
    return np.lexsort((np.arange(srow.size), -srow.astype(np.float64)))


def _prefix_len(srow: np.ndarray, mode: int, param: float) -> Tuple[int, np.ndarray, np.ndarray]:
    """Length of the kept prefix of the descending order, the order itself and
    the float64 prefix masses (mass[n] = mass of the first n blocks)."""
    order = _order(srow)
    n = srow.size
    s = srow.astype(np.float64)[order]
    w = np.exp(s - s[0])
    mass = np.concatenate([[0.0], np.cumsum(w) / w.sum()])
    if mode == TOPK:
        return min(int(param), n), order, mass
    if mode == TOPP:
        hit = np.flatnonzero(mass[1:] >= param)
        return (int(hit[0]) + 1 if hit.size else n), order, mass
    raise ValueError("mode must be TOPK or TOPP")


def select_row(srow: np.ndarray, i: int, mode: int, param: float) -> np.ndarray:
    """Kept blocks (ascending) of row i with scores srow[0..i]."""
    n, order, _ = _prefix_len(srow[: i + 1], mode, param)
    kept = set(order[:n].tolist())
    kept.add(i)
    return np.array(sorted(kept), dtype=np.int32)


def select(S: np.ndarray, mode: int, param: float):
    """Whole layer: S [Hq, nb, nb] fp32 block scores (-inf above the
    diagonal).  Returns (keep bool [Hq, nb, nb], row_max fp32 [Hq, nb])."""
    check_param(mode, param)
    Hq, nb, _ = S.shape
    keep = np.zeros(S.shape, dtype=bool)
    for h in range(Hq):
        for i in range(nb):
            keep[h, i, select_row(S[h, i], i, mode, param)] = True
    return keep, S.max(axis=2).astype(np.float32)


def check_param(mode: int, param: float) -> None:
    if mode == TOPK:
        if not (param >= 1 and float(param) == int(param)):
            raise ValueError("k must be a positive integer")
    elif mode == TOPP:
        if not (0.0 < param <= 1.0):
            raise ValueError("p must lie in (0, 1]")
    else:
        raise ValueError("mode must be TOPK or TOPP")


def accepted(gpu_kept: np.ndarray, srow: np.ndarray, i: int, mode: int, param: float,
             rel: float = 1e-5) -> bool:
    """Whether a kept set computed in another rounding order is a correct
    answer for row i: the top n blocks of a descending order in which scores
    within `rel` (relative, floor 1) of the cut may come in either order, plus
    the diagonal, for an n the rule allows (top-k: n = k; top-p: the exact n,
    or any n whose prefix mass on either side lies within `rel` of p).

    For a candidate n with cut score c = the n-th largest score:
      * blocks scoring above c + tol must be kept;
      * blocks scoring below c - tol must not be, except the diagonal;
      * the kept count is n, plus one if the diagonal is kept only because it
        is forced (below the band: exactly n + 1; inside it: n or n + 1).
    """
    row = srow[: i + 1].astype(np.float64)
    n_exact, order, mass = _prefix_len(srow[: i + 1], mode, param)
    if mode == TOPK:
        ns = [n_exact]
    else:
        ns = sorted({n_exact} | {n for n in range(1, row.size + 1)
                                 if abs(mass[n - 1] - param) <= rel or abs(mass[n] - param) <= rel})
    got = {int(j) for j in gpu_kept}
    if i not in got or any(j < 0 or j > i for j in got):
        return False
    srt = row[order]
    for n in ns:
        c = srt[n - 1]
        tol = rel * max(1.0, abs(c))
        above = {int(j) for j in np.flatnonzero(row > c + tol)}
        below = {int(j) for j in np.flatnonzero(row < c - tol)}
        if not above <= got or (below - {i}) & got:
            continue
        if row[i] > c + tol:
            ok = len(got) == n
        elif row[i] < c - tol:
            ok = len(got) == n + 1
        else:
            ok = len(got) in (n, n + 1)
        if ok:
            return True
    return False
