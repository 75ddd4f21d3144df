"""Pins of the sort / cumulative-sum selection baselines of the oracle
(oracle/sorted_select_oracle.py): brute force over all subsets, the special
cases that reduce to keeping everything or only the argmax, nesting, a
hand-built pattern, and agreement with the max threshold where the rules
coincide.  CPU only."""
import itertools
import math

import numpy as np
import pytest

import oracle.flashprefill_oracle as O
import oracle.sorted_select_oracle as SO


def _mass(srow, subset):
    w = np.exp(srow.astype(np.float64) - float(srow.max()))
    return w[list(subset)].sum() / w.sum()


@pytest.mark.parametrize("seed", range(12))
def test_topk_is_the_best_subset_by_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 9))
    srow = rng.normal(size=n).astype(np.float32)  # distinct with probability 1
    i = n - 1
    for k in range(1, n + 1):
        best = max(itertools.combinations(range(n), k), key=lambda c: srow[list(c)].astype(np.float64).sum())
        want = sorted(set(best) | {i})
        assert SO.select_row(srow, i, SO.TOPK, k).tolist() == want


@pytest.mark.parametrize("seed", range(12))
def test_topp_is_the_smallest_subset_reaching_p_by_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 9))
    srow = (2.0 * rng.normal(size=n)).astype(np.float32)
    i = n - 1
    for p in (0.05, 0.3, 0.5, 0.77, 0.95, 0.999):
        # smallest size whose best subset reaches p, and that best subset
        for size in range(1, n + 1):
            best = max(itertools.combinations(range(n), size), key=lambda c: _mass(srow, c))
            if _mass(srow, best) >= p:
                break
        want = sorted(set(best) | {i})
        assert SO.select_row(srow, i, SO.TOPP, p).tolist() == want, (p, srow)


def test_special_cases_keep_everything_or_the_argmax():
    rng = np.random.default_rng(7)
    srow = rng.normal(size=40).astype(np.float32)
    i = 39
    everything = list(range(40))
    assert SO.select_row(srow, i, SO.TOPK, 40).tolist() == everything
    assert SO.select_row(srow, i, SO.TOPK, 1000).tolist() == everything
    assert SO.select_row(srow, i, SO.TOPP, 1.0).tolist() == everything
    arg = int(np.argmax(srow))
    assert SO.select_row(srow, i, SO.TOPK, 1).tolist() == sorted({arg, i})
    assert SO.select_row(srow, i, SO.TOPP, 1e-12).tolist() == sorted({arg, i})


def test_topp_boundary_is_reached_not_exceeded():
    # four equal scores: the first two hold exactly half of the mass, so
    # p = 0.5 keeps two blocks (a rule with ">" would keep three)
    srow = np.ones(4, np.float32)
    assert SO.select_row(srow, 3, SO.TOPP, 0.5).tolist() == [0, 1, 3]
    assert SO.select_row(srow, 3, SO.TOPP, 0.5000001).tolist() == [0, 1, 2, 3]


def test_ties_go_to_the_smaller_block_index():
    srow = np.array([1.0, 3.0, 2.0, 3.0, 3.0, 0.0], np.float32)
    i = 5
    assert SO.select_row(srow, i, SO.TOPK, 2).tolist() == [1, 3, 5]
    assert SO.select_row(srow, i, SO.TOPK, 1).tolist() == [1, 5]


def test_nesting_in_k_and_p():
    rng = np.random.default_rng(3)
    srow = (3.0 * rng.normal(size=64)).astype(np.float32)
    i = 63
    prev = set()
    for k in range(1, 65):
        cur = set(SO.select_row(srow, i, SO.TOPK, k).tolist())
        assert prev <= cur
        prev = cur
    prev = set()
    for p in np.linspace(0.01, 1.0, 40):
        cur = set(SO.select_row(srow, i, SO.TOPP, float(p)).tolist())
        assert prev <= cur
        prev = cur


def test_hand_built_pattern_comes_back_exactly():
    # scores alpha on a chosen set P, 0 elsewhere (plus tiny distinct offsets
    # so that the order is unique); the diagonal is outside P.
    nb, i = 48, 47
    P = [0, 5, 17, 18, 30, 41]
    srow = np.zeros(nb, np.float32) + np.arange(nb, dtype=np.float32) * -1e-4
    srow[P] += 6.0
    assert SO.select_row(srow, i, SO.TOPK, len(P)).tolist() == P + [i]
    massP = _mass(srow, P)
    assert SO.select_row(srow, i, SO.TOPP, massP * (1 - 1e-9)).tolist() == P + [i]
    assert SO.select_row(srow, i, SO.TOPP, min(1.0, massP * (1 + 1e-6))).tolist() != P + [i]


def test_agrees_with_the_max_threshold_on_two_valued_rows():
    # on a row of two values h > l the threshold with exp(l - h) < tau keeps
    # exactly the h blocks (plus the diagonal), as do top-k with k = |P| and
    # top-p with p = mass(P)
    nb = 32
    P = [2, 3, 11, 20]
    srow = np.full(nb, -1.0, np.float32)
    srow[P] = 1.5
    S = np.full((1, nb, nb), -np.inf, np.float32)
    for r in range(nb):
        S[0, r, : r + 1] = 0.0
    S[0, nb - 1] = srow
    keep, _ = O.select(S, 0.5)
    want = sorted(P + [nb - 1])
    assert np.flatnonzero(keep[0, nb - 1]).tolist() == want
    assert SO.select_row(srow, nb - 1, SO.TOPK, len(P)).tolist() == want
    assert SO.select_row(srow, nb - 1, SO.TOPP, _mass(srow, P) * (1 - 1e-9)).tolist() == want


def test_whole_layer_matches_rows_and_row_max():
    rng = np.random.default_rng(11)
    Hq, nb = 2, 20
    qbar = rng.normal(size=(Hq, nb, 16)).astype(np.float32)
    kbar = rng.normal(size=(1, nb, 16)).astype(np.float32)
    S = O.block_scores(qbar, kbar, 0.25)
    for mode, param in ((SO.TOPK, 3), (SO.TOPP, 0.6)):
        keep, m = SO.select(S, mode, param)
        for h in range(Hq):
            for i in range(nb):
                assert np.flatnonzero(keep[h, i]).tolist() == SO.select_row(S[h, i], i, mode, param).tolist()
                assert keep[h, i, i] and not keep[h, i, i + 1:].any()
        np.testing.assert_array_equal(m, S.max(axis=2))


def test_acceptance_of_other_rounding_orders():
    srow = np.array([0.0, 2.0, 1.0, 2.0 + 1e-7, -3.0, 0.5], np.float32)
    i = 5
    exact = SO.select_row(srow, i, SO.TOPK, 2)
    assert SO.accepted(exact, srow, i, SO.TOPK, 2)
    # the two near-equal leaders in either order are both kept: fine
    assert SO.accepted(np.array([1, 3, 5]), srow, i, SO.TOPK, 2)
    # a clearly lower block instead of a leader: wrong
    assert not SO.accepted(np.array([1, 2, 5]), srow, i, SO.TOPK, 2)
    # a near tie at the cut may go either way
    srow2 = np.array([3.0, 1.0, 1.0 + 2e-6, -2.0, 0.0], np.float32)
    assert SO.accepted(np.array([0, 1, 4]), srow2, 4, SO.TOPK, 2)
    assert SO.accepted(np.array([0, 2, 4]), srow2, 4, SO.TOPK, 2)
    assert not SO.accepted(np.array([0, 4]), srow2, 4, SO.TOPK, 2)
    # the diagonal must be there
    assert not SO.accepted(np.array([0, 2]), srow2, 4, SO.TOPK, 2)


def test_parameters_are_checked():
    for mode, param in ((SO.TOPK, 0), (SO.TOPK, 2.5), (SO.TOPP, 0.0), (SO.TOPP, 1.5), (7, 1)):
        with pytest.raises(ValueError):
            SO.check_param(mode, param)
    assert math.isfinite(SO.TOPP)
