"""Pins of the CPU oracle against things other than itself: closed forms,
brute force on tiny inputs, a float64 textbook / library attention, and
invariants of the method.  Each test names the mistake it is meant to catch.
"""
import math

import numpy as np
import pytest
import torch

import oracle.flashprefill_oracle as O


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


# ----------------------------------------------------------------------------
# pool
# ----------------------------------------------------------------------------

def test_pool_constant_rows_exact():
    # constant c (a power of two) per head: every block mean is exactly c,
    # including the partial last block (L=37, B=8 -> last block has 5 rows).
    L, H, d, B = 37, 3, 4, 8
    x = np.zeros((L, H, d), np.float32)
    for h in range(H):
        x[:, h, :] = 2.0 ** (h - 1)
    p = O.pool(x, B)
    assert p.shape == (H, 5, d)
    for h in range(H):
        assert np.all(p[h] == np.float32(2.0 ** (h - 1)))


def test_pool_partial_block_closed_form():
    # x[t] = t: the mean of rows [s, e) is (s + e - 1) / 2.  A last block
    # divided by B instead of its own length, or a block end that ignores L,
    # fails here.
    L, B = 10, 4
    x = np.arange(L, dtype=np.float32)[:, None, None] * np.ones((1, 2, 3), np.float32)
    p = O.pool(x, B)
    expect = [(0 + 3) / 2, (4 + 7) / 2, (8 + 9) / 2]
    for b, e in enumerate(expect):
        assert np.all(p[:, b, :] == np.float32(e))


def test_pool_brute_force_float64():
    L, H, d, B = 45, 2, 5, 16
    x = rnd((L, H, d), 1)
    p = O.pool(x, B)
    for h in range(H):
        for b in range(O.num_blocks(L, B)):
            rows = [t for t in range(L) if t // B == b]
            want = [sum(float(x[t, h, c]) for t in rows) / len(rows) for c in range(d)]
            np.testing.assert_allclose(p[h, b], want, rtol=0, atol=2e-6)


# ----------------------------------------------------------------------------
# block scores
# ----------------------------------------------------------------------------

def test_scores_bilinearity_token_logit_block_mean():
    # For full blocks S[h,i,j] equals the mean of the B x B block of token
    # logits (q_t . k_s) * scale.  A transposed operand, a wrong scale
    # (1/d instead of 1/sqrt(d)) or a wrong GQA head map fails here.
    L, Hq, Hkv, d, B = 32, 4, 2, 8, 8
    q, k = rnd((L, Hq, d), 2), rnd((L, Hkv, d), 3)
    scale = 1.0 / math.sqrt(d)
    S = O.block_scores(O.pool(q, B), O.pool(k, B), scale)
    nb = L // B
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(nb):
            for j in range(nb):
                if j > i:
                    assert S[h, i, j] == -np.inf
                    continue
                tot = 0.0
                for t in range(i * B, (i + 1) * B):
                    for s in range(j * B, (j + 1) * B):
                        tot += float(np.dot(q[t, h].astype(np.float64), k[s, g].astype(np.float64)))
                want = tot / (B * B) * scale
                assert abs(S[h, i, j] - want) <= 2e-6 * max(1.0, abs(want)), (h, i, j)


def test_scores_partial_block_uses_own_length():
    # Ragged L: the last proxy averages its own rows, so the bilinearity
    # identity holds with the true row counts.
    L, d, B = 20, 4, 8
    q, k = rnd((L, 1, d), 4), rnd((L, 1, d), 5)
    S = O.block_scores(O.pool(q, B), O.pool(k, B), 0.5)
    rows = [range(0, 8), range(8, 16), range(16, 20)]
    for i in range(3):
        for j in range(i + 1):
            tot = sum(float(np.dot(q[t, 0].astype(np.float64), k[s, 0].astype(np.float64)))
                      for t in rows[i] for s in rows[j])
            want = tot / (len(rows[i]) * len(rows[j])) * 0.5
            assert abs(S[0, i, j] - want) <= 2e-6 * max(1.0, abs(want))


# ----------------------------------------------------------------------------
# threshold / selection
# ----------------------------------------------------------------------------

def test_select_hand_example():
    # Row 2: m = 2; block 1 has block probability ratio exp(ln 0.05) = 0.05 < 0.1
    # -> dropped; block 0 ties the max -> kept; block 2 is the diagonal ->
    # kept although it is exp(-5) below the max.  Row 1: the max is block 0;
    # the diagonal (ratio e^-1 >= 0.1) is kept anyway.
    S = np.full((1, 3, 3), -np.inf, np.float32)
    S[0, 0, 0] = 0.0
    S[0, 1, :2] = [1.0, 0.0]
    S[0, 2, :] = [2.0, 2.0 + math.log(0.05), 2.0 - 5.0]
    keep, m = O.select(S, 0.1)
    assert keep[0].tolist() == [[True, False, False], [True, True, False], [True, False, True]]
    assert m[0].tolist() == [0.0, 1.0, 2.0]
    # tau = 0.04 keeps block 1 of row 2 (0.05 >= 0.04)
    keep, _ = O.select(S, 0.04)
    assert keep[0, 2].tolist() == [True, True, True]


def _brute_keep(S, tau):
    Hq, nb, _ = S.shape
    keep = np.zeros_like(S, dtype=bool)
    for h in range(Hq):
        for i in range(nb):
            m = max(float(S[h, i, j]) for j in range(i + 1))
            for j in range(i + 1):
                # the block-level probability relative to the row's largest
                keep[h, i, j] = (j == i) or math.exp(float(S[h, i, j]) - m) >= tau
    return keep


@pytest.mark.parametrize("tau", [0.0, 0.05, 0.1, 0.3, 1.0])
def test_select_brute_force_exp_ratio(tau):
    L, Hq, Hkv, d, B = 96, 4, 2, 16, 8
    q, k = rnd((L, Hq, d), 6) * 3, rnd((L, Hkv, d), 7) * 3
    S = O.block_scores(O.pool(q, B), O.pool(k, B), 1.0 / math.sqrt(d))
    keep, m = O.select(S, tau)
    want = _brute_keep(S, tau)
    amb = O.ambiguous(S, m, tau)
    assert np.array_equal(keep & ~amb, want & ~amb)
    if tau == 0.0:
        assert keep.sum() == Hq * (L // B) * (L // B + 1) // 2


def test_select_tau_one_is_argmax_and_diagonal():
    L, d, B = 64, 8, 8
    q, k = rnd((L, 2, d), 8), rnd((L, 1, d), 9)
    S = O.block_scores(O.pool(q, B), O.pool(k, B), 1.0 / math.sqrt(d))
    keep, m = O.select(S, 1.0)
    for h in range(2):
        for i in range(L // B):
            row = S[h, i, : i + 1]
            want = set(np.flatnonzero(row == row.max()).tolist()) | {i}
            assert set(np.flatnonzero(keep[h, i]).tolist()) == want


def test_select_monotone_in_tau_and_invariants():
    L, Hq, d, B = 128, 2, 16, 8
    q, k = rnd((L, Hq, d), 10) * 2, rnd((L, 1, d), 11) * 2
    S = O.block_scores(O.pool(q, B), O.pool(k, B), 0.25)
    prev = None
    for tau in [0.0, 0.01, 0.1, 0.5, 1.0]:
        keep, m = O.select(S, tau)
        nb = L // B
        assert np.all(keep[:, np.arange(nb), np.arange(nb)])  # diagonal kept
        for h in range(Hq):
            for i in range(nb):
                assert keep[h, i, int(np.argmax(S[h, i, : i + 1]))]  # argmax kept
                assert not keep[h, i, i + 1:].any()  # causal
        if prev is not None:
            assert not (keep & ~prev).any()  # kept(tau2) subset of kept(tau1)
        prev = keep


def test_select_key_shift_invariance():
    # Adding one vector c to every key row adds Qbar_i . c * scale to the whole
    # row i of S, which the exp-ratio rule ignores.  A rule on raw logits
    # (S >= tau * m) fails this test.
    L, Hq, d, B = 128, 2, 16, 8
    q, k = rnd((L, Hq, d), 12) * 2, rnd((L, 1, d), 13) * 2
    c = rnd((d,), 14) * 4
    S1 = O.block_scores(O.pool(q, B), O.pool(k, B), 0.25)
    S2 = O.block_scores(O.pool(q, B), O.pool(k + c, B), 0.25)
    for tau in [0.05, 0.2]:
        k1, m1 = O.select(S1, tau)
        k2, m2 = O.select(S2, tau)
        amb = O.ambiguous(S1, m1, tau, rel=1e-4) | O.ambiguous(S2, m2, tau, rel=1e-4)
        assert np.array_equal(k1 & ~amb, k2 & ~amb)
        assert (k1 != k2).sum() <= amb.sum()


def test_select_rejects_bad_tau():
    S = np.zeros((1, 2, 2), np.float32)
    for bad in [-0.1, 1.5, float("nan")]:
        with pytest.raises(ValueError):
            O.select(S, bad)


def _pattern_inputs(nb, B, d, patterns, alpha):
    """Hand-built keys/queries: every key of block j is alpha*e_j, every query
    of block i is sum_{j in P_i} e_j, so S[i,j] = alpha*scale*[j in P_i]."""
    L = nb * B
    k = np.zeros((L, 1, d), np.float32)
    q = np.zeros((L, 1, d), np.float32)
    for j in range(nb):
        k[j * B:(j + 1) * B, 0, j] = alpha
    for i in range(nb):
        for j in patterns[i]:
            q[i * B:(i + 1) * B, 0, j] = 1.0
    return q, k


@pytest.mark.parametrize("kind", ["vertical", "slash", "block"])
def test_select_recovers_hand_built_patterns(kind):
    # The pages say vertical, slash and block patterns are found together by
    # the block proxies.  With orthogonal block keys each pattern must come
    # back exactly (plus the forced diagonal).
    nb, B, d, alpha = 12, 4, 16, 16.0
    if kind == "vertical":
        P = [[j for j in (0, 3) if j <= i] for i in range(nb)]
    elif kind == "slash":
        P = [[i - o for o in (2, 5) if i - o >= 0] for i in range(nb)]
    else:
        P = [[j for j in range(4, 8) if j <= i] if 5 <= i <= 9 else [] for i in range(nb)]
    q, k = _pattern_inputs(nb, B, d, P, alpha)
    S = O.block_scores(O.pool(q, B), O.pool(k, B), 0.25)
    keep, _ = O.select(S, 0.1)  # off-pattern gap -alpha*scale = -4 < ln 0.1 = -2.3
    for i in range(nb):
        want = set(P[i]) | {i}
        if not P[i]:
            want = set(range(i + 1))  # all-zero row: every score ties the max
        assert set(np.flatnonzero(keep[0, i]).tolist()) == want, (kind, i)


def test_block_lists_invariants():
    L, Hq, d, B = 200, 2, 8, 16
    q, k = rnd((L, Hq, d), 15) * 3, rnd((L, 1, d), 16) * 3
    S = O.block_scores(O.pool(q, B), O.pool(k, B), 1 / math.sqrt(d))
    keep, _ = O.select(S, 0.1)
    lists = O.block_lists(keep)
    for h in range(Hq):
        for i, lst in enumerate(lists[h]):
            assert len(lst) == keep[h, i].sum()
            assert np.all(np.diff(lst) > 0)
            assert lst[-1] == i and lst[0] >= 0


def test_ambiguous_zone():
    S = np.full((1, 2, 2), -np.inf, np.float32)
    lt = float(np.float32(math.log(0.1)))
    S[0, 1, 1] = 10.0
    S[0, 1, 0] = np.float32(10.0 + lt + 5e-5)  # 5e-5 above T, tol = 1e-5*10=1e-4
    S[0, 0, 0] = 0.0
    _, m = O.select(S, 0.1)
    amb = O.ambiguous(S, m, 0.1)
    assert amb[0, 1, 0] and not amb[0, 1, 1] and not amb[0, 0, 0]
    S[0, 1, 0] = np.float32(10.0 + lt + 5e-3)
    assert not O.ambiguous(S, m, 0.1)[0, 1, 0]


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def _all_lists(Hq, nb):
    return [[np.arange(i + 1, dtype=np.int32) for i in range(nb)] for _ in range(Hq)]


def test_attention_dense_equals_textbook_and_torch_sdpa():
    L, Hq, Hkv, d, B = 70, 4, 2, 16, 16  # ragged: 70 = 4*16 + 6
    q, k, v = rnd((L, Hq, d), 17), rnd((L, Hkv, d), 18), rnd((L, Hkv, d), 19)
    sc = 1 / math.sqrt(d)
    nb = O.num_blocks(L, B)
    out = O.sparse_attention(q, k, v, _all_lists(Hq, nb), B, sc)
    dense = O.dense_causal_attention(q, k, v, sc)
    np.testing.assert_allclose(out, dense, rtol=0, atol=1e-12)
    # library cross-check in float64
    tq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)
    tk = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    tv = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=sc)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_attention_brute_force_sparse_rows():
    # Python loops over individual keys with math.exp: an independent
    # statement of softmax over the kept blocks with the causal mask.
    L, Hq, Hkv, d, B = 24, 2, 1, 4, 8
    q, k, v = rnd((L, Hq, d), 20), rnd((L, Hkv, d), 21), rnd((L, Hkv, d), 22)
    lists = [[np.array([0]), np.array([1]), np.array([0, 2])],
             [np.array([0]), np.array([0, 1]), np.array([1, 2])]]
    sc = 0.7
    out = O.sparse_attention(q, k, v, lists, B, sc)
    for h in range(Hq):
        for t in range(L):
            i = t // B
            keys = [s for j in lists[h][i] for s in range(j * B, (j + 1) * B) if s <= t]
            lg = [sum(float(q[t, h, c]) * float(k[s, 0, c]) for c in range(d)) * sc for s in keys]
            mx = max(lg)
            w = [math.exp(x - mx) for x in lg]
            z = sum(w)
            for c in range(d):
                want = sum(wi * float(v[s, 0, c]) for wi, s in zip(w, keys)) / z
                assert abs(out[t, h, c] - want) < 1e-12


def test_attention_invariants():
    L, Hq, Hkv, d, B = 48, 4, 2, 8, 16
    q, k, v = rnd((L, Hq, d), 23), rnd((L, Hkv, d), 24), rnd((L, Hkv, d), 25)
    S = O.block_scores(O.pool(q, B), O.pool(k, B), 0.3)
    keep, _ = O.select(S, 0.5)
    lists = O.block_lists(keep)
    out = O.sparse_attention(q, k, v, lists, B, 0.3)
    # probabilities sum to one
    for h in range(Hq):
        for i in range(L // B):
            _, p, _ = O.attend_row_block(q, k, v, h, i, lists[h][i], B, 0.3, 2, return_probs=True)
            np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    # V + c -> out + c ; alpha V -> alpha out
    c = rnd((d,), 26)
    np.testing.assert_allclose(O.sparse_attention(q, k, v + c, lists, B, 0.3), out + c, atol=1e-6)
    np.testing.assert_allclose(O.sparse_attention(q, k, 2.5 * v, lists, B, 0.3), 2.5 * out,
                               atol=1e-6)
    # the first query attends to key 0 only
    np.testing.assert_allclose(out[0], v[0][np.arange(Hq) // 2], atol=1e-12)
    # GQA equals MHA with repeated K/V
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    np.testing.assert_allclose(O.sparse_attention(q, kr, vr, lists, B, 0.3), out, atol=1e-12)


def test_attention_ignores_unlisted_blocks():
    L, d, B = 48, 8, 16
    q, k, v = rnd((L, 1, d), 27), rnd((L, 1, d), 28), rnd((L, 1, d), 29)
    lists = [[np.array([0]), np.array([1]), np.array([0, 2])]]
    out = O.sparse_attention(q, k, v, lists, B, 0.3)
    k2, v2 = k.copy(), v.copy()
    k2[16:32] += 100.0
    v2[16:32] -= 50.0  # block 1 is only listed for row 1
    out2 = O.sparse_attention(q, k2, v2, lists, B, 0.3)
    np.testing.assert_array_equal(out[32:], out2[32:])
    np.testing.assert_array_equal(out[:16], out2[:16])
    assert not np.allclose(out[16:32], out2[16:32])


def test_prefill_dense_tau_zero_matches_textbook():
    L, Hq, Hkv, d, B = 64, 2, 1, 8, 16
    q, k, v = rnd((L, Hq, d), 30), rnd((L, Hkv, d), 31), rnd((L, Hkv, d), 32)
    r = O.prefill(q, k, v, B, 0.0)
    assert all(len(r["lists"][h][i]) == i + 1 for h in range(Hq) for i in range(4))
    np.testing.assert_allclose(r["out"], O.dense_causal_attention(q, k, v, 1 / math.sqrt(d)),
                               atol=1e-12)


@pytest.mark.parametrize("tau", [0.0, 0.1, 1.0])
def test_select_rows_equals_whole_layer_selection(tau):
    """select_rows (selection of sampled rows, used where a layer is too large
    to score whole) is pinned to the whole-layer chain pool -> block_scores ->
    select -> ambiguous: for every (h, i) of structured GQA layers with a
    ragged last block, the same row max, the same scores and the same kept set
    outside the tie zone.  Two kv groups with different structure, so a wrong
    head-to-group map changes the selection; rows whose lists reach their
    diagonal, so a wrong slice bound changes it too."""
    from block_sparse_long_04_amd.inputs import CONFIGS, make_layer
    for Hq, Hkv, L in ((8, 2, 1000), (8, 4, 1300), (6, 2, 777)):
        cfg = CONFIGS["c2"].with_(seq_len=L, num_q_heads=Hq, num_kv_heads=Hkv)
        lay = make_layer(cfg)
        q, k = lay.q32.numpy(), lay.k32.numpy()
        B, G, sc = cfg.block_size, Hq // Hkv, 1.0 / math.sqrt(cfg.head_dim)
        qbar, kbar = O.pool(q, B), O.pool(k, B)
        S = O.block_scores(qbar, kbar, sc)
        keep, m = O.select(S, tau)
        amb = O.ambiguous(S, m, tau)
        # the row's tie zone must be the whole-layer one up to the rounding of
        # its scores: between the zones of half and twice the tolerance
        amb_lo = O.ambiguous(S, m, tau, rel=0.5e-5)
        amb_hi = O.ambiguous(S, m, tau, rel=2e-5)
        nb = qbar.shape[1]
        rows = [(h, i) for h in range(Hq) for i in range(nb)]
        res = O.select_rows(qbar[[h for h, _ in rows], [i for _, i in rows]], kbar, rows, tau, sc, G)
        n_kept_off_diag = 0
        for (h, i), (kept, mr, srow, amb_r) in zip(rows, res):
            assert abs(float(mr) - float(m[h, i])) <= 1e-6 * max(1.0, abs(float(m[h, i])))
            np.testing.assert_allclose(srow, S[h, i, : i + 1], rtol=1e-6, atol=1e-6)
            assert srow.shape == (i + 1,) and amb_r.shape == (i + 1,)
            got = np.zeros(i + 1, bool)
            got[kept] = True
            free = ~(amb[h, i, : i + 1] | amb_r)
            assert np.array_equal(got[free], keep[h, i, : i + 1][free]), (h, i)
            assert got[i] and not amb_r[i]
            assert not (amb_lo[h, i, : i + 1] & ~amb_r).any(), (h, i)
            assert not (amb_r & ~amb_hi[h, i, : i + 1]).any(), (h, i)
            n_kept_off_diag += int(got[:i].sum())
        # the layers select non-trivially (not only the diagonal, not all)
        if tau == 0.1:
            total = sum(i for _, i in rows)
            assert 0 < n_kept_off_diag < total


def test_select_rows_tie_zone_hand_built():
    """Hand-placed scores around the threshold T = m + ln(0.1): pooled keys
    are unit vectors, so S[i, j] = Qbar[i, j] exactly (sm_scale 1).  With
    m = 2.5 the zone half-width is 1e-5 * |m| = 2.5e-5, wider than the floor
    1e-5, so a block 1.8e-5 above T is ambiguous only through the |m| term; a
    block at T (to fp32 rounding) is ambiguous; blocks 1e-3 either side are
    decided.  select_rows must give the whole-layer tie zone and decisions."""
    nb, d = 6, 8
    lt = float(O.ln_tau(0.1))
    m = 2.5
    T = m + lt
    row = np.array([m, T + 1.8e-5, T, T + 1e-3, T - 1e-3, 0.0], np.float32)
    qbar = np.zeros((1, nb, d), np.float32)
    qbar[0, nb - 1, :nb] = row
    kbar = np.zeros((1, nb, d), np.float32)
    kbar[0, np.arange(nb), np.arange(nb)] = 1.0
    S = O.block_scores(qbar, kbar, 1.0)
    keep, mm = O.select(S, 0.1)
    amb = O.ambiguous(S, mm, 0.1)
    i = nb - 1
    assert amb[0, i].tolist() == [False, True, True, False, False, False]
    kept, mr, srow, amb_r = O.select_rows(qbar[:, i], kbar, [(0, i)], 0.1, 1.0, 1)[0]
    assert float(mr) == float(mm[0, i]) == np.float32(m)
    assert amb_r.tolist() == amb[0, i].tolist()
    assert kept.tolist() == np.flatnonzero(keep[0, i]).tolist()
    assert set(kept.tolist()) >= {0, 3, i} and 4 not in kept.tolist()
