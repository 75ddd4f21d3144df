"""Pins of the group-shared selection oracle (oracle/group_oracle.py): one
list per kv group, the union of its heads' own selections.  CPU only."""
import math

import numpy as np

import oracle.flashprefill_oracle as O
import oracle.group_oracle as GO


def _rand(L, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(L, Hq, d)).astype(np.float32)
    k = rng.normal(size=(L, Hkv, d)).astype(np.float32)
    v = rng.normal(size=(L, Hkv, d)).astype(np.float32)
    return q, k, v


def _blocky(L, Hq, Hkv, d, B, seed, s=2.0):
    """Random rows plus one N(0, s^2) vector per (block, head) added to every
    row of the block, so that pooled scores spread over several units and the
    threshold keeps some off-diagonal blocks and drops others."""
    q, k, v = _rand(L, Hq, Hkv, d, seed)
    rng = np.random.default_rng(seed + 100)
    nb = (L + B - 1) // B
    bq = np.repeat(rng.normal(scale=s, size=(nb, Hq, d)), B, axis=0)[:L]
    bk = np.repeat(rng.normal(scale=s, size=(nb, Hkv, d)), B, axis=0)[:L]
    return (q + bq).astype(np.float32), (k + bk).astype(np.float32), v


def _nontrivial(keep):
    nb = keep.shape[-1]
    off = np.tril(np.ones((nb, nb), dtype=bool), -1)
    kept = keep[..., off]
    assert 0.05 < kept.mean() < 0.95, kept.mean()


def _keep_of(lists, nb):
    out = np.zeros((len(lists), nb, nb), dtype=bool)
    for h, rows in enumerate(lists):
        for i, lst in enumerate(rows):
            out[h, i, lst] = True
    return out


def test_one_head_per_group_is_the_per_head_selection():
    q, k, v = _rand(700, 3, 3, 32, 0)  # ragged last block, G = 1
    sc = 1.0 / math.sqrt(32)
    per = O.prefill(q, k, v, 64, 0.1, sc, attention=False)
    grp = GO.prefill_group(q, k, v, 64, 0.1, sc, attention=False)
    assert np.array_equal(grp["keep_group"], per["keep"])
    for h in range(3):
        for i in range(len(per["lists"][h])):
            assert np.array_equal(grp["lists"][h][i], per["lists"][h][i])


def test_heads_with_equal_queries_share_their_own_selection():
    # the G heads of each group carry the same queries, so each head's own
    # rule already gives the group's list
    q, k, v = _blocky(900, 8, 2, 32, 64, 1)
    q = np.repeat(q[:, ::4], 4, axis=1)  # head h copies head 4 (h // 4)
    per = O.prefill(q, k, v, 64, 0.05, 0.25, attention=False)
    _nontrivial(per["keep"])
    assert not np.array_equal(per["keep"][0], per["keep"][4])  # the groups differ
    grp = GO.select_group(per["S"], 0.05, 2)
    for h in range(8):
        assert np.array_equal(grp["keep_group"][h // 4], per["keep"][h])


def test_hand_built_head_patterns_give_their_exact_union():
    # Keys of block j are alpha * e_j (every token of the block), so the
    # pooled key is alpha * e_j; the queries of head h in block i are the sum
    # of e_j over a chosen set P_h(i) containing i.  Then S_h[i, j] = alpha *
    # scale * [j in P_h(i)], the row max is alpha * scale, and for
    # ln tau > -alpha * scale a head keeps exactly P_h(i).
    B, nb, d, alpha = 16, 12, 16, 40.0
    L, Hq, Hkv = nb * B, 4, 1
    sc = 1.0 / math.sqrt(d)
    k = np.zeros((L, Hkv, d), np.float32)
    for j in range(nb):
        k[j * B:(j + 1) * B, 0, j] = alpha
    pats = [
        lambda i: {i, 3} if i >= 3 else {i},          # a vertical column at block 3
        lambda i: {i, i - 1} if i >= 1 else {i},      # the slash next to the diagonal
        lambda i: {i, 0},                             # the sink block
        lambda i: {i},                                # the diagonal alone
    ]
    q = np.zeros((L, Hq, d), np.float32)
    for h, P in enumerate(pats):
        for i in range(nb):
            for j in P(i):
                q[i * B:(i + 1) * B, h, j] = 1.0
    tau = 0.1
    assert math.log(tau) > -alpha * sc
    r = GO.prefill_group(q, k, k, B, tau, sc, attention=False)
    for i in range(nb):
        want = sorted(set().union(*(P(i) for P in pats)))
        assert r["lists_group"][0][i].tolist() == want, i
    for h, P in enumerate(pats):
        for i in range(nb):
            assert np.flatnonzero(r["keep_head"][h, i]).tolist() == sorted(P(i))
    assert not r["amb_group"].any()


def test_union_contains_every_head_and_stays_causal():
    q, k, v = _blocky(1100, 8, 2, 32, 64, 2)
    r = GO.prefill_group(q, k, v, 64, 0.1, 0.2, attention=False)
    _nontrivial(r["keep_head"])
    nb = r["keep_group"].shape[1]
    # the union adds blocks: some head's own set is a strict subset
    assert any(r["keep_group"][h // 4].sum() > r["keep_head"][h].sum() for h in range(8))
    causal = np.tril(np.ones((nb, nb), dtype=bool))
    for h in range(8):
        assert np.all(r["keep_group"][h // 4] >= r["keep_head"][h])
    assert np.all(r["keep_group"] <= causal[None])
    assert np.all(r["keep_group"][:, np.arange(nb), np.arange(nb)])
    kg = _keep_of(r["lists"], nb)
    for h in range(8):
        assert np.array_equal(kg[h], r["keep_group"][h // 4])
        for i in range(nb):
            lst = r["lists"][h][i]
            assert np.all(np.diff(lst) > 0) and lst[-1] == i


def test_union_by_brute_force_in_float64():
    # tiny input, every score computed with Python loops in float64; blocks
    # within 1e-4 of a head's threshold are skipped (fp32 rounding decides
    # them)
    q, k, _ = _blocky(200, 4, 2, 8, 32, 3)
    B, tau, sc = 32, 0.2, 0.35
    nb = O.num_blocks(200, B)

    def mean_rows(x, j, h):
        rows = range(j * B, min((j + 1) * B, 200))
        return [sum(float(x[t, h, c]) for t in rows) / len(rows) for c in range(8)]

    S = {}
    for h in range(4):
        for i in range(nb):
            qb = mean_rows(q, i, h)
            for j in range(i + 1):
                kb = mean_rows(k, j, h // 2)
                S[h, i, j] = sum(a * b for a, b in zip(qb, kb)) * sc
    r = GO.select_group(O.block_scores(O.pool(q, B), O.pool(k, B), sc), tau, 2)
    _nontrivial(r["keep_group"])
    lt = math.log(tau)
    checked = 0
    for g in range(2):
        for i in range(nb):
            for j in range(i):
                gaps = []
                for h in (2 * g, 2 * g + 1):
                    m = max(S[h, i, jj] for jj in range(i + 1))
                    gaps.append(S[h, i, j] - m - lt)
                if any(x >= 1e-4 for x in gaps):      # some head keeps it for sure
                    assert r["keep_group"][g, i, j], (g, i, j)
                elif all(x <= -1e-4 for x in gaps):   # every head drops it for sure
                    assert not r["keep_group"][g, i, j], (g, i, j)
                else:
                    continue
                checked += 1
            assert r["keep_group"][g, i, i]
    assert checked >= 0.9 * 2 * nb * (nb - 1) / 2


def test_dense_group_attention_is_textbook_attention():
    q, k, v = _rand(333, 4, 2, 16, 4)
    sc = 0.25
    r = GO.prefill_group(q, k, v, 64, 0.0, sc)
    want = O.dense_causal_attention(q, k, v, sc)
    assert np.max(np.abs(r["out"] - want)) < 1e-10


def test_group_tie_zone():
    # a head that keeps a block outside its tie zone fixes the union there;
    # a block only some head has in its tie zone, and no head keeps surely,
    # is ambiguous
    keep = np.zeros((2, 3, 3), dtype=bool)
    amb = np.zeros((2, 3, 3), dtype=bool)
    keep[0, 2, 0], amb[1, 2, 0] = True, True     # sure keep by head 0
    amb[0, 2, 1] = True                           # tie for head 0 only
    keep[1, 2, 1] = True                          # head 1 keeps it, but inside its tie zone
    amb[1, 2, 1] = True
    ga = GO.group_ambiguous(keep, amb, 1)
    assert not ga[0, 2, 0]
    assert ga[0, 2, 1]
    assert not ga[0, 1, 0]
