"""Pins of the query-probe oracle (oracle/probe_oracle.py): the mean
reduction gives back the pooled block scores, brute force over tokens in
float64, max >= mean, and a single-token spike that only the probe rule
keeps.  CPU only."""
import math

import numpy as np

import oracle.flashprefill_oracle as O
import oracle.probe_oracle as P


def _rand(L, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(L, Hq, d)).astype(np.float32)
    k = rng.normal(size=(L, Hkv, d)).astype(np.float32)
    return q, k


def test_mean_reduction_is_the_pooled_score():
    q, k = _rand(300, 4, 2, 32, 0)  # ragged last block
    B, sc = 64, 1.0 / math.sqrt(32)
    qbar = O.pool(q, B)
    got = P.probe_scores(qbar, k, B, sc, "mean")
    want = O.block_scores(qbar, O.pool(k, B), sc)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.max(np.abs(got[fin] - want[fin])) < 1e-5


def test_max_reduction_by_brute_force():
    q, k = _rand(150, 2, 1, 16, 1)
    B, sc = 32, 0.25
    qbar = O.pool(q, B)
    got = P.probe_scores(qbar, k, B, sc, "max")
    nb = qbar.shape[1]
    for h in range(2):
        for i in range(nb):
            for j in range(nb):
                if j > i:
                    assert got[h, i, j] == -np.inf
                    continue
                best = max(float(np.dot(qbar[h, i].astype(np.float64), k[t, 0].astype(np.float64)))
                           for t in range(j * B, min((j + 1) * B, 150)))
                assert abs(got[h, i, j] - best * sc) < 1e-5 * max(1.0, abs(best * sc))


def test_max_is_at_least_the_mean():
    q, k = _rand(256, 2, 2, 16, 2)
    qbar = O.pool(q, 32)
    mx = P.probe_scores(qbar, k, 32, 0.3, "max")
    mn = P.probe_scores(qbar, k, 32, 0.3, "mean")
    fin = np.isfinite(mn)
    assert np.all(mx[fin] >= mn[fin] - 1e-6)


def test_single_token_spike_is_kept_by_the_probe_only():
    # one key token of block 2 is aligned with the probe of the last block;
    # the block mean dilutes it by 1/B, the token max does not
    L, B, d = 512, 64, 32
    rng = np.random.default_rng(3)
    q = (0.1 * rng.normal(size=(L, 1, d))).astype(np.float32)
    k = (0.1 * rng.normal(size=(L, 1, d))).astype(np.float32)
    u = np.zeros(d, np.float32)
    u[0] = 1.0
    q[-B:, 0] += 4.0 * u          # the last block's probe points along u
    k[2 * B + 17, 0] += 6.0 * u   # one token of block 2 does too (token logit 4.2)
    k[5 * B: 6 * B, 0] += 4.0 * u  # every token of block 5 a little (logit 2.8)
    sc = 1.0 / math.sqrt(d)
    probe = P.select_probe(q, k, B, 0.1, sc)
    pooled = O.prefill(q, k, k, B, 0.1, sc, attention=False)
    last = L // B - 1
    # pooled: block 5 sets the max (2.8) and block 2's diluted mean (0.07)
    # falls below max + ln 0.1; probe: block 2 sets the max, block 5 stays
    assert probe["lists"][0][last].tolist() == [2, 5, last]
    assert pooled["lists"][0][last].tolist() == [5, last]


def test_probe_select_rows_equals_whole_layer():
    """probe_select_rows (sampled rows of large layers) against select_probe
    on whole structured GQA layers with a ragged last block: same row max,
    scores, tie zone and kept set for every (h, i)."""
    from block_sparse_long_04_amd.inputs import CONFIGS, make_layer
    for Hq, Hkv, L in ((8, 2, 1000), (4, 4, 1300)):
        cfg = CONFIGS["c2"].with_(seq_len=L, num_q_heads=Hq, num_kv_heads=Hkv)
        lay = make_layer(cfg)
        q, k = lay.q32.numpy(), lay.k32.numpy()
        B, G, sc = cfg.block_size, Hq // Hkv, 1.0 / math.sqrt(cfg.head_dim)
        for tau in (0.1, 1.0):
            ref = P.select_probe(q, k, B, tau, sc)
            nb = ref["qbar"].shape[1]
            rows = [(h, i) for h in range(Hq) for i in range(nb)]
            qr = ref["qbar"][[h for h, _ in rows], [i for _, i in rows]]
            res = P.probe_select_rows(qr, k, rows, B, tau, sc, G)
            # a row's scores come from a matrix-vector product, the layer's
            # from a matrix product: equal to fp32 rounding, so the tie zone
            # lies between the whole-layer zones of half and twice the width
            lo = O.ambiguous(ref["S"], ref["row_max"], tau, rel=0.5e-5)
            hi = O.ambiguous(ref["S"], ref["row_max"], tau, rel=2e-5)
            for (h, i), (kept, m, srow, amb) in zip(rows, res):
                m0 = float(ref["row_max"][h, i])
                assert abs(float(m) - m0) <= 1e-6 * max(1.0, abs(m0))
                np.testing.assert_allclose(srow, ref["S"][h, i, : i + 1], rtol=1e-6, atol=1e-6)
                assert not (lo[h, i, : i + 1] & ~amb).any() and not (amb & ~hi[h, i, : i + 1]).any()
                got = np.zeros(i + 1, bool)
                got[kept] = True
                free = ~(amb | ref["amb"][h, i, : i + 1])
                assert np.array_equal(got[free], ref["keep"][h, i, : i + 1][free]), (h, i)
                assert got[i]
