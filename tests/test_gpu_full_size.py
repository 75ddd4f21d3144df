"""GPU parity at the benchmarked sizes (32 q / 8 kv heads, d = 128, B = 128,
L = 32K, 128K, 256K), launched exactly as the benchmark launches them.  The
oracle cannot score or attend whole layers this large in seconds, so it is
run on samples: all pooled key proxies, and for a set of (head, query-block)
rows (the heaviest rows, the last row of every head, the first row, random
rows) the pooled query proxy, the selection and the attention output.  Whole
layer properties (list shape, counts) are checked everywhere.
"""
import math

import numpy as np
import pytest
import torch

import oracle.flashprefill_oracle as O
from block_sparse_long_04_amd import _lib
from block_sparse_long_04_amd.inputs import CONFIGS, make_layer
from tests.parity_util import POOL_RTOL, TOL, require_gpu, say

pytestmark = pytest.mark.gpu

CASES = [
    ("c3", 0.05), ("c3", 0.1), ("c3", 0.2),
    ("c4", 0.1), ("c4_fp8", 0.1), ("c4_dense", 0.0),
    ("c5", 0.1),
]


def _host(t, scale, g=None):
    x = t if g is None else t[:, g:g + 1]
    x = x.float()
    if t.dtype == torch.float8_e4m3fn:
        x = x * scale
    return x.cpu().numpy()


@pytest.mark.parametrize("name,tau", CASES, ids=[f"{n}_tau{t}" for n, t in CASES])
def test_full_size_sampled_parity(name, tau):
    dev = require_gpu()
    cfg = CONFIGS[name]
    L, B, Hq, Hkv, d = cfg.seq_len, cfg.block_size, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    G, nb = Hq // Hkv, cfg.num_blocks
    say(f"[full {name} tau={tau}] L={L} {cfg.dtype}")
    lay = make_layer(cfg, device=dev, keep_fp32=False)
    pf = _lib.Prefill(lay.q, lay.k, lay.v, block_size=B, threshold=tau,
                      q_scale=lay.q_scale, k_scale=lay.k_scale, v_scale=lay.v_scale)
    pf.run()
    torch.cuda.synchronize()
    counts = pf.ws.counts().cpu().numpy()
    idx = pf.ws.indices()
    row_max = pf.ws.row_max().cpu().numpy()
    kbar_gpu = pf.ws.k_pool().cpu().numpy()
    qbar_gpu = pf.ws.q_pool()

    def lst(h, i):
        off = h * (nb * (nb + 1) // 2) + i * (i + 1) // 2
        return idx[off: off + int(counts[h, i])].cpu().numpy()

    # whole-layer list shape: 1 <= count <= i+1
    ii = np.arange(nb)[None, :]
    assert (counts >= 1).all() and (counts <= ii + 1).all()

    # pooled keys, all heads and blocks
    kh = _host(lay.k, lay.k_scale)
    kbar = O.pool(kh, B)
    err = np.max(np.abs(kbar_gpu - kbar) / np.maximum(np.abs(kbar), 1.0))
    assert err <= POOL_RTOL, err
    vh = _host(lay.v, lay.v_scale)

    rng = np.random.default_rng(0)
    rows = set()
    heavy = np.argsort(-counts.ravel(), kind="stable")[:8]
    rows.update((int(r // nb), int(r % nb)) for r in heavy)
    rows.update((h, nb - 1) for h in range(Hq))
    rows.update((int(h), 0) for h in rng.integers(0, Hq, 2))
    rows.update((int(h), int(i)) for h, i in zip(rng.integers(0, Hq, 12), rng.integers(0, nb, 12)))
    if name == "c4_dense":  # dense rows attend to every earlier key: keep the sample small
        rows = {r for r in rows if r[1] < 160} | {(0, nb - 1), (Hq - 1, nb // 2)}
    rows = sorted(rows)
    sc = 1.0 / math.sqrt(d)
    qfull = np.zeros((L, 1, d), np.float32)
    worst, sum_abs, n_abs, sel_bad, amb_total = 0.0, 0.0, 0, 0, 0
    for (h, i) in rows:
        s, e = i * B, min((i + 1) * B, L)
        qrows = _host(lay.q[s:e, h:h + 1], lay.q_scale)
        qbar = O.pool(qrows, B)[0, 0]
        qg = qbar_gpu[h, i].cpu().numpy()
        assert np.max(np.abs(qg - qbar) / np.maximum(np.abs(qbar), 1.0)) <= POOL_RTOL
        kept, m, srow, amb = O.select_rows(qbar[None], kbar, [(h, i)], tau, sc, G)[0]
        assert abs(row_max[h, i] - m) <= 1e-5 * max(1.0, abs(float(m)))
        gl = lst(h, i)
        assert len(gl) >= 1 and gl[-1] == i and np.all(np.diff(gl) > 0)
        got = np.zeros(i + 1, bool)
        got[gl] = True
        want = np.zeros(i + 1, bool)
        want[kept] = True
        sel_bad += int(((got != want) & ~amb).sum())
        amb_total += int(((got != want) & amb).sum())
        qfull[s:e] = qrows
        g = h // G
        ref = O.attend_row_block(qfull, kh[:, g:g + 1], vh[:, g:g + 1], 0, i, gl, B, sc, 1)
        out = pf.out[s:e, h, :].float().cpu().numpy()
        dd = np.abs(out - ref)
        worst = max(worst, float(dd.max()))
        sum_abs += float(dd.sum())
        n_abs += dd.size
    tmax, tmean = TOL[cfg.dtype]
    say(f"    {len(rows)} rows: selection mismatches {sel_bad} (tie zone {amb_total}); "
        f"out max-abs {worst:.3e} mean-abs {sum_abs / n_abs:.3e}; density "
        f"{counts.sum() / (Hq * nb * (nb + 1) / 2):.4f}")
    assert sel_bad == 0
    assert worst <= tmax and sum_abs / n_abs <= tmean


def test_maximum_block_count_2m_tokens():
    """The largest layer the library takes: 16384 blocks of 128 tokens (2M
    tokens), 32 q / 8 kv heads, bf16.  One kv head of K then spans 4 GiB of
    token-major memory, so the attention must address K per key block.
    Whole-layer list shape everywhere; sampled rows of two kv groups against
    the oracle (selection and attention)."""
    dev = require_gpu()
    nbmax = 16384
    cfg = CONFIGS["c4"].with_(seq_len=nbmax * 128)
    tau = 0.1
    L, B, Hq, Hkv, d = cfg.seq_len, cfg.block_size, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    G, nb = Hq // Hkv, cfg.num_blocks
    assert nb == nbmax
    say(f"[max size] L={L} nb={nb} {cfg.dtype}; K spans {L * Hkv * d * 2 / 2**30:.0f} GiB")
    lay = make_layer(cfg, device=dev, keep_fp32=False)
    pf = _lib.Prefill(lay.q, lay.k, lay.v, block_size=B, threshold=tau)
    pf.run()
    torch.cuda.synchronize()
    say("    layer done")
    counts = pf.ws.counts()
    idx = pf.ws.indices()
    ii = torch.arange(nb, device=dev, dtype=torch.int64)
    assert bool(((counts >= 1) & (counts <= ii[None, :] + 1)).all())
    # every list ends with its diagonal block
    hh = torch.arange(Hq, device=dev, dtype=torch.int64)[:, None]
    last = hh * (nb * (nb + 1) // 2) + ii * (ii + 1) // 2 + counts.long() - 1
    assert bool((idx[last] == ii[None, :].int()).all())
    density = float(counts.sum()) / (Hq * nb * (nb + 1) / 2)
    cnt = counts.cpu().numpy()
    row_max = pf.ws.row_max().cpu().numpy()
    sc = 1.0 / math.sqrt(d)
    worst = sum_abs = 0.0
    n_abs = sel_bad = 0
    rng = np.random.default_rng(7)
    qfull = np.zeros((L, 1, d), np.float32)
    for g in (0, Hkv - 1):
        kh = lay.k[:, g:g + 1].float().cpu().numpy()
        vh = lay.v[:, g:g + 1].float().cpu().numpy()
        kbar = O.pool(kh, B)  # [1, nb, d]
        rows = [(g * G, nb - 1), (g * G + G - 1, 0), (g * G + 1, nb // 2)]
        rows += [(g * G + int(u), int(i)) for u, i in zip(rng.integers(0, G, 3), rng.integers(0, nb, 3))]
        for (h, i) in rows:
            s0, s1 = i * B, (i + 1) * B
            qrows = lay.q[s0:s1, h:h + 1].float().cpu().numpy()
            qbar = O.pool(qrows, B)[0, 0]
            kept, m, srow, amb = O.select_rows(qbar[None], kbar, [(0, i)], tau, sc, 1)[0]
            assert abs(row_max[h, i] - m) <= 1e-5 * max(1.0, abs(float(m)))
            off = h * (nb * (nb + 1) // 2) + i * (i + 1) // 2
            gl = idx[off: off + int(cnt[h, i])].cpu().numpy()
            got = np.zeros(i + 1, bool)
            got[gl] = True
            want = np.zeros(i + 1, bool)
            want[kept] = True
            sel_bad += int(((got != want) & ~amb).sum())
            qfull[s0:s1] = qrows
            ref = O.attend_row_block(qfull, kh, vh, 0, i, gl, B, sc, 1)
            qfull[s0:s1] = 0.0
            out = pf.out[s0:s1, h, :].float().cpu().numpy()
            dd = np.abs(out - ref)
            worst = max(worst, float(dd.max()))
            sum_abs += float(dd.sum())
            n_abs += dd.size
        del kh, vh
    say(f"    density {density:.4f}; sampled rows: selection mismatches {sel_bad}; "
        f"out max-abs {worst:.3e} mean-abs {sum_abs / n_abs:.3e}")
    assert sel_bad == 0
    tmax, tmean = TOL["bf16"]
    assert worst <= tmax and sum_abs / n_abs <= tmean
