"""GPU parity of the query-probe selection (fp_block_select_probe) against
oracle/probe_oracle.py: row maxima of the token-level scores within 1e-5,
kept sets equal outside the tie zone (|S' - T| <= 1e-5 max(1, |T|, |m|)),
whole small layers (bf16, e4m3, ragged), a hand-built single-token spike
that only this rule keeps, and sampled rows at 128K."""
import math

import numpy as np
import pytest
import torch

import oracle.flashprefill_oracle as O
import oracle.probe_oracle as P
from block_sparse_long_04_amd import _lib
from block_sparse_long_04_amd.inputs import CONFIGS, make_layer
from tests.parity_util import check_lists_wellformed, gpu_lists, require_gpu, say, selection_mismatch

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_ragged": ("c2", {"seq_len": 3000, "num_q_heads": 8, "num_kv_heads": 2}, 0.1),
    "bf16_L8192": ("c2", {"num_q_heads": 4, "num_kv_heads": 1}, 0.05),
    "fp8_ragged": ("c4_fp8", {"seq_len": 2500, "num_q_heads": 8, "num_kv_heads": 2}, 0.1),
}


def _gpu_probe(q, k, v, B, tau, qs=1.0, ks=1.0, vs=1.0):
    pf = _lib.Prefill(q, k, v, block_size=B, threshold=tau, q_scale=qs, k_scale=ks, v_scale=vs)
    pf.pool()
    pf.select_probe()
    torch.cuda.synchronize()
    nb = pf.ws.nb
    return pf, gpu_lists(pf.ws.counts().cpu().numpy(), pf.ws.indices().cpu().numpy(), nb)


@pytest.mark.parametrize("name", list(CASES))
def test_probe_selection_small_layers(name):
    dev = require_gpu()
    cname, over, tau = CASES[name]
    cfg = CONFIGS[cname].with_(**over)
    say(f"[probe {name}] L={cfg.seq_len} Hq={cfg.num_q_heads} tau={tau}")
    lay = make_layer(cfg)
    sc = 1.0 / math.sqrt(cfg.head_dim)
    ref = P.select_probe(lay.q32.numpy(), lay.k32.numpy(), cfg.block_size, tau, sc)
    pf, lists = _gpu_probe(lay.q.to(dev), lay.k.to(dev), lay.v.to(dev), cfg.block_size, tau,
                           lay.q_scale, lay.k_scale, lay.v_scale)
    np.testing.assert_allclose(pf.ws.row_max().cpu().numpy(), ref["row_max"], rtol=1e-5, atol=1e-5)
    check_lists_wellformed(lists, cfg.num_blocks)
    bad, amb = selection_mismatch(lists, ref["keep"], ref["amb"])
    say(f"    {bad} mismatches outside the tie zone, {amb} inside")
    assert bad == 0


def test_probe_keeps_a_single_token_spike_on_the_gpu():
    dev = require_gpu()
    L, B, d = 1024, 128, 128
    g = torch.Generator().manual_seed(5)
    q = 0.1 * torch.randn(L, 1, d, generator=g)
    k = 0.1 * torch.randn(L, 1, d, generator=g)
    q[-B:, 0, 0] += 4.0             # the last block's probe points along dim 0
    k[2 * B + 17, 0, 0] += 12.0     # one token of block 2: logit about 4.2
    k[5 * B: 6 * B, 0, 0] += 8.0    # all tokens of block 5: logit about 2.8
    qb, kb = q.to(torch.bfloat16), k.to(torch.bfloat16)
    sc = 1.0 / math.sqrt(d)
    ref = P.select_probe(qb.float().numpy(), kb.float().numpy(), B, 0.1, sc)
    pf, lists = _gpu_probe(qb.to(dev), kb.to(dev), kb.to(dev), B, 0.1)
    last = L // B - 1
    assert lists[0][last].tolist() == ref["lists"][0][last].tolist() == [2, 5, last]
    pf.select()  # the pooled rule drops the spike's block
    torch.cuda.synchronize()
    pooled = gpu_lists(pf.ws.counts().cpu().numpy(), pf.ws.indices().cpu().numpy(), pf.ws.nb)
    assert 2 not in pooled[0][last].tolist()


def test_probe_selection_c4_sampled_rows():
    dev = require_gpu()
    cfg = CONFIGS["c4"]
    B, d, nb, G = cfg.block_size, cfg.head_dim, cfg.num_blocks, cfg.num_q_heads // cfg.num_kv_heads
    say("[probe c4 sampled]")
    lay = make_layer(cfg, device=dev, keep_fp32=False)
    pf = _lib.Prefill(lay.q, lay.k, lay.v, block_size=B, threshold=0.1)
    pf.pool()
    pf.select_probe()
    torch.cuda.synchronize()
    counts = pf.ws.counts().cpu().numpy()
    idx = pf.ws.indices()
    rmax = pf.ws.row_max().cpu().numpy()
    rng = np.random.default_rng(2)
    rows = sorted({(int(h), int(i)) for h, i in zip(rng.integers(0, 32, 10), rng.integers(0, nb, 10))}
                  | {(0, nb - 1), (31, nb - 1), (5, 0)})
    sc = 1.0 / math.sqrt(d)
    bad = 0
    kh = lay.k.float().cpu().numpy()
    for h, i in rows:
        qbar = O.pool(lay.q[i * B:(i + 1) * B, h:h + 1].float().cpu().numpy(), B)[0, 0]
        kept, m, srow, amb = P.probe_select_rows(qbar[None], kh, [(h, i)], B, 0.1, sc, G)[0]
        assert abs(rmax[h, i] - m) <= 1e-5 * max(1.0, abs(float(m)))
        keep = np.zeros(i + 1, bool)
        keep[kept] = True
        off = h * (nb * (nb + 1) // 2) + i * (i + 1) // 2
        got = np.zeros(i + 1, bool)
        got[idx[off: off + int(counts[h, i])].cpu().numpy()] = True
        bad += int(((got != keep) & ~amb).sum())
    say(f"    {len(rows)} rows, {bad} mismatches outside the tie zone")
    assert bad == 0
