"""GPU parity of the sort / cumulative-sum selection baselines (top-k,
top-p; fp_block_select_sorted) against the oracle (oracle/sorted_select_oracle).

Bar: every row's kept set is a correct answer of the rule for the oracle's
scores (SO.accepted: only rounding-level near-ties at the cut, and cut
positions whose prefix mass lies within 1e-5 of p, may go either way); the row
maxima equal the oracle's within 1e-5 and are bit-identical to the threshold
kernel's (same score arithmetic); attention on these lists matches the oracle
on the same lists.  Whole layers up to 32K tokens, sampled rows at 128K and
256K (2048 blocks, the largest the baseline takes).
"""
import math

import numpy as np
import pytest
import torch

import oracle.flashprefill_oracle as O
import oracle.sorted_select_oracle as SO
from block_sparse_long_04_amd import _lib
from block_sparse_long_04_amd.inputs import CONFIGS, make_layer
from tests.parity_util import (POOL_RTOL, check_lists_wellformed, check_out, gpu_lists, oracle_full,
                               require_gpu, say, sm_scale)

pytestmark = pytest.mark.gpu

RULES = {"topk": _lib.FP_SELECT_TOPK, "topp": _lib.FP_SELECT_TOPP}

SMALL = {
    # name: (config, overrides)
    "bf16_ragged_gqa": ("c2", {"seq_len": 1000, "num_q_heads": 8, "num_kv_heads": 2}),
    "bf16_L4096": ("c2", {"seq_len": 4096, "num_q_heads": 8, "num_kv_heads": 2}),
    "d64_b64": ("c2", {"seq_len": 1500, "num_q_heads": 4, "num_kv_heads": 2, "head_dim": 64,
                       "block_size": 64}),
    "fp8": ("c4_fp8", {"seq_len": 2048, "num_q_heads": 8, "num_kv_heads": 2}),
}
PARAMS = [("topk", 1), ("topk", 8), ("topk", 1000), ("topp", 0.5), ("topp", 0.9), ("topp", 1.0)]


def _check_rows(lists, S_rows, rule, param):
    bad = 0
    for (h, i), srow in S_rows:
        if not SO.accepted(lists[h][i], srow, i, RULES[rule], param):
            bad += 1
            if bad <= 3:
                say(f"    row ({h},{i}) gpu {lists[h][i].tolist()[:12]} oracle "
                    f"{SO.select_row(srow, i, RULES[rule], param).tolist()[:12]}")
    return bad


@pytest.mark.parametrize("name", list(SMALL))
def test_sorted_selection_small_layers(name):
    dev = require_gpu()
    cname, over = SMALL[name]
    cfg = CONFIGS[cname].with_(**over)
    say(f"[sorted {name}] L={cfg.seq_len} Hq={cfg.num_q_heads} d={cfg.head_dim} B={cfg.block_size}")
    layer = make_layer(cfg)
    ref = oracle_full(layer, 0.1, attention=False)
    q, k, v = (t.to(dev) for t in (layer.q, layer.k, layer.v))
    pf = _lib.Prefill(q, k, v, block_size=cfg.block_size, threshold=0.1, q_scale=layer.q_scale,
                      k_scale=layer.k_scale, v_scale=layer.v_scale)
    pf.pool()
    pf.select()
    torch.cuda.synchronize()
    rm_thresh = pf.ws.row_max().clone()
    nb = cfg.num_blocks
    S = ref["S"]
    rows = [((h, i), S[h, i]) for h in range(cfg.num_q_heads) for i in range(nb)]
    for rule, param in PARAMS:
        pf.select_sorted(RULES[rule], param)
        torch.cuda.synchronize()
        assert torch.equal(pf.ws.row_max(), rm_thresh)
        np.testing.assert_allclose(pf.ws.row_max().cpu().numpy(), ref["row_max"], rtol=1e-5, atol=1e-5)
        lists = gpu_lists(pf.ws.counts().cpu().numpy(), pf.ws.indices().cpu().numpy(), nb)
        check_lists_wellformed(lists, nb)
        bad = _check_rows(lists, rows, rule, param)
        say(f"    {rule} {param}: {bad} rows outside the rule")
        assert bad == 0
        if rule == "topk" and param == 8 and name != "fp8":
            pf.attend()
            torch.cuda.synchronize()
            want = O.sparse_attention(ref["q"], ref["k"], ref["v"], lists, cfg.block_size, sm_scale(layer))
            check_out(pf.out.float().cpu().numpy(), want, cfg.dtype)


@pytest.mark.parametrize("rule,param", [("topk", 35), ("topp", 0.9)])
def test_sorted_selection_c3_whole_layer(rule, param):
    dev = require_gpu()
    cfg = CONFIGS["c3"]
    say(f"[sorted c3 whole layer] {rule} {param}")
    lay = make_layer(cfg, device=dev, keep_fp32=False)
    pf = _lib.Prefill(lay.q, lay.k, lay.v, block_size=cfg.block_size, threshold=0.1)
    pf.pool()
    pf.select_sorted(RULES[rule], param)
    torch.cuda.synchronize()
    nb = cfg.num_blocks
    qbar = O.pool(lay.q.float().cpu().numpy(), cfg.block_size)
    kbar = O.pool(lay.k.float().cpu().numpy(), cfg.block_size)
    S = O.block_scores(qbar, kbar, 1.0 / math.sqrt(cfg.head_dim))
    lists = gpu_lists(pf.ws.counts().cpu().numpy(), pf.ws.indices().cpu().numpy(), nb)
    check_lists_wellformed(lists, nb)
    bad = _check_rows(lists, [((h, i), S[h, i]) for h in range(cfg.num_q_heads) for i in range(nb)],
                      rule, param)
    say(f"    {bad} rows outside the rule; density "
        f"{pf.ws.counts().sum().item() / (cfg.num_q_heads * nb * (nb + 1) / 2):.4f}")
    assert bad == 0


@pytest.mark.parametrize("name,rule,param", [("c4", "topk", 35), ("c4", "topp", 0.9),
                                             ("c5", "topk", 64), ("c5", "topp", 0.95)])
def test_sorted_selection_full_size_sampled(name, rule, param):
    dev = require_gpu()
    cfg = CONFIGS[name]
    B, d, nb, G = cfg.block_size, cfg.head_dim, cfg.num_blocks, cfg.num_q_heads // cfg.num_kv_heads
    say(f"[sorted {name} sampled] {rule} {param}")
    lay = make_layer(cfg, device=dev, keep_fp32=False)
    pf = _lib.Prefill(lay.q, lay.k, lay.v, block_size=B, threshold=0.1)
    pf.pool()
    pf.select_sorted(RULES[rule], param)
    torch.cuda.synchronize()
    counts = pf.ws.counts().cpu().numpy()
    idx = pf.ws.indices()
    kbar = O.pool(lay.k.float().cpu().numpy(), B)
    kbar_gpu = pf.ws.k_pool().cpu().numpy()
    assert np.max(np.abs(kbar_gpu - kbar) / np.maximum(np.abs(kbar), 1.0)) <= POOL_RTOL
    rng = np.random.default_rng(1)
    rows = {(h, nb - 1) for h in range(0, cfg.num_q_heads, 3)}
    rows |= {(int(h), int(i)) for h, i in zip(rng.integers(0, cfg.num_q_heads, 24), rng.integers(0, nb, 24))}
    rows |= {(0, 0), (1, 63), (2, 64)}
    sc = np.float32(1.0 / math.sqrt(d))
    bad = 0
    for h, i in sorted(rows):
        qbar = O.pool(lay.q[i * B:(i + 1) * B, h:h + 1].float().cpu().numpy(), B)[0, 0]
        srow = ((kbar[h // G, : i + 1].astype(np.float32) @ qbar.astype(np.float32)) * sc).astype(np.float32)
        off = h * (nb * (nb + 1) // 2) + i * (i + 1) // 2
        lst = idx[off: off + int(counts[h, i])].cpu().numpy()
        assert len(lst) >= 1 and lst[-1] == i and np.all(np.diff(lst) > 0)
        bad += 0 if SO.accepted(lst, srow, i, RULES[rule], param) else 1
    say(f"    {len(rows)} rows, {bad} outside the rule")
    assert bad == 0
