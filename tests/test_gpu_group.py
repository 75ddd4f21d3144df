"""GPU parity of group-shared selection (fp_block_select_group): one list per
kv group, the union of its heads' own threshold selections, written as the
list of every head of the group; the attention that follows is unchanged.

Small layers: the GPU's lists against the oracle's group lists
(oracle/group_oracle.py) outside the group tie zone, every head of a group
holding the same list, row maxima equal to each head's own, the group list
containing the per-head list fp_block_select gives on the same workspace,
and outputs on the GPU's lists within the bf16 / fp8 / fp32 tolerances.
At 128K (32 q / 8 kv heads, as benchmarked): sampled (group, query block)
rows against the oracle's union of its heads' own rows, attention on sampled
rows, and for every row that the group list is the union of the per-head
lists.
"""
import math

import numpy as np
import pytest
import torch

import oracle.flashprefill_oracle as O
import oracle.group_oracle as GO
from block_sparse_long_04_amd import _lib
from block_sparse_long_04_amd.inputs import CONFIGS, make_layer
from tests.parity_util import TOL, check_lists_wellformed, check_out, gpu_lists, require_gpu, say, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    # name: (config, overrides, tau)
    "bf16_ragged_8x2": ("c2", {"seq_len": 1000, "num_q_heads": 8, "num_kv_heads": 2}, 0.1),
    "bf16_32x8_L4096": ("c3", {"seq_len": 4096}, 0.05),
    "fp8_ragged_8x2": ("c4_fp8", {"seq_len": 1500, "num_q_heads": 8, "num_kv_heads": 2}, 0.1),
    "f32_d64_b64_4x1": ("c1", {"recipe": "structured", "n_vertical": 4, "num_q_heads": 4}, 0.1),
    "bf16_mha": ("c2", {"seq_len": 777, "num_q_heads": 4, "num_kv_heads": 4}, 0.1),
    "bf16_gqa3": ("c2", {"seq_len": 2000, "num_q_heads": 12, "num_kv_heads": 4}, 0.1),
}


def _tri(h, i, nb):
    return h * (nb * (nb + 1) // 2) + i * (i + 1) // 2


@pytest.mark.parametrize("name", list(CASES))
def test_group_selection_against_the_oracle(name):
    dev = require_gpu()
    cname, over, tau = CASES[name]
    cfg = CONFIGS[cname].with_(**over)
    Hq, Hkv, nb, B = cfg.num_q_heads, cfg.num_kv_heads, cfg.num_blocks, cfg.block_size
    G = Hq // Hkv
    say(f"[group {name}] L={cfg.seq_len} Hq={Hq} Hkv={Hkv} d={cfg.head_dim} B={B} {cfg.dtype} tau={tau}")
    layer = make_layer(cfg)
    q, k, v = to_dev(layer, dev)
    pf = _lib.Prefill(q, k, v, block_size=B, threshold=tau, q_scale=layer.q_scale,
                      k_scale=layer.k_scale, v_scale=layer.v_scale)
    pf.pool()
    pf.select()
    torch.cuda.synchronize()
    per = gpu_lists(pf.ws.counts().cpu().numpy(), pf.ws.indices().cpu().numpy(), nb)
    pf.select_group()
    pf.attend()
    torch.cuda.synchronize()
    lists = gpu_lists(pf.ws.counts().cpu().numpy(), pf.ws.indices().cpu().numpy(), nb)
    row_max = pf.ws.row_max().cpu().numpy()
    sc = 1.0 / math.sqrt(cfg.head_dim)
    q32, k32, v32 = layer.q32.cpu().numpy(), layer.k32.cpu().numpy(), layer.v32.cpu().numpy()
    ref = GO.prefill_group(q32, k32, v32, B, tau, sc, attention=False)

    check_lists_wellformed(lists, nb)
    np.testing.assert_allclose(row_max, ref["row_max"], rtol=1e-5, atol=1e-5)
    bad = amb_diff = grew = 0
    for h in range(Hq):
        g = h // G
        for i in range(nb):
            assert np.array_equal(lists[h][i], lists[g * G][i]), (h, i)  # one list per group
            assert set(per[h][i].tolist()) <= set(lists[h][i].tolist()), (h, i)
            grew += len(lists[h][i]) - len(per[h][i])
            got = np.zeros(nb, bool)
            got[lists[h][i]] = True
            diff = got != ref["keep_group"][g, i]
            bad += int((diff & ~ref["amb_group"][g, i]).sum())
            amb_diff += int((diff & ref["amb_group"][g, i]).sum())
    tot = sum(len(x) for row in lists for x in row)
    say(f"    group selection: {bad} mismatches outside the tie zone, {amb_diff} inside; "
        f"{grew} blocks added to per-head lists ({tot} kept)")
    assert bad == 0
    if G > 1 and name != "f32_d64_b64_4x1":
        assert grew > 0  # the union really adds blocks on these layers
    want = O.sparse_attention(q32, k32, v32, lists, B, sc)
    check_out(pf.out.float().cpu().numpy(), want, cfg.dtype)


def test_group_selection_full_size_128k():
    dev = require_gpu()
    cfg = CONFIGS["c4"]
    tau = 0.1
    L, B, Hq, Hkv, d = cfg.seq_len, cfg.block_size, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    G, nb = Hq // Hkv, cfg.num_blocks
    tri = nb * (nb + 1) // 2
    say(f"[group full c4 tau={tau}] L={L} {cfg.dtype}")
    lay = make_layer(cfg, device=dev, keep_fp32=False)
    pf = _lib.Prefill(lay.q, lay.k, lay.v, block_size=B, threshold=tau)
    pf.pool()
    pf.select()
    torch.cuda.synchronize()
    per_cnt = pf.ws.counts().clone()
    per_idx = pf.ws.indices().clone()
    pf.select_group()
    pf.attend()
    torch.cuda.synchronize()
    cnt = pf.ws.counts()
    idx = pf.ws.indices()

    # every row: the group list is the union of the per-head lists (bitmaps
    # built from the lists with torch on the device)
    ii = torch.arange(nb, device=dev)
    roff = ii * (ii + 1) // 2
    slot = torch.arange(tri, device=dev)
    row_i = torch.searchsorted(roff, slot, right=True) - 1
    e = slot - roff[row_i]

    def bitmap(c, ix):
        keep = torch.zeros(Hq, nb, nb, dtype=torch.bool, device=dev)
        for h in range(Hq):
            seg = ix[h * tri:(h + 1) * tri]
            valid = e < c[h][row_i]
            keep[h, row_i[valid], seg[valid].long()] = True
        return keep

    kp = bitmap(per_cnt, per_idx)
    kg = bitmap(cnt, idx)
    union = kp.view(Hkv, G, nb, nb).any(1)
    for h in range(Hq):
        assert torch.equal(kg[h], union[h // G]), h
    assert torch.equal(cnt, kg.sum(-1).to(cnt.dtype))  # no duplicates in a list
    dens_h = float(per_cnt.sum()) / (Hq * tri)
    dens_g = float(cnt.sum()) / (Hq * tri)

    # sampled rows against the oracle: every head of the group selects on
    # its own (pooled on the host), then the union
    kh = lay.k.float().cpu().numpy()
    vh = lay.v.float().cpu().numpy()
    kbar = O.pool(kh, B)
    sc = 1.0 / math.sqrt(d)
    rng = np.random.default_rng(1)
    rows = {(0, nb - 1), (Hkv - 1, nb - 1), (3, 0)} | {
        (int(g), int(i)) for g, i in zip(rng.integers(0, Hkv, 10), rng.integers(0, nb, 10))}
    bad = 0
    worst = sum_abs = 0.0
    n_abs = 0
    for (g, i) in sorted(rows):
        s0, s1 = i * B, min((i + 1) * B, L)
        qrows = lay.q[s0:s1, g * G:(g + 1) * G].float().cpu().numpy()
        qbar = O.pool(qrows, B)[:, 0]  # [G, d]: the pooled probes of the group's heads
        res = O.select_rows(qbar, kbar, [(g * G + u, i) for u in range(G)], tau, sc, G)
        sure = np.zeros(i + 1, bool)
        some_amb = np.zeros(i + 1, bool)
        for kept, m, srow, amb in res:
            k1 = np.zeros(i + 1, bool)
            k1[kept] = True
            sure |= k1 & ~amb
            some_amb |= amb
        gl = idx[_tri(g * G, i, nb):_tri(g * G, i, nb) + int(cnt[g * G, i])].cpu().numpy()
        got = np.zeros(i + 1, bool)
        got[gl] = True
        undecided = some_amb & ~sure
        bad += int(((got != sure) & ~undecided).sum())
        # attention of the group's first head on the group list
        qfull = np.zeros((L, 1, d), np.float32)
        qfull[s0:s1] = qrows[:, :1]
        want = O.attend_row_block(qfull, kh[:, g:g + 1], vh[:, g:g + 1], 0, i, gl, B, sc, 1)
        out = pf.out[s0:s1, g * G, :].float().cpu().numpy()
        dd = np.abs(out - want)
        worst = max(worst, float(dd.max()))
        sum_abs += float(dd.sum())
        n_abs += dd.size
    say(f"    density per head {dens_h:.4f} -> group {dens_g:.4f}; {len(rows)} sampled rows: "
        f"{bad} mismatches; out max-abs {worst:.3e} mean-abs {sum_abs / n_abs:.3e}")
    assert bad == 0
    tmax, tmean = TOL["bf16"]
    assert worst <= tmax and sum_abs / n_abs <= tmean
