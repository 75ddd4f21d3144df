"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, at
sizes the oracle finishes in seconds: several tiles, ragged tails, GQA and
MHA, every input dtype, strided views, and the degenerate cases.

Bars: pooled proxies within 1e-5 relative; kept-block sets equal outside the
tie zone |S - T| <= 1e-5 max(1, |T|, |m|); outputs on the same mask within
max-abs / mean-abs 2e-2 / 2e-3 (bf16), 5e-2 / 5e-3 (fp8), 1e-4 / 1e-5 (fp32).
"""
import math

import numpy as np
import pytest
import torch

import oracle.flashprefill_oracle as O
from block_sparse_long_04_amd import _lib
from block_sparse_long_04_amd.inputs import CONFIGS, make_layer
from tests.parity_util import (check_lists_wellformed, check_out, check_pool, gpu_lists, oracle_full,
                               require_gpu, run_gpu, say, selection_mismatch, sm_scale, to_dev)

pytestmark = pytest.mark.gpu

CASES = {
    # name: (config, overrides, tau)
    "c1_tiny_f32": ("c1", {}, 0.1),
    "c1s_structured_f32": ("c1", {"recipe": "structured", "n_vertical": 4}, 0.1),
    "bf16_ragged_gqa": ("c2", {"seq_len": 1000, "num_q_heads": 8, "num_kv_heads": 2}, 0.1),
    "bf16_mha_L2048": ("c2", {"seq_len": 2048, "num_q_heads": 4, "num_kv_heads": 4}, 0.05),
    "bf16_d64_b64": ("c2", {"seq_len": 1500, "num_q_heads": 4, "num_kv_heads": 2,
                            "head_dim": 64, "block_size": 64}, 0.1),
    "bf16_d128_b64": ("c2", {"seq_len": 1100, "num_q_heads": 4, "num_kv_heads": 1,
                             "block_size": 64}, 0.2),
    "fp8_ragged": ("c4_fp8", {"seq_len": 1000, "num_q_heads": 8, "num_kv_heads": 2}, 0.1),
    # e4m3 with d = B = 64 and with B = 64 only: the vector-ALU attention
    "fp8_d64_b64": ("c4_fp8", {"seq_len": 1100, "num_q_heads": 4, "num_kv_heads": 2,
                               "head_dim": 64, "block_size": 64}, 0.1),
    "fp8_d128_b64": ("c4_fp8", {"seq_len": 900, "num_q_heads": 4, "num_kv_heads": 1,
                                "block_size": 64}, 0.1),
    # bf16 with d = 64, B = 128 (the 64-key-unit kernel, two units per block)
    "bf16_d64_b128": ("c2", {"seq_len": 1300, "num_q_heads": 6, "num_kv_heads": 2,
                             "head_dim": 64}, 0.1),
    "f32_d128_b128": ("c2", {"seq_len": 700, "num_q_heads": 2, "num_kv_heads": 1,
                             "dtype": "f32"}, 0.1),
    # three q heads per kv head and 4 kv heads: the attention's plain work order
    "bf16_gqa3": ("c2", {"seq_len": 2000, "num_q_heads": 12, "num_kv_heads": 4}, 0.1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_end_to_end_parity(name):
    dev = require_gpu()
    cname, over, tau = CASES[name]
    cfg = CONFIGS[cname].with_(**over)
    say(f"[case {name}] L={cfg.seq_len} Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads} "
        f"d={cfg.head_dim} B={cfg.block_size} {cfg.dtype} tau={tau}")
    layer = make_layer(cfg)
    ref = oracle_full(layer, tau, attention=False)
    pf, res = run_gpu(layer, tau, dev)
    check_pool(res, ref["qbar"], ref["kbar"])
    np.testing.assert_allclose(res["row_max"], ref["row_max"], rtol=1e-5, atol=1e-5)
    check_lists_wellformed(res["lists"], cfg.num_blocks)
    bad, amb = selection_mismatch(res["lists"], ref["keep"], ref["amb"])
    say(f"    selection: {bad} mismatches outside the tie zone, {amb} inside; "
        f"density {ref['keep'].sum() / (cfg.num_q_heads * cfg.num_blocks * (cfg.num_blocks + 1) / 2):.3f}")
    assert bad == 0
    # attention on the GPU's own (validated) mask
    want = O.sparse_attention(ref["q"], ref["k"], ref["v"], res["lists"], cfg.block_size,
                              sm_scale(layer))
    check_out(res["out"], want, cfg.dtype)


@pytest.mark.parametrize("name", ["bf16_ragged_gqa", "fp8_ragged", "c1_tiny_f32"])
def test_attention_on_injected_oracle_mask(name):
    # The oracle's own mask written into the workspace: attention parity that
    # does not depend on the GPU selection.
    dev = require_gpu()
    cname, over, tau = CASES[name]
    cfg = CONFIGS[cname].with_(**over)
    say(f"[inject {name}]")
    layer = make_layer(cfg)
    ref = oracle_full(layer, tau)
    _, res = run_gpu(layer, tau, dev, lists=ref["lists"])
    assert all(np.array_equal(a, b) for ra, rb in zip(res["lists"], ref["lists"])
               for a, b in zip(ra, rb))
    check_out(res["out"], ref["out"], cfg.dtype)


def test_dense_tau_zero_matches_textbook_attention():
    dev = require_gpu()
    cfg = CONFIGS["c2"].with_(seq_len=1536, num_q_heads=4, num_kv_heads=1)
    say("[dense tau=0] L=1536")
    layer = make_layer(cfg)
    _, res = run_gpu(layer, 0.0, dev)
    nb = cfg.num_blocks
    assert all(len(res["lists"][h][i]) == i + 1 for h in range(4) for i in range(nb))
    q, k, v = (t.numpy() for t in (layer.q32, layer.k32, layer.v32))
    dense = O.dense_causal_attention(q, k, v, sm_scale(layer))
    check_out(res["out"], dense, "bf16")


@pytest.mark.parametrize("d,B,L", [(64, 64, 64 * 150 + 17), (64, 128, 128 * 70 + 5), (128, 64, 64 * 130 + 33)])
def test_dense_lists_past_one_window(d, B, L):
    # tau = 0 keeps every causal block: the late query blocks' lists run past
    # 64 and 128 entries, the size of the list window the d / B = 64 kernel
    # reads with one load.
    dev = require_gpu()
    cfg = CONFIGS["c2"].with_(seq_len=L, num_q_heads=2, num_kv_heads=1, head_dim=d, block_size=B)
    say(f"[dense long lists] d={d} B={B} L={L}")
    layer = make_layer(cfg)
    _, res = run_gpu(layer, 0.0, dev)
    nb = cfg.num_blocks
    assert all(len(res["lists"][h][i]) == i + 1 for h in range(2) for i in range(nb))
    q, k, v = (t.numpy() for t in (layer.q32, layer.k32, layer.v32))
    dense = O.dense_causal_attention(q, k, v, sm_scale(layer))
    check_out(res["out"], dense, "bf16")


DEGENERATE = [(L, 128, 128) for L in (1, 77, 128, 129, 256)] + [
    # the 64-key-unit kernel: a block whose second unit lies wholly past L,
    # one-token and one-block layers
    (L, d, B) for (d, B) in ((64, 128), (64, 64), (128, 64)) for L in (1, 63, 65, 129)]


@pytest.mark.parametrize("L,d,B", DEGENERATE, ids=[f"L{L}_d{d}_B{B}" for L, d, B in DEGENERATE])
def test_degenerate_lengths(L, d, B):
    dev = require_gpu()
    cfg = CONFIGS["c2"].with_(seq_len=L, num_q_heads=4, num_kv_heads=2, head_dim=d, block_size=B)
    say(f"[length {L} d={d} B={B}]")
    layer = make_layer(cfg)
    ref = oracle_full(layer, 0.1)
    _, res = run_gpu(layer, 0.1, dev)
    bad, _ = selection_mismatch(res["lists"], ref["keep"], ref["amb"])
    assert bad == 0
    want = O.sparse_attention(ref["q"], ref["k"], ref["v"], res["lists"], B, sm_scale(layer))
    check_out(res["out"], want, "bf16")
    if L == 1:
        # one token attends to itself only
        np.testing.assert_allclose(res["out"][0], ref["v"][0][[0, 0, 1, 1]], atol=1e-2)


def test_strided_views_and_head_major_output():
    # q/k/v are column slices of one fused [L, Hq + 2Hkv, d] projection and
    # the output is a head-major [Hq, L, d] buffer seen as [L, Hq, d].
    dev = require_gpu()
    cfg = CONFIGS["c2"].with_(seq_len=640, num_q_heads=4, num_kv_heads=2)
    say("[strided views]")
    layer = make_layer(cfg)
    fused = torch.cat([layer.q, layer.k, layer.v], dim=1).to(dev)
    q, k, v = fused[:, :4], fused[:, 4:6], fused[:, 6:8]
    out = torch.empty(4, 640, 128, dtype=torch.bfloat16, device=dev).permute(1, 0, 2)
    ref = oracle_full(layer, 0.1)
    _, res = run_gpu(layer, 0.1, dev, q=q, k=k, v=v, out=out)
    bad, _ = selection_mismatch(res["lists"], ref["keep"], ref["amb"])
    assert bad == 0
    want = O.sparse_attention(ref["q"], ref["k"], ref["v"], res["lists"], 128, sm_scale(layer))
    check_out(res["out"], want, "bf16")


def test_repeat_runs_are_bitwise_identical():
    dev = require_gpu()
    cfg = CONFIGS["c2"].with_(seq_len=2048, num_q_heads=8, num_kv_heads=2)
    say("[determinism]")
    layer = make_layer(cfg)
    _, a = run_gpu(layer, 0.1, dev)
    _, b = run_gpu(layer, 0.1, dev)
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(a["counts"], b["counts"])
    assert np.array_equal(a["row_max"], b["row_max"])


def test_c2_full_layer_parity():
    # The Llama-3-8B-shaped 8K layer exactly as benchmarked (32/8 heads).
    dev = require_gpu()
    cfg = CONFIGS["c2"]
    say("[c2 full] L=8192 32/8 heads")
    layer = make_layer(cfg)
    ref = oracle_full(layer, 0.1, attention=False)
    _, res = run_gpu(layer, 0.1, dev)
    check_pool(res, ref["qbar"], ref["kbar"])
    bad, amb = selection_mismatch(res["lists"], ref["keep"], ref["amb"])
    say(f"    selection mismatches {bad} (tie zone {amb})")
    assert bad == 0
    want = O.sparse_attention(ref["q"], ref["k"], ref["v"], res["lists"], 128, sm_scale(layer))
    check_out(res["out"], want, "bf16")


def test_e4m3_decode_of_every_code_in_pool_and_vt():
    """Every e4m3fn code (NaN included) reaches the pooled proxies and the
    V^T layout with exactly the value torch's own e4m3fn decode gives.  With
    L = 129 and B = 128, token 128 is a one-token last block, whose mean is
    the token itself."""
    dev = require_gpu()
    say("[e4m3 decode] all 256 codes")
    L, H, d, B = 129, 2, 128, 128
    g = torch.Generator(device="cpu").manual_seed(7)
    codes = torch.randint(0, 256, (L, H, d), generator=g, dtype=torch.int32)
    codes[codes == 0x7f] = 0x10
    codes[codes == 0xff] = 0x90
    codes[128] = torch.arange(256, dtype=torch.int32).view(H, d)  # the lone token of block 1
    q8 = codes.to(torch.uint8).view(torch.float8_e4m3fn)
    k8 = q8.clone()
    v8 = q8.clone()
    q, k, v = q8.to(dev), k8.to(dev), v8.to(dev)
    pf = _lib.Prefill(q, k, v, block_size=B, threshold=0.1, q_scale=1.0, k_scale=1.0, v_scale=1.0)
    pf.pool()
    pf.select()
    pf.attend()  # writes its V^T scratch, then attends (NaN codes give NaN outputs; not checked)
    torch.cuda.synchronize()
    want = q8[128].float()  # torch decode, [H, d]
    for got in (pf.ws.k_pool()[:, 1, :].cpu(), pf.ws.q_pool()[:, 1, :].cpu()):
        assert torch.equal(torch.isnan(got), torch.isnan(want))
        fin = ~torch.isnan(want)
        assert torch.equal(got[fin], want[fin])
    # V^T: [Hkv][d][nb*B] bf16, token 128 of every (kv head, dim) row
    lay = pf.ws.layout
    nb = 2
    vt = pf.ws.buf[lay.v_t: lay.v_t + H * d * nb * B * 2].view(torch.bfloat16).view(H, d, nb * B)
    col = vt[:, :, 128].float().cpu()
    assert torch.equal(torch.isnan(col), torch.isnan(want))
    fin = ~torch.isnan(want)
    assert torch.equal(col[fin], want[fin])
    # zero padding past L
    assert torch.count_nonzero(vt[:, :, L:].float()).item() == 0


# Selection at shapes that reach every work split of the selection kernel
# (a workgroup owns 4, 2 or 1 tiles of 16 query-block rows, paired short
# with long), with the odd cases: an odd number of tile pairs (the middle
# pair alone), an odd number of tiles (the last pair has one tile), and a
# ragged last tile and block.  Pooling, row maxima and kept sets against the
# oracle (no attention: the oracle's selection is the part under test).
SPLIT_CASES = {
    # name: (overrides, tau); 32 q / 8 kv heads, B = 64
    "four_tiles_odd_pairs": ({"seq_len": 464 * 64 + 51}, 0.1),      # nb 465: 30 tiles, 15 pairs
    "four_tiles_odd_tiles": ({"seq_len": 488 * 64 + 37}, 0.05),     # nb 489: 31 tiles
    "two_tiles_d64": ({"seq_len": 232 * 64 + 30, "head_dim": 64}, 0.1),  # nb 233: 15 tiles
    "four_tiles_dense": ({"seq_len": 464 * 64 + 51}, 0.0),
}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_selection_work_splits(name):
    dev = require_gpu()
    over, tau = SPLIT_CASES[name]
    cfg = CONFIGS["c3"].with_(block_size=64, **over)
    nb = cfg.num_blocks
    say(f"[split {name}] L={cfg.seq_len} nb={nb} d={cfg.head_dim} tau={tau}")
    layer = make_layer(cfg)
    ref = oracle_full(layer, tau, attention=False)
    q, k, v = (t.to(dev) for t in (layer.q, layer.k, layer.v))
    pf = _lib.Prefill(q, k, v, block_size=cfg.block_size, threshold=tau)
    pf.pool()
    pf.select()
    torch.cuda.synchronize()
    res = dict(qbar=pf.ws.q_pool().cpu().numpy(), kbar=pf.ws.k_pool().cpu().numpy())
    check_pool(res, ref["qbar"], ref["kbar"])
    np.testing.assert_allclose(pf.ws.row_max().cpu().numpy(), ref["row_max"], rtol=1e-5, atol=1e-5)
    lists = gpu_lists(pf.ws.counts().cpu().numpy(), pf.ws.indices().cpu().numpy(), nb)
    check_lists_wellformed(lists, nb)
    bad, amb = selection_mismatch(lists, ref["keep"], ref["amb"])
    say(f"    selection: {bad} mismatches outside the tie zone, {amb} inside")
    assert bad == 0
    if tau == 0.0:
        for row in lists:
            for i, lst in enumerate(row):
                assert len(lst) == i + 1


def test_tau_one_keeps_the_row_argmax_and_the_diagonal():
    # ln(1) = 0: a block survives only at the row maximum (ties included)
    # or on the diagonal.  Structured layer, plus a layer whose keys repeat
    # one block's content so that several blocks tie exactly at the maximum.
    dev = require_gpu()
    cfg = CONFIGS["c2"].with_(seq_len=1500, num_q_heads=4, num_kv_heads=2)
    say("[tau=1] L=1500")
    layer = make_layer(cfg)
    ref = oracle_full(layer, 1.0)
    _, res = run_gpu(layer, 1.0, dev)
    bad, _ = selection_mismatch(res["lists"], ref["keep"], ref["amb"])
    assert bad == 0
    nb = cfg.num_blocks
    for h in range(4):
        for i in range(nb):
            assert 1 <= len(res["lists"][h][i]) <= 2 or ref["amb"][h, i].any()
    # The row's own maximum has S - m = 0 >= ln 1, so it is kept.  The
    # argmax itself lies in the tie zone (|S - T| = 0), so the comparison
    # above cannot see a dropped one; where the maximum lies clearly off the
    # diagonal (by far more than the rounding of the scores), a list holding
    # only the diagonal means the maximum was dropped.
    S = ref["S"].astype(np.float64)
    m = ref["row_max"].astype(np.float64)
    clear = 0
    for h in range(4):
        for i in range(1, nb):
            margin = 1e-3 * max(1.0, abs(m[h, i]))
            if S[h, i, :i].max() >= S[h, i, i] + margin:
                clear += 1
                assert len(res["lists"][h][i]) >= 2, (h, i)
    say(f"    {clear} rows with the maximum clearly off the diagonal keep it")
    assert clear > 0
    want = O.sparse_attention(ref["q"], ref["k"], ref["v"], res["lists"], 128, sm_scale(layer))
    check_out(res["out"], want, "bf16")

    # exact ties: every key block holds the same 128 rows, so every full
    # causal block of a row has the same proxy score.  The matrix cores do not
    # return bit-identical fp32 results for identical inputs in different
    # output columns, so which tied blocks reach the maximum is decided by
    # rounding: every tied block lies in the tie zone, and the lists must
    # still agree with the oracle outside it and end with the diagonal.
    k32 = layer.k32.clone()
    for j in range(1, nb):
        n = min(128, 1500 - j * 128)
        k32[j * 128: j * 128 + n] = layer.k32[:n]
    q32, v32 = layer.q32.numpy(), layer.v32.numpy()
    r = O.prefill(q32, k32.numpy(), v32, 128, 1.0, sm_scale(layer), attention=False)
    amb = O.ambiguous(r["S"], r["row_max"], 1.0)
    full = [j for j in range(nb) if (j + 1) * 128 <= 1500]
    for h in range(4):
        for i in full:
            assert amb[h, i, :i].all(), (h, i)  # the construction really ties
    q, _, v = to_dev(layer, dev)
    pf = _lib.Prefill(q, k32.to(torch.bfloat16).to(dev), v, block_size=128, threshold=1.0)
    pf.pool()
    pf.select()
    pf.attend()
    torch.cuda.synchronize()
    lists = gpu_lists(pf.ws.counts().cpu().numpy(), pf.ws.indices().cpu().numpy(), nb)
    check_lists_wellformed(lists, nb)
    bad, amb_diff = selection_mismatch(lists, r["keep"], amb)
    say(f"    tie layer: {amb_diff} tied blocks decided differently from the oracle (allowed)")
    assert bad == 0
    want = O.sparse_attention(q32, k32.numpy(), v32, lists, 128, sm_scale(layer))
    check_out(pf.out.float().cpu().numpy(), want, "bf16")
