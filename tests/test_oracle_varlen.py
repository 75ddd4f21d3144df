"""Pins of the varlen / paged-KV oracle (oracle/varlen_oracle.py): at tau = 0
a batch equals one textbook attention over the packed tokens with a
same-sequence causal mask (and torch's CPU attention with that mask); the
page gather inverts the scatter; sequences are independent.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle.flashprefill_oracle as O
import oracle.varlen_oracle as V
from block_sparse_long_04_amd.inputs import CONFIGS, make_batch

LENS = [300, 129, 77, 640]


def _cfg(**kw):
    return CONFIGS["c2"].with_(num_q_heads=4, num_kv_heads=2, **kw)


def test_dense_batch_equals_masked_attention_over_packed_tokens():
    cfg = _cfg(block_size=64, head_dim=64)
    b = make_batch(cfg, LENS)
    sc = 1.0 / math.sqrt(cfg.head_dim)
    q, k, v = b.q32.numpy(), b.k32.numpy(), b.v32.numpy()
    got = V.prefill_varlen(q, k, v, b.cu_seqlens, cfg.block_size, 0.0, sc)["out"]
    want = V.dense_varlen_attention(q, k, v, b.cu_seqlens, sc)
    assert np.max(np.abs(got - want)) < 1e-9
    # library cross-check of the masked formulation
    T = q.shape[0]
    seg = np.repeat(np.arange(len(LENS)), LENS)
    pos = np.arange(T)
    mask = torch.from_numpy((seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None]))
    G = cfg.num_q_heads // cfg.num_kv_heads
    Q = torch.from_numpy(q).double().permute(1, 0, 2)
    K = torch.from_numpy(k).double().repeat_interleave(G, dim=1).permute(1, 0, 2)
    Vv = torch.from_numpy(v).double().repeat_interleave(G, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, Vv, attn_mask=mask, scale=sc)
    assert np.max(np.abs(ref.permute(1, 0, 2).numpy() - want)) < 1e-9


def test_page_gather_inverts_the_scatter():
    cfg = _cfg()
    b = make_batch(cfg, LENS, paged=True)
    kc, vc, table = b.k_cache.float().numpy(), b.v_cache.float().numpy(), b.block_table.numpy()
    for s in range(len(LENS)):
        ks, vs = V.sequence_kv(None, None, b.cu_seqlens, s, cfg.block_size, kc, vc, table)
        c0, c1 = b.cu_seqlens[s], b.cu_seqlens[s + 1]
        np.testing.assert_array_equal(ks, b.k.float().numpy()[c0:c1])
        np.testing.assert_array_equal(vs, b.v.float().numpy()[c0:c1])
    # every used page is distinct and some pages are unused
    used = table[table >= 0]
    assert len(set(used.tolist())) == used.size and used.size < kc.shape[0]


def test_sequences_do_not_see_each_other():
    cfg = _cfg()
    b = make_batch(cfg, LENS)
    q, k, v = b.q32.numpy().copy(), b.k32.numpy().copy(), b.v32.numpy().copy()
    r0 = V.prefill_varlen(q, k, v, b.cu_seqlens, cfg.block_size, 0.1)
    c0, c1 = b.cu_seqlens[1], b.cu_seqlens[2]
    rng = np.random.default_rng(0)
    q[c0:c1] += rng.normal(size=q[c0:c1].shape).astype(np.float32)
    k[c0:c1] *= 3.0
    v[c0:c1] -= 1.0
    r1 = V.prefill_varlen(q, k, v, b.cu_seqlens, cfg.block_size, 0.1)
    for s in (0, 2, 3):
        a, c = b.cu_seqlens[s], b.cu_seqlens[s + 1]
        np.testing.assert_array_equal(r0["out"][a:c], r1["out"][a:c])
        assert all(np.array_equal(x, y) for x, y in zip(sum(r0["seqs"][s]["lists"], []),
                                                        sum(r1["seqs"][s]["lists"], [])))
    assert not np.array_equal(r0["out"][c0:c1], r1["out"][c0:c1])


def test_paged_and_packed_agree_and_one_sequence_is_the_single_layer():
    cfg = _cfg()
    b = make_batch(cfg, LENS, paged=True)
    q, k, v = b.q32.numpy(), b.k32.numpy(), b.v32.numpy()
    packed = V.prefill_varlen(q, k, v, b.cu_seqlens, cfg.block_size, 0.1)
    paged = V.prefill_varlen(q, None, None, b.cu_seqlens, cfg.block_size, 0.1,
                             k_cache=b.k_cache.float().numpy(), v_cache=b.v_cache.float().numpy(),
                             table=b.block_table.numpy())
    np.testing.assert_array_equal(packed["out"], paged["out"])
    L = LENS[3]
    c0 = b.cu_seqlens[3]
    single = O.prefill(q[c0:c0 + L], k[c0:c0 + L], v[c0:c0 + L], cfg.block_size, 0.1,
                       1.0 / math.sqrt(cfg.head_dim))
    np.testing.assert_array_equal(single["out"], packed["out"][c0:c0 + L])
