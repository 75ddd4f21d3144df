"""Seeded synthetic attention layers for block-sparse causal prefill.

This module only builds inputs: it holds none of the block-sparse method's
arithmetic (no pooling, no block scores, no thresholding, no attention).  The
GPU path, the tests and the CPU oracle all take their Q/K/V from here, so both
sides of every parity check see the same bytes.

Structure of the layers (the pages measure on real long-context prompts and
models that are not available here; these synthetic layers stand in for a
Llama-3-8B-shaped attention layer: 32 query heads, 8 key/value heads,
head_dim 128, RoPE base 5e5):

* Q, K, V are i.i.d. N(0, 1), drawn in that order from one seeded
  ``torch.Generator`` on the requested device.  The CPU and GPU generators of
  torch produce different streams for the same seed; each is deterministic.
* "literal_sink" (the tiny single-head case): a seeded unit vector u; K rows
  0-3 get ``+2.0*u`` and every Q row gets ``+0.5*u``.
* "structured" (the Llama-shaped cases), per key/value head g, shared by the
  G query heads of its group:
    - slash band: a unit vector c_g supported on the rotate-half RoPE pairs
      whose frequency lies in [1/W, 4/W] (W = 256).  Before RoPE, Q += beta*c_g
      and K += beta * sum_{o in offsets} R(o) c_g, where R(o) is the RoPE
      rotation by o positions; after RoPE this lifts q_t.k_s near s = t - o.
    - RoPE (rotate-half, base theta) is applied to Q and K.
    - after RoPE, a unit vector u_g; Q += a*u_g (a = 8).
    - sinks: K rows 0-3 += (8*sqrt(d)/a) u_g, a token-logit lift of +8.
    - vertical runs: n_vertical runs of 64 keys at starts ~ U{4, L-64}; each
      run's K rows += (gap*sqrt(d)/a) u_g with gap ~ U(2, 5) logits.
  V is left i.i.d. N(0, 1).
* Casting is last: bf16 round-to-nearest-even, or fp8 e4m3fn with one
  per-tensor scale amax/448 (values clamped to +-448 before the cast).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import torch


@dataclass(frozen=True)
class LayerConfig:
    """One synthetic prefill layer."""

    name: str
    seq_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str  # "f32" | "bf16" | "fp8"
    recipe: str  # "literal_sink" | "structured"
    taus: Sequence[float] = (0.1,)
    rope_theta: float = 5e5
    n_vertical: int = 16
    slash_offsets: Sequence[int] = (0,)
    slash_width: int = 256
    beta: float = 8.0
    a: float = 8.0
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_blocks(self) -> int:
        return (self.seq_len + self.block_size - 1) // self.block_size

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


# The five workloads (sizes, head layout, block size and structure as listed
# for the Llama-3-8B-shaped layer and the tiny single-head case).
CONFIGS = {
    "c1": LayerConfig("c1_tiny_f32_L1024", 1024, 1, 1, 64, 64, "f32", "literal_sink",
                      taus=(0.1,), seed=1),
    "c2": LayerConfig("c2_llama8b_bf16_L8192", 8192, 32, 8, 128, 128, "bf16", "structured",
                      taus=(0.1,), seed=2),
    "c3": LayerConfig("c3_llama8b_bf16_L32768", 32768, 32, 8, 128, 128, "bf16", "structured",
                      taus=(0.05, 0.1, 0.2), seed=3),
    "c4": LayerConfig("c4_llama8b_bf16_L131072", 131072, 32, 8, 128, 128, "bf16", "structured",
                      taus=(0.1,), seed=4),
    "c4_fp8": LayerConfig("c4_llama8b_fp8_L131072", 131072, 32, 8, 128, 128, "fp8", "structured",
                          taus=(0.1,), seed=4),
    "c4_dense": LayerConfig("c4_llama8b_bf16_L131072_dense", 131072, 32, 8, 128, 128, "bf16",
                            "structured", taus=(0.0,), seed=4),
    "c5": LayerConfig("c5_llama8b_bf16_L262144", 262144, 32, 8, 128, 128, "bf16", "structured",
                      taus=(0.1,), n_vertical=64, slash_offsets=(0, 4096), seed=5),
}


@dataclass
class Layer:
    """Inputs of one layer: fp32 master tensors plus the cast the kernels read."""

    cfg: LayerConfig
    q32: torch.Tensor  # [L, Hq, d] fp32: exactly the values the kernels see
    k32: torch.Tensor  # [L, Hkv, d]
    v32: torch.Tensor  # [L, Hkv, d]
    q: torch.Tensor  # kernel input (f32 / bf16 / float8_e4m3fn)
    k: torch.Tensor
    v: torch.Tensor
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    meta: dict = field(default_factory=dict)


def _unit(gen: torch.Generator, n: int, device) -> torch.Tensor:
    x = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
    return x / x.norm()


def rope_tables(seq_len: int, head_dim: int, theta: float, device, positions=None):
    """cos/sin tables [L, d/2] for rotate-half RoPE (angles formed in float64)."""
    half = head_dim // 2
    inv_freq = theta ** (-torch.arange(half, dtype=torch.float64, device=device) * 2.0 / head_dim)
    if positions is None:
        positions = torch.arange(seq_len, dtype=torch.float64, device=device)
    ang = positions.to(torch.float64)[:, None] * inv_freq[None, :]
    return ang.cos().to(torch.float32), ang.sin().to(torch.float32), inv_freq


def apply_rope_(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, chunk: int = 8192):
    """In-place rotate-half RoPE on x [L, H, d] (processed in token chunks)."""
    half = x.shape[-1] // 2
    for s in range(0, x.shape[0], chunk):
        e = min(s + chunk, x.shape[0])
        c = cos[s:e, None, :]
        sn = sin[s:e, None, :]
        x1 = x[s:e, :, :half].clone()
        x2 = x[s:e, :, half:]
        x[s:e, :, :half] = x1 * c - x2 * sn
        x[s:e, :, half:] = x2 * c + x1 * sn


def _rotate_vec(c: torch.Tensor, offset: int, inv_freq: torch.Tensor) -> torch.Tensor:
    """R(offset) c for one head vector c [d] (rotate-half convention)."""
    half = c.shape[0] // 2
    ang = offset * inv_freq
    co = ang.cos().to(torch.float32)
    si = ang.sin().to(torch.float32)
    c1, c2 = c[:half], c[half:]
    return torch.cat([c1 * co - c2 * si, c2 * co + c1 * si])


def _build_fp32(cfg: LayerConfig, seed: int, device) -> tuple:
    L, Hq, Hkv, d = cfg.seq_len, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    G = Hq // Hkv
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = torch.randn(L, Hq, d, generator=gen, device=device, dtype=torch.float32)
    k = torch.randn(L, Hkv, d, generator=gen, device=device, dtype=torch.float32)
    v = torch.randn(L, Hkv, d, generator=gen, device=device, dtype=torch.float32)
    meta = {"recipe": cfg.recipe}
    if cfg.recipe == "literal_sink":
        u = _unit(gen, d, device)
        k[0:4] += 2.0 * u
        q += 0.5 * u
        return q, k, v, meta
    if cfg.recipe != "structured":
        raise ValueError(f"unknown recipe {cfg.recipe}")
    half = d // 2
    cos, sin, inv_freq = rope_tables(L, d, cfg.rope_theta, device)
    W = float(cfg.slash_width)
    pair_idx = torch.nonzero((inv_freq >= 1.0 / W) & (inv_freq <= 4.0 / W)).flatten()
    meta["slash_pairs"] = pair_idx.tolist()
    verts = []
    us = []
    for g in range(Hkv):
        c = torch.zeros(d, dtype=torch.float32, device=device)
        raw = torch.randn(2 * pair_idx.numel(), generator=gen, device=device, dtype=torch.float32)
        c[pair_idx] = raw[: pair_idx.numel()]
        c[pair_idx + half] = raw[pair_idx.numel():]
        c = c / c.norm()
        q[:, g * G:(g + 1) * G, :] += cfg.beta * c
        kc = torch.zeros(d, dtype=torch.float32, device=device)
        for o in cfg.slash_offsets:
            kc += _rotate_vec(c, int(o), inv_freq)
        k[:, g, :] += cfg.beta * kc
    apply_rope_(q, cos, sin)
    apply_rope_(k, cos, sin)
    del cos, sin
    for g in range(Hkv):
        u = _unit(gen, d, device)
        us.append(u)
        q[:, g * G:(g + 1) * G, :] += cfg.a * u
        k[0:4, g, :] += (8.0 * math.sqrt(d) / cfg.a) * u
        hi = max(L - 64, 5)
        starts = torch.randint(4, hi, (cfg.n_vertical,), generator=gen, device=device)
        gaps = 2.0 + 3.0 * torch.rand(cfg.n_vertical, generator=gen, device=device)
        for s, gp in zip(starts.tolist(), gaps.tolist()):
            k[s:s + 64, g, :] += (gp * math.sqrt(d) / cfg.a) * u
            verts.append((g, int(s), float(gp)))
    meta["verticals"] = verts
    return q, k, v, meta


def _fp8_quant(x: torch.Tensor):
    amax = float(x.abs().max())
    scale = amax / 448.0 if amax > 0 else 1.0
    xq = (x / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return xq, scale


def make_layer(cfg: LayerConfig, device="cpu", seed: Optional[int] = None,
               keep_fp32: bool = True) -> Layer:
    """Build the seeded layer for ``cfg`` on ``device`` and cast it to cfg.dtype.

    ``q32/k32/v32`` are the exact fp32 values the kernels receive (bf16 upcast,
    or fp8 dequantised as code * scale in fp32).  With keep_fp32=False they are
    left as None to save memory for the largest layers.
    """
    seed = cfg.seed if seed is None else seed
    q, k, v, meta = _build_fp32(cfg, seed, device)
    if cfg.dtype == "f32":
        lay = Layer(cfg, q, k, v, q, k, v, meta=meta)
        return lay
    if cfg.dtype == "bf16":
        qb, kb, vb = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
        del q, k, v
        if keep_fp32:
            return Layer(cfg, qb.float(), kb.float(), vb.float(), qb, kb, vb, meta=meta)
        return Layer(cfg, None, None, None, qb, kb, vb, meta=meta)
    if cfg.dtype == "fp8":
        qq, sq = _fp8_quant(q)
        del q
        kq, sk = _fp8_quant(k)
        del k
        vq, sv = _fp8_quant(v)
        del v
        if keep_fp32:
            return Layer(cfg, qq.float() * sq, kq.float() * sk, vq.float() * sv, qq, kq, vq,
                         sq, sk, sv, meta=meta)
        return Layer(cfg, None, None, None, qq, kq, vq, sq, sk, sv, meta=meta)
    raise ValueError(f"unknown dtype {cfg.dtype}")


def dequant(x: torch.Tensor, scale: float = 1.0) -> torch.Tensor:
    """fp32 values of a kernel input (exact: bf16/e4m3 upcast, then * scale)."""
    if x.dtype == torch.float8_e4m3fn:
        return x.float() * scale
    return x.float()


@dataclass
class Batch:
    """A packed batch of independent sequences (varlen), optionally with K/V
    in a paged cache.  Data layout only; no method arithmetic."""

    cfg: LayerConfig
    seq_lens: Sequence[int]
    cu_seqlens: Sequence[int]  # [S + 1] token offsets into q / out (and k / v when packed)
    q32: torch.Tensor  # [T, Hq, d] fp32, exactly the values the kernels see
    k32: torch.Tensor  # [T, Hkv, d]
    v32: torch.Tensor
    q: torch.Tensor  # kernel inputs, packed
    k: torch.Tensor
    v: torch.Tensor
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    # paged K/V: cache [num_pages, B, Hkv, d] in the kernel dtype (pages past a
    # sequence's end are zero) and block_table [S, max_blocks] of page ids
    # (-1 where a sequence has no block)
    k_cache: Optional[torch.Tensor] = None
    v_cache: Optional[torch.Tensor] = None
    block_table: Optional[torch.Tensor] = None


def make_batch(cfg: LayerConfig, seq_lens: Sequence[int], device="cpu", seed: Optional[int] = None,
               paged: bool = False, spare_pages: int = 3) -> Batch:
    """Sequences of the given lengths, each built like ``make_layer`` with its
    own seed (seed + 1000 s), concatenated token-major and cast once (one
    per-tensor fp8 scale for the batch).  With ``paged``, K and V also go to a
    cache of block_size-token pages in a seeded random order, with
    ``spare_pages`` unused pages mixed in."""
    seed = cfg.seed if seed is None else seed
    parts = []
    for s, L in enumerate(seq_lens):
        c = replace(cfg, seq_len=int(L))
        qs, ks, vs, _ = _build_fp32(c, seed + 1000 * s, device)
        parts.append((qs, ks, vs))
    q = torch.cat([p[0] for p in parts])
    k = torch.cat([p[1] for p in parts])
    v = torch.cat([p[2] for p in parts])
    del parts
    cu = [0]
    for L in seq_lens:
        cu.append(cu[-1] + int(L))
    if cfg.dtype == "f32":
        b = Batch(cfg, list(seq_lens), cu, q, k, v, q, k, v)
    elif cfg.dtype == "bf16":
        qb, kb, vb = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
        b = Batch(cfg, list(seq_lens), cu, qb.float(), kb.float(), vb.float(), qb, kb, vb)
    elif cfg.dtype == "fp8":
        (qq, sq), (kq, sk), (vq, sv) = _fp8_quant(q), _fp8_quant(k), _fp8_quant(v)
        b = Batch(cfg, list(seq_lens), cu, qq.float() * sq, kq.float() * sk, vq.float() * sv,
                  qq, kq, vq, sq, sk, sv)
    else:
        raise ValueError(f"unknown dtype {cfg.dtype}")
    if paged:
        B = cfg.block_size
        nbs = [(L + B - 1) // B for L in seq_lens]
        n_pages = sum(nbs) + spare_pages
        gen = torch.Generator(device="cpu").manual_seed(seed + 7)
        perm = torch.randperm(n_pages, generator=gen).tolist()
        Hkv, d = cfg.num_kv_heads, cfg.head_dim
        kc = torch.zeros((n_pages, B, Hkv, d), dtype=b.k.dtype, device=device)
        vc = torch.zeros((n_pages, B, Hkv, d), dtype=b.v.dtype, device=device)
        table = torch.full((len(seq_lens), max(max(nbs), 1)), -1, dtype=torch.int32)
        nxt = 0
        for s, L in enumerate(seq_lens):
            for j in range(nbs[s]):
                pg = perm[nxt]
                nxt += 1
                t0, t1 = cu[s] + j * B, min(cu[s] + (j + 1) * B, cu[s + 1])
                kc[pg, : t1 - t0] = b.k[t0:t1]
                vc[pg, : t1 - t0] = b.v[t0:t1]
                table[s, j] = pg
        b.k_cache, b.v_cache, b.block_table = kc, vc, table.to(device)
    return b
