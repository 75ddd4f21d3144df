"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
read its workspace, and compare with the CPU oracle."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle.flashprefill_oracle as O
from block_sparse_long_04_amd import _lib
from block_sparse_long_04_amd.inputs import Layer

# Output tolerances (max-abs, mean-abs) of GPU attention against the float64
# oracle on the same mask.  bf16 and fp8 are the stated bounds; fp32 is derived
# from fp32 accumulation over at most a few thousand keys.
TOL = {"bf16": (2e-2, 2e-3), "fp8": (5e-2, 5e-3), "f32": (1e-4, 1e-5)}
# Pooled proxies: fp32 sums over at most 128 rows in a different order.
POOL_RTOL = 1e-5


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    _lib.load_library()
    return torch.device("cuda:0")


def to_dev(layer: Layer, dev):
    return layer.q.to(dev), layer.k.to(dev), layer.v.to(dev)


def gpu_lists(counts: np.ndarray, indices: np.ndarray, nb: int):
    Hq = counts.shape[0]
    out = []
    for h in range(Hq):
        row = []
        for i in range(nb):
            off = h * (nb * (nb + 1) // 2) + i * (i + 1) // 2
            row.append(indices[off: off + counts[h, i]].copy())
        out.append(row)
    return out


def inject_lists(pf: _lib.Prefill, lists) -> None:
    """Write a given mask into the workspace (counts + triangular indices)."""
    nb = pf.ws.nb
    Hq = pf.ws.Hq
    counts = np.zeros((Hq, nb), np.int32)
    idx = np.zeros(Hq * nb * (nb + 1) // 2, np.int32)
    for h in range(Hq):
        for i in range(nb):
            lst = np.asarray(lists[h][i], np.int32)
            counts[h, i] = len(lst)
            off = h * (nb * (nb + 1) // 2) + i * (i + 1) // 2
            idx[off: off + len(lst)] = lst
    pf.ws.set_lists(counts, idx)


def run_gpu(layer: Layer, tau: float, dev, lists=None, q=None, k=None, v=None, out=None):
    """pool -> select -> (optionally replace the mask) -> attend on the GPU.
    Returns (Prefill, dict of host results)."""
    if q is None:
        q, k, v = to_dev(layer, dev)
    cfg = layer.cfg
    pf = _lib.Prefill(q, k, v, block_size=cfg.block_size, threshold=tau,
                      q_scale=layer.q_scale, k_scale=layer.k_scale, v_scale=layer.v_scale, out=out)
    pf.pool()
    pf.select()
    if lists is not None:
        inject_lists(pf, lists)
    pf.attend()
    torch.cuda.synchronize()
    nb = pf.ws.nb
    res = dict(
        qbar=pf.ws.q_pool().cpu().numpy(),
        kbar=pf.ws.k_pool().cpu().numpy(),
        row_max=pf.ws.row_max().cpu().numpy(),
        counts=pf.ws.counts().cpu().numpy(),
    )
    res["lists"] = gpu_lists(res["counts"], pf.ws.indices().cpu().numpy(), nb)
    res["out"] = pf.out.float().cpu().numpy()
    return pf, res


def check_pool(res, ref_q, ref_k):
    for got, want in ((res["qbar"], ref_q), (res["kbar"], ref_k)):
        scale = np.maximum(np.abs(want), 1.0)
        err = np.max(np.abs(got - want) / scale)
        assert err <= POOL_RTOL, f"pool rel err {err}"


def selection_mismatch(gpu_lists_, ref_keep, amb):
    """Count (h,i,j) where GPU and oracle differ outside the ambiguous set."""
    Hq, nb, _ = ref_keep.shape
    bad = 0
    amb_diff = 0
    for h in range(Hq):
        for i in range(nb):
            g = np.zeros(nb, bool)
            g[gpu_lists_[h][i]] = True
            diff = g != ref_keep[h, i]
            bad += int((diff & ~amb[h, i]).sum())
            amb_diff += int((diff & amb[h, i]).sum())
    return bad, amb_diff


def check_lists_wellformed(lists, nb):
    for row in lists:
        for i, lst in enumerate(row):
            assert len(lst) >= 1 and lst[-1] == i, (i, lst)
            assert np.all(np.diff(lst) > 0)
            assert lst[0] >= 0


def out_errors(got: np.ndarray, want: np.ndarray):
    d = np.abs(got.astype(np.float64) - want)
    return float(d.max()), float(d.mean())


def check_out(got, want, dtype_key):
    mx, mean = out_errors(got, want)
    tmax, tmean = TOL[dtype_key]
    say(f"    out max-abs {mx:.3e} (<= {tmax}), mean-abs {mean:.3e} (<= {tmean})")
    assert np.isfinite(got).all()
    assert mx <= tmax and mean <= tmean, (mx, mean)


def dtype_key(layer: Layer) -> str:
    return layer.cfg.dtype


def sm_scale(layer: Layer) -> float:
    return 1.0 / math.sqrt(layer.cfg.head_dim)


def oracle_full(layer: Layer, tau: float, attention: bool = True):
    q, k, v = layer.q32.cpu().numpy(), layer.k32.cpu().numpy(), layer.v32.cpu().numpy()
    r = O.prefill(q, k, v, layer.cfg.block_size, tau, sm_scale(layer), attention=attention)
    r["amb"] = O.ambiguous(r["S"], r["row_max"], tau)
    r["q"], r["k"], r["v"] = q, k, v
    return r
