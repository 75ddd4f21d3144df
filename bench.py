#!/usr/bin/env python3
"""Block-sparse causal prefill benchmark on one MI355X.

One step = one layer's whole hot path through the C ABI:
fp_block_pool (pool Q/K) -> fp_block_select (scores, max threshold, lists)
-> fp_sparse_prefill (V^T layout pass, then attention over the kept
blocks), on
seeded synthetic inputs already resident in HBM.  The default workload is the
Llama-3-8B-shaped layer at L = 131072 (32 q / 8 kv heads, d = 128, B = 128,
bf16, tau = 0.1).

Prints ONE JSON line: value = kept-block TFLOP/s over the whole step
(algorithmic FLOPs of the kept (query, key) pairs / ms per layer), plus
per-stage times, the attention kernel's roofline, the CPU oracle timed on a
bounded sample of the same layer on this host, (up to 2048 blocks) the
sorting / cumulative-sum selection baselines timed next to the threshold, and
(for the default workload) a serving-like batch of sequences with K/V in a
paged cache, run as one batch and one sequence at a time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse prefill ms/layer + kept-block TFLOP/s (frac of MFMA peak) at 128K"
# MI355X published peaks
PEAK = {"bf16": 2500.0, "fp8": 5000.0, "fp32": 157.3, "hbm_gbs": 8000.0}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c4",
                    help="workload key: c1 c2 c3 c4 c4_fp8 c4_dense c5")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--head-dim", type=int, default=None,
                    help="override the workload's head dimension (64 or 128)")
    ap.add_argument("--block-size", type=int, default=None,
                    help="override the workload's block size (64 or 128)")
    ap.add_argument("--evict-mib", type=int, default=512,
                    help="before each timed step, outside its events, read a buffer of this many "
                         "MiB so the Infinity Cache (256 MiB) holds none of the previous step's data "
                         "(0: off)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the batch (varlen, paged K/V) measurement of the default workload")
    ap.add_argument("--select", choices=("threshold", "group"), default="threshold",
                    help="selection of the timed step: each head's own threshold lists, or one "
                         "union list per kv group (fp_block_select_group)")
    ap.add_argument("--no-group", action="store_true",
                    help="skip the group-shared selection measurement")
    ap.add_argument("--attention", choices=("default", "pack"), default="default",
                    help="attention of the timed step: fp_sparse_prefill, or fp_sparse_prefill_pack "
                         "(two query heads per workgroup; bf16 with an even group size)")
    ap.add_argument("--no-pack", action="store_true",
                    help="skip the two-heads-per-workgroup attention measurement")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 5 plain device copies of MIB MiB "
                         "(the known-size kernel that scales the HBM byte counters)")
    return ap.parse_args()


def copy_calibration(mib: int):
    """Plain device-to-device copies of a known size: rocprofv3's FETCH_SIZE and
    WRITE_SIZE on these give the counter-to-byte factor."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(5):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / 5
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": round(ms, 4),
                      "gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def kept_pairs(counts, L, B):
    """Causal (query, key) pairs of the kept blocks: off-diagonal blocks are
    full (j < i), the diagonal contributes n_i(n_i+1)/2."""
    import numpy as np
    nb = counts.shape[1]
    n = np.full(nb, B, dtype=np.float64)
    n[-1] = L - (nb - 1) * B
    c = counts.astype(np.float64)
    return float((n[None, :] * B * (c - 1.0) + n[None, :] * (n[None, :] + 1) / 2.0).sum())


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


ATTN_SOURCES = {
    "default": ["block_sparse_long_04_amd/csrc/attn_mfma.hip",
                "block_sparse_long_04_amd/csrc/attn_common.h",
                "block_sparse_long_04_amd/csrc/common.h"],
    "pack": ["block_sparse_long_04_amd/csrc/attn_pack.hip",
             "block_sparse_long_04_amd/csrc/attn_common.h",
             "block_sparse_long_04_amd/csrc/common.h"],
    "small": ["block_sparse_long_04_amd/csrc/attn_small.hip",
              "block_sparse_long_04_amd/csrc/attn_common.h",
              "block_sparse_long_04_amd/csrc/common.h"],
    "generic": ["block_sparse_long_04_amd/csrc/attn_generic.hip",
                "block_sparse_long_04_amd/csrc/common.h"],
}


def attention_kernel(dtype: str, d: int, B: int, attention: str = "default") -> str:
    """Which attention kernel a layer runs: the d = B = 128 matrix-core kernel
    (bf16 / e4m3; its two-heads variant when asked), the 64-key-unit
    matrix-core kernel for bf16 with d or B = 64, else the generic one."""
    if dtype in ("bf16", "fp8") and d == 128 and B == 128:
        return "pack" if attention == "pack" else "default"
    if dtype == "bf16" and d in (64, 128) and B in (64, 128):
        return "small"
    return "generic"


def measured_traffic(workload: str, kernel: str = "default"):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, only if it was taken on the current attention source."""
    path = os.path.join(ROOT, "profiles", "attn_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except Exception:
        return None
    if not rec or rec.get("source_hash") != source_hash(ATTN_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(layer_dev, lists_gpu, counts, cfg, tau, budget_s):
    """The CPU oracle (as it stands) on a bounded sample of the same layer:
    pool all blocks of the sampled kv heads' keys, then select + attend sampled
    (head, query-block) rows, heaviest first, until the time budget is spent.
    Also compares those rows with the GPU (selection outside the tie zone,
    output error on the GPU's mask)."""
    import numpy as np
    import torch

    import oracle.flashprefill_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    L, B, d = cfg.seq_len, cfg.block_size, cfg.head_dim
    G = cfg.group
    nb = cfg.num_blocks
    sc = 1.0 / math.sqrt(d)
    heads = [0, cfg.num_q_heads // 2 + 1] if cfg.num_q_heads > 1 else [0]
    kvh = sorted({h // G for h in heads})
    lay = layer_dev

    def host(t, g, scale):
        x = t[:, g:g + 1, :].float()
        if t.dtype == torch.float8_e4m3fn:
            x = x * scale
        return x.cpu().numpy()

    kh = {g: host(lay.k, g, lay.k_scale) for g in kvh}
    vh = {g: host(lay.v, g, lay.v_scale) for g in kvh}
    rng = np.random.default_rng(0)
    per_head = []
    for h in heads:
        order = list(np.argsort(-counts[h], kind="stable")[:4]) + list(rng.permutation(nb))
        seen, lst = set(), []
        for i in order:
            if int(i) not in seen:
                seen.add(int(i))
                lst.append((h, int(i)))
        per_head.append(lst)
    rows = [r for tup in zip(*per_head) for r in tup]  # heads interleaved
    qfull = np.zeros((L, 1, d), np.float32)  # rows s:e are filled per sampled block
    t0 = time.perf_counter()
    kbar = {g: O.pool(kh[g], B)[0] for g in kvh}
    t_pool_k = time.perf_counter() - t0
    done, flops, tsel, tatt, tq = [], 0.0, 0.0, 0.0, 0.0
    sel_bad, max_abs, sum_abs, n_abs = 0, 0.0, 0.0, 0
    kbar_all = None
    start = time.perf_counter()
    for (h, i) in rows:
        if time.perf_counter() - start > budget_s and len(done) >= 4:
            break
        g = h // G
        s, e = i * B, min((i + 1) * B, L)
        ta = time.perf_counter()
        qrows = lay.q[s:e, h:h + 1, :].float()
        if lay.q.dtype == torch.float8_e4m3fn:
            qrows = qrows * lay.q_scale
        qrows = qrows.cpu().numpy()
        tq += time.perf_counter() - ta
        ta = time.perf_counter()
        qbar = O.pool(qrows, B)[0, 0]
        if kbar_all is None:
            kbar_all = np.zeros((cfg.num_kv_heads, nb, d), np.float32)
            for gg in kvh:
                kbar_all[gg] = kbar[gg]
        kept, m, srow, amb = O.select_rows(qbar[None], kbar_all, [(h, i)], tau, sc, G)[0]
        tb = time.perf_counter()
        tsel += tb - ta
        # attention of the sampled row (oracle mask), float64
        qfull[s:e] = qrows
        out = O.attend_row_block(qfull, kh[g], vh[g], 0, i, kept, B, sc, 1)
        tatt += time.perf_counter() - tb
        n_i = e - s
        flops += 4.0 * d * (n_i * B * (len(kept) - 1) + n_i * (n_i + 1) / 2.0)
        done.append((h, i))
        # parity of this row against the GPU
        gl = np.zeros(i + 1, bool)
        gl[lists_gpu(h, i)] = True
        ol = np.zeros(i + 1, bool)
        ol[kept] = True
        sel_bad += int(((gl != ol) & ~amb).sum())
        gout = lay.out[s:e, h, :].float().cpu().numpy()
        want = O.attend_row_block(qfull, kh[g], vh[g], 0, i, lists_gpu(h, i), B, sc, 1)
        err = np.abs(gout - want)
        max_abs = max(max_abs, float(err.max()))
        sum_abs += float(err.sum())
        n_abs += err.size
    total = t_pool_k + tsel + tatt
    return {
        "value": flops / total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{len(done)} (head, query-block) rows of heads {heads} (4 heaviest + random), "
                   f"keys of kv heads {kvh} pooled in full; float64 attention, fp32 selection; "
                   f"{total:.1f} s of CPU work"),
        "seconds": {"pool_k": round(t_pool_k, 3), "select": round(tsel, 3),
                    "attention": round(tatt, 3)},
        "parity_rows": {"rows": len(done), "selection_mismatch_outside_tie_zone": sel_bad,
                        "out_max_abs": max_abs, "out_mean_abs": sum_abs / max(n_abs, 1)},
    }


def select_baselines(pf, _lib, torch, thr_ms, k, p, reps=5):
    """Median device time of fp_block_select_sorted (top-k, top-p) against
    the threshold selection of the same run."""
    out = {"threshold_ms": round(thr_ms, 4)}
    for name, rule, param in (("topk", _lib.FP_SELECT_TOPK, k), ("topp", _lib.FP_SELECT_TOPP, p)):
        pf.select_sorted(rule, param)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            pf.select_sorted(rule, param)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[reps // 2]
        out[name] = {"param": param, "ms": round(ms, 4), "vs_threshold": round(ms / thr_ms, 2),
                     "kept_blocks": int(pf.ws.counts().sum().item())}
    if pf.ws.nb <= 1024 and pf.prob.dtype != _lib.FP_F32 and pf.prob.head_dim == 128 and pf.prob.block_size == 128:
        # the query-probe reading of stage 1 (token-level max per key block)
        pf.select_probe()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            pf.select_probe()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[reps // 2]
        out["probe_max"] = {"ms": round(ms, 4), "vs_threshold": round(ms / thr_ms, 2),
                            "kept_blocks": int(pf.ws.counts().sum().item())}
    return out


def pack_attention(pf, torch, flops, attn_ms, reps=5):
    """fp_sparse_prefill_pack on the step's own lists (median of `reps`
    runs), against the step's fp_sparse_prefill time; the outputs of the two
    are bit-identical (checked here too)."""
    pf.attend()
    ref = pf.out.clone()
    pf.attend_pack()
    torch.cuda.synchronize()
    same = bool(torch.equal(ref, pf.out))
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pf.attend_pack()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = sorted(ts)[reps // 2]
    return {"attention_ms": round(ms, 4), "attention_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "vs_default_attention": round(ms / attn_ms, 3), "bit_identical_to_default": same}


def group_select(pf, torch, kept_pairs, cfg, per_head, reps=5):
    """Group-shared selection (fp_block_select_group: each head's own
    threshold, then one union list per kv group) and the attention on its
    lists, median of `reps` runs each, against the per-head figures of the
    same run (per_head: stage_ms of the timed steps)."""
    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[reps // 2]

    sel_ms = timed(pf.select_group)
    att_ms = timed(pf.attend)
    counts = pf.ws.counts().cpu().numpy()
    nb = cfg.num_blocks
    flops = 4.0 * cfg.head_dim * kept_pairs(counts, cfg.seq_len, cfg.block_size)
    layer_ms = per_head["pool"] + sel_ms + att_ms
    return {"select_ms": round(sel_ms, 4), "attention_ms": round(att_ms, 4),
            "ms_per_layer": round(layer_ms, 4),
            "density": round(float(counts.sum()) / (cfg.num_q_heads * nb * (nb + 1) / 2), 5),
            "kept_tflop": round(flops / 1e12, 4),
            "attention_tflops": round(flops / (att_ms * 1e-3) / 1e12, 2),
            "vs_per_head_ms_per_layer": round(layer_ms / sum(per_head.values()), 3)}


# a serving-like mix of prompts: 4 of about 8K, 8 of 4K, 16 of 2K, 32 of 1K
# tokens (ragged lengths), 128K tokens in all
VARLEN_LENS = tuple([8192 - 37 * k for k in range(4)] + [4096 - 29 * k for k in range(8)] +
                    [2048 - 13 * k for k in range(16)] + [1024 - 7 * k for k in range(32)])


def varlen_batch(cfg, _lib, make_batch, kept_pairs, torch, np, reps=5):
    """A serving-like batch (VARLEN_LENS, K/V in a paged cache) through the
    fp_*_varlen calls, against the same sequences run one at a time through the
    single-sequence calls.  Median of `reps` whole runs each."""
    dev = torch.device("cuda:0")
    b = make_batch(cfg, VARLEN_LENS, device=dev, paged=True)
    tau = cfg.taus[0]
    pv = _lib.PrefillVarlen(b.q, b.k_cache, b.v_cache, b.cu_seqlens, block_size=cfg.block_size,
                            threshold=tau, block_table=b.block_table)
    singles = []
    for s in range(len(VARLEN_LENS)):
        c0, c1 = b.cu_seqlens[s], b.cu_seqlens[s + 1]
        singles.append(_lib.Prefill(b.q[c0:c1].contiguous(), b.k[c0:c1].contiguous(),
                                    b.v[c0:c1].contiguous(), block_size=cfg.block_size, threshold=tau))

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[reps // 2]

    ms_batch = timed(pv.run)
    ms_single = timed(lambda: [x.run() for x in singles])
    counts = pv.counts().cpu().numpy()
    pairs, first = 0, 0
    for L in VARLEN_LENS:
        nb = (L + cfg.block_size - 1) // cfg.block_size
        pairs += kept_pairs(counts[:, first:first + nb], L, cfg.block_size)
        first += nb
    flops = 4.0 * cfg.head_dim * pairs
    return {"seq_lens": list(VARLEN_LENS), "tokens": int(b.cu_seqlens[-1]), "paged_kv": True,
            "ms_batch": round(ms_batch, 4), "ms_one_by_one": round(ms_single, 4),
            "kept_tflops_batch": round(flops / (ms_batch * 1e-3) / 1e12, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures the single-GPU path; this build has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from block_sparse_long_04_amd import _lib
    from block_sparse_long_04_amd.inputs import CONFIGS, make_layer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    _lib.load_library()
    dev = torch.device("cuda:0")
    cfg = CONFIGS[args.config]
    over = {}
    if args.head_dim is not None:
        over["head_dim"] = args.head_dim
    if args.block_size is not None:
        over["block_size"] = args.block_size
    if over:
        cfg = cfg.with_(name=cfg.name + "".join(f"_{k[0]}{v}" for k, v in sorted(over.items())), **over)
    tau = cfg.taus[0] if args.tau is None else args.tau
    print(f"[bench] building {cfg.name} on the GPU", file=sys.stderr, flush=True)
    layer = make_layer(cfg, device=dev, keep_fp32=False)
    pf = _lib.Prefill(layer.q, layer.k, layer.v, block_size=cfg.block_size, threshold=tau,
                      q_scale=layer.q_scale, k_scale=layer.k_scale, v_scale=layer.v_scale)
    layer.out = pf.out

    select = pf.select_group if args.select == "group" else pf.select
    attend = pf.attend_pack if args.attention == "pack" else pf.attend

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pf.pool()
        if ev is not None:
            ev[1].record()
        select()
        if ev is not None:
            ev[2].record()
        attend()
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    # Eviction reads a buffer: written lines would leave dirty data in the
    # cache whose write-back then competes with the step's first reads.
    evict = torch.ones(args.evict_mib << 20, dtype=torch.uint8, device=dev) if args.evict_mib > 0 else None
    if evict is not None:
        evict.max()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for k in range(args.steps):
        if evict is not None:
            evict.max()  # same stream, before the step's first event
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    st = {"pool": [], "select": [], "attention": []}
    for ev in evs:
        st["pool"].append(ev[0].elapsed_time(ev[1]))
        st["select"].append(ev[1].elapsed_time(ev[2]))
        st["attention"].append(ev[2].elapsed_time(ev[3]))
    stage_ms = {k: float(np.mean(v)) for k, v in st.items()}
    per_step = [ev[0].elapsed_time(ev[3]) for ev in evs]
    ms_step = float(np.mean(per_step))
    counts = pf.ws.counts().cpu().numpy()
    L, B, d, Hq, Hkv = cfg.seq_len, cfg.block_size, cfg.head_dim, cfg.num_q_heads, cfg.num_kv_heads
    nb = cfg.num_blocks
    pairs = kept_pairs(counts, L, B)
    flops = 4.0 * d * pairs
    density = float(counts.sum()) / (Hq * nb * (nb + 1) / 2)
    esz = {"bf16": 2, "fp8": 1, "f32": 4}[cfg.dtype]
    kernel = attention_kernel(cfg.dtype, d, B, args.attention)
    mfma_path = kernel != "generic"  # matrix cores (and the V^T layout pass in the stage)
    # algorithmic bytes of step 1: Q and K read once, the pooled proxies written
    pool_bytes = L * (Hq + Hkv) * d * esz + (Hq + Hkv) * nb * d * 4
    sel_flops = 2.0 * d * Hq * nb * (nb + 1) / 2
    attn_tflops = flops / (stage_ms["attention"] * 1e-3) / 1e12
    # matrix-core attention (bf16 / e4m3); the generic kernel (fp32 inputs)
    # runs on the fp32 vector ALUs
    bound = "mfma" if mfma_path else "alu"
    peak = PEAK["fp8"] if cfg.dtype == "fp8" else (PEAK["bf16"] if mfma_path else PEAK["fp32"])
    wl = (cfg.name + f"_tau{tau:g}" + ("_group" if args.select == "group" else "")
          + ("_pack" if args.attention == "pack" else ""))
    traffic = measured_traffic(wl, kernel)
    res = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_layer": round(ms_step, 4),
        "ms_per_step_median": round(float(np.median(per_step)), 4),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "infinity_cache_evicted_mib": args.evict_mib,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; sink / vertical / slash structure, RoPE theta 5e5)",
        "config": {"workload": wl, "seq_len": L, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": d, "block_size": B, "tau": tau, "dtype": cfg.dtype,
                   "batch": 1},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "density": round(density, 5),
        "kept_tflop": round(flops / 1e12, 4),
        "row_counts": {"mean": round(float(counts.mean()), 2), "max": int(counts.max()),
                       "p50": float(np.percentile(counts, 50)),
                       "p99": float(np.percentile(counts, 99))},
        "attention_tflops": round(attn_tflops, 2),
        "pool_gbs": round(pool_bytes / (stage_ms["pool"] * 1e-3) / 1e9, 1),
        "pool_hbm_frac": round(pool_bytes / (stage_ms["pool"] * 1e-3) / 1e9 / PEAK["hbm_gbs"], 4),
        "select_tflops_fp32": round(sel_flops / (stage_ms["select"] * 1e-3) / 1e12, 2),
        "select_fp32_frac": round(sel_flops / (stage_ms["select"] * 1e-3) / 1e12 / PEAK["fp32"], 4),
        # the attention stage's events also hold its V^T layout pass (matrix-core
        # path), so "achieved" slightly understates the attention kernel alone
        "roofline": {"bound": bound, "achieved": round(attn_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                     "traffic": traffic},
        "attention_kernel": kernel,
        "attention_stage_includes_vt_pass": bool(mfma_path),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.select == "threshold":  # its sample checks per-head lists
        print("[bench] CPU oracle sample", file=sys.stderr, flush=True)
        idx = pf.ws.indices()
        tri = lambda h, i: h * (nb * (nb + 1) // 2) + i * (i + 1) // 2  # noqa: E731

        def lists_gpu(h, i):
            o = tri(h, i)
            return idx[o:o + int(counts[h, i])].cpu().numpy()

        res["cpu_baseline"] = cpu_baseline(layer, lists_gpu, counts, cfg, tau, args.cpu_seconds)
    if nb <= 2048:
        # the sorting / cumulative-sum selection rules the threshold replaces,
        # on the same proxies, timed outside the step (top-k at the threshold's
        # mean kept count, top-p at 0.9)
        k_match = max(1, int(round(float(counts.mean()))))
        res["select_baselines"] = select_baselines(pf, _lib, torch, stage_ms["select"], k_match, 0.9)
        select()  # leave the step's lists in the workspace
    if (not args.no_pack and args.attention == "default" and cfg.dtype == "bf16" and d == 128 and B == 128
            and (Hq // Hkv) % 2 == 0):
        # the same lists attended with two query heads per workgroup
        print("[bench] two-heads-per-workgroup attention", file=sys.stderr, flush=True)
        res["pack_attention"] = pack_attention(pf, torch, flops, stage_ms["attention"])
    if not args.no_group and args.select == "threshold" and Hq > Hkv and tau > 0:
        # one list per kv group (the union of its heads' selections)
        print("[bench] group-shared selection", file=sys.stderr, flush=True)
        res["group_select"] = group_select(pf, torch, kept_pairs, cfg, stage_ms)
        pf.select()
    if not args.no_varlen and args.config == "c4":
        # a batch of sequences with K/V in pages, totalling about the same tokens
        print("[bench] varlen batch", file=sys.stderr, flush=True)
        from block_sparse_long_04_amd.inputs import make_batch
        del layer
        res["varlen_batch"] = varlen_batch(cfg, _lib, make_batch, kept_pairs, torch, np)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
