"""Host logic of bench.py (CPU only): the kept-pair count behind the FLOP
figures, the single-GPU guard, and the traffic record lookup."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _pairs_by_enumeration(counts, L, B):
    # every row keeps its c - 1 earliest blocks and the diagonal; count the
    # (query t, key s) pairs with s in a kept block and s <= t one by one
    total = 0
    Hq, nb = counts.shape
    for h in range(Hq):
        for i in range(nb):
            kept = list(range(int(counts[h, i]) - 1)) + [i]
            for t in range(i * B, min((i + 1) * B, L)):
                for j in kept:
                    total += sum(1 for s in range(j * B, min((j + 1) * B, L)) if s <= t)
    return total


def test_kept_pairs_match_enumeration_with_a_ragged_last_block():
    L, B = 300, 64  # 5 blocks, the last one 44 rows
    nb = (L + B - 1) // B
    rng = np.random.default_rng(0)
    counts = np.array([[rng.integers(1, i + 2) for i in range(nb)] for _ in range(2)], dtype=np.int32)
    assert bench.kept_pairs(counts, L, B) == _pairs_by_enumeration(counts, L, B)


def test_dense_kept_pairs_are_the_causal_triangle():
    L, B = 1000, 128
    nb = (L + B - 1) // B
    counts = np.tile(np.arange(1, nb + 1, dtype=np.int32), (3, 1))
    assert bench.kept_pairs(counts, L, B) == 3 * L * (L + 1) // 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single-GPU" in r.stderr


def test_traffic_record_needs_the_current_attention_source(tmp_path, monkeypatch):
    rec = {"w": {"bytes_per_launch": 123, "source_hash": bench.source_hash(bench.ATTN_SOURCES["default"])},
           "w_pack": {"bytes_per_launch": 77, "source_hash": bench.source_hash(bench.ATTN_SOURCES["pack"])},
           "stale": {"bytes_per_launch": 456, "source_hash": "0" * 16}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "attn_traffic.json").write_text(json.dumps(rec))
    for f in set(bench.ATTN_SOURCES["default"]) | set(bench.ATTN_SOURCES["pack"]):
        os.makedirs(tmp_path / os.path.dirname(f), exist_ok=True)
        with open(os.path.join(ROOT, f), "rb") as src, open(tmp_path / f, "wb") as dst:
            dst.write(src.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w") == 123
    assert bench.measured_traffic("w_pack", "pack") == 77
    assert bench.measured_traffic("w_pack") is None  # keyed on the other kernel's sources
    assert bench.measured_traffic("stale") is None
    assert bench.measured_traffic("missing") is None
    # a change to a source of one kernel invalidates that kernel's record only
    with open(tmp_path / bench.ATTN_SOURCES["pack"][0], "ab") as f:
        f.write(b"\n")
    assert bench.measured_traffic("w_pack", "pack") is None
    assert bench.measured_traffic("w") == 123


def test_attention_kernel_follows_the_library_dispatch():
    # the same rule as the library's dispatch: d = B = 128 bf16 / e4m3 on the
    # 128-wide kernel, other bf16 shapes with d, B in {64, 128} on the 64-key
    # unit kernel, the rest (fp32, e4m3 with d or B = 64) on the generic one
    assert bench.attention_kernel("bf16", 128, 128) == "default"
    assert bench.attention_kernel("fp8", 128, 128) == "default"
    assert bench.attention_kernel("bf16", 128, 128, "pack") == "pack"
    assert bench.attention_kernel("bf16", 64, 64) == "small"
    assert bench.attention_kernel("bf16", 64, 128) == "small"
    assert bench.attention_kernel("bf16", 128, 64) == "small"
    assert bench.attention_kernel("fp8", 64, 128) == "generic"
    assert bench.attention_kernel("f32", 128, 128) == "generic"
    assert bench.attention_kernel("f32", 64, 64) == "generic"
