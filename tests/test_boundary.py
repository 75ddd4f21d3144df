"""CPU checks of the C-ABI library: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any launch (every
call here returns an error code without touching a GPU)."""
import ctypes
import math
import os
import re

import pytest

import block_sparse_long_04_amd as fp
from block_sparse_long_04_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashprefill.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(fp_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = fp.load_library()
    names = header_functions()
    assert names == sorted(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_header(tmp_path):
    # offsets and sizes of the ctypes mirrors equal what a C compiler makes of
    # the header
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "flashprefill.h"',
             'int main(void) {']
    structs = (("fp_problem", fp.FpProblem), ("fp_ws_layout", fp.FpWsLayout), ("fp_varlen", fp.FpVarlen),
               ("fp_ws_layout_varlen", fp.FpWsLayoutVarlen))
    for struct, cls in structs:
        lines.append(f'printf("{struct} %zu\\n", sizeof({struct}));')
        for name, _ in cls._fields_:
            lines.append(f'printf("{struct}.{name} %zu\\n", offsetof({struct}, {name}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = dict(ln.split() for ln in subprocess.run([str(exe)], capture_output=True, text=True,
                                                    check=True).stdout.splitlines())
    for struct, cls in structs:
        assert int(got[struct]) == ctypes.sizeof(cls)
        for name, _ in cls._fields_:
            assert int(got[f"{struct}.{name}"]) == getattr(cls, name).offset, name


def prob(**kw):
    base = dict(seq_len=1000, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype=fp.FP_BF16)
    base.update({k: v for k, v in kw.items() if k in base})
    p = fp.make_problem(None, None, None, None, kw.get("block_size", 128), kw.get("threshold", 0.1),
                        **base)
    for k, v in kw.items():
        if k not in base and k not in ("block_size", "threshold"):
            setattr(p, k, v)
    return p


def test_workspace_layout_sizes_and_alignment():
    p = prob()
    lay = fp.fp_workspace_layout(p)
    nb = 8
    assert lay.q_pool == 0
    assert lay.k_pool == 8 * nb * 128 * 4
    offs = [lay.q_pool, lay.k_pool, lay.row_max, lay.counts, lay.indices, lay.v_t, lay.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.indices - lay.counts >= 8 * nb * 4
    assert lay.v_t - lay.indices >= 8 * nb * (nb + 1) // 2 * 4
    assert lay.total - lay.v_t == 2 * 128 * nb * 128 * 2  # V^T in bf16
    lay32 = fp.fp_workspace_layout(prob(dtype=fp.FP_F32))
    assert lay32.total == lay32.v_t  # no V^T for fp32 inputs


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("d,B", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_vt_section_follows_the_attention_dispatch(dtype, d, B):
    # The V^T section exists exactly when the attention runs on the matrix
    # cores (its kernels read V^T): bf16 or e4m3 with d = B = 128, bf16 with
    # d and B in {64, 128}.  The host computes the layout, so the dispatch
    # rule is checked here without a GPU, against the same rule bench.py
    # uses to name the kernel it measures.
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    code = {"f32": fp.FP_F32, "bf16": fp.FP_BF16, "fp8": fp.FP_FP8_E4M3}[dtype]
    lay = fp.fp_workspace_layout(prob(dtype=code, head_dim=d, block_size=B))
    nb = (1000 + B - 1) // B
    matrix = bench.attention_kernel(dtype, d, B) != "generic"
    assert lay.total - lay.v_t == (2 * d * nb * B * 2 if matrix else 0)


@pytest.mark.parametrize("field,value,code", [
    ("threshold", float("nan"), fp.FP_ERR_INVALID),
    ("threshold", -0.01, fp.FP_ERR_INVALID),
    ("threshold", 1.5, fp.FP_ERR_INVALID),
    ("num_kv_heads", 3, fp.FP_ERR_INVALID),
    ("num_q_heads", 0, fp.FP_ERR_INVALID),
    ("seq_len", -1, fp.FP_ERR_INVALID),
    ("head_dim", 96, fp.FP_ERR_UNSUPPORTED),
    ("block_size", 32, fp.FP_ERR_UNSUPPORTED),
    ("causal", 0, fp.FP_ERR_UNSUPPORTED),
    ("dtype", 7, fp.FP_ERR_INVALID),
    ("q_stride_head", 100, fp.FP_ERR_INVALID),  # 200 bytes: not a multiple of 16
    ("o_stride_tok", 128, fp.FP_ERR_INVALID),   # output rows of different heads overlap
    ("sm_scale", float("inf"), fp.FP_ERR_INVALID),
    ("seq_len", 16385 * 128, fp.FP_ERR_UNSUPPORTED),
])
def test_invalid_problem_rejected(field, value, code):
    p = prob()
    setattr(p, field, value)
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_workspace_layout(p)
    assert e.value.code == code


def test_fp8_scales_validated():
    p = prob(dtype=fp.FP_FP8_E4M3)
    p.q_scale = 0.0
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_workspace_layout(p)
    assert e.value.code == fp.FP_ERR_INVALID
    p.q_scale = float("inf")
    with pytest.raises(fp.FlashPrefillError):
        fp.fp_workspace_layout(p)


def test_entry_points_reject_before_launch():
    # Host-side errors come back before any HIP call: null tensors, null or
    # misaligned or short workspace.  Fake addresses are never dereferenced.
    p = prob()
    lay = fp.fp_workspace_layout(p)
    fake = 1 << 20
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_block_pool(p, fake, lay.total, 0)  # q/k are NULL
    assert e.value.code == fp.FP_ERR_INVALID
    p.q, p.k, p.v, p.out = fake, fake, fake, fake
    for fn in (fp.fp_block_pool, fp.fp_block_select, fp.fp_block_select_group, fp.fp_sparse_prefill):
        with pytest.raises(fp.FlashPrefillError) as e:
            fn(p, 0, lay.total, 0)
        assert e.value.code == fp.FP_ERR_WORKSPACE
        with pytest.raises(fp.FlashPrefillError) as e:
            fn(p, fake + 16, lay.total, 0)
        assert e.value.code == fp.FP_ERR_WORKSPACE
        with pytest.raises(fp.FlashPrefillError) as e:
            fn(p, fake, lay.total - 1, 0)
        assert e.value.code == fp.FP_ERR_WORKSPACE
    p.q = fake + 8  # misaligned tensor
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_block_pool(p, fake, lay.total, 0)
    assert e.value.code == fp.FP_ERR_INVALID


def test_empty_problem_is_a_no_op():
    p = prob(seq_len=0)
    lay = fp.fp_workspace_layout(p)
    for fn in (fp.fp_block_pool, fp.fp_block_select, fp.fp_block_select_group, fp.fp_sparse_prefill):
        fn(p, 0, 0, 0)  # nothing launched, nothing read
    assert lay.total == 0


def test_group_selection_validates_like_the_main_selection():
    fake = 1 << 20
    for field, value, code in (("threshold", 1.5, fp.FP_ERR_INVALID), ("num_kv_heads", 3, fp.FP_ERR_INVALID),
                               ("causal", 0, fp.FP_ERR_UNSUPPORTED)):
        p = prob(**{field: value})
        with pytest.raises(fp.FlashPrefillError) as e:
            fp.fp_block_select_group(p, fake, 1 << 40, 0)
        assert e.value.code == code, field


def test_strerror_texts():
    for code in (0, -1, -2, -3, -4):
        assert fp.strerror(code)
    assert "unknown" in fp.strerror(12345)


def test_sorted_selection_rejects_bad_rules_and_sizes_before_launch():
    p = prob()
    lay = fp.fp_workspace_layout(p)
    fake = 1 << 20
    p.q, p.k, p.v, p.out = fake, fake, fake, fake
    for rule, param in ((fp.FP_SELECT_TOPK, 0.0), (fp.FP_SELECT_TOPK, 2.5), (fp.FP_SELECT_TOPK, -3.0),
                        (fp.FP_SELECT_TOPP, 0.0), (fp.FP_SELECT_TOPP, 1.5),
                        (fp.FP_SELECT_TOPP, float("nan")), (0, 1.0), (3, 1.0)):
        with pytest.raises(fp.FlashPrefillError) as e:
            fp.fp_block_select_sorted(p, rule, param, fake, lay.total, 0)
        assert e.value.code == fp.FP_ERR_INVALID, (rule, param)
    # workspace checks as for the other entry points
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_block_select_sorted(p, fp.FP_SELECT_TOPK, 4.0, fake, lay.total - 1, 0)
    assert e.value.code == fp.FP_ERR_WORKSPACE
    # rows are sorted whole in LDS: more than 2048 blocks is unsupported
    big = prob(seq_len=2049 * 128)
    big.q, big.k, big.v, big.out = fake, fake, fake, fake
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_block_select_sorted(big, fp.FP_SELECT_TOPP, 0.9, fake, 1 << 40, 0)
    assert e.value.code == fp.FP_ERR_UNSUPPORTED
    # empty problem: nothing launched
    fp.fp_block_select_sorted(prob(seq_len=0), fp.FP_SELECT_TOPK, 1.0, 0, 0, 0)


def _varlen(lens, table=False, max_blocks=0, num_pages=0, kps=0, vps=0):
    vl = fp.FpVarlen()
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    arr = (ctypes.c_int32 * len(cu))(*cu)
    vl.num_seqs = len(lens)
    vl.cu_seqlens = arr
    vl.cu_seqlens_dev = 1 << 20
    vl.block_table_dev = (1 << 21) if table else None
    vl.max_blocks, vl.num_pages, vl.k_page_stride, vl.v_page_stride = max_blocks, num_pages, kps, vps
    return vl, arr, cu[-1]


def test_varlen_layout_and_host_validation():
    lens = [300, 129, 0, 1000]
    vl, arr, T = _varlen(lens)
    p = prob(seq_len=T)
    lay = fp.fp_workspace_layout_varlen(p, vl)
    nbs = [(L + 127) // 128 for L in lens]
    NB = sum(nbs)
    offs = [lay.q_pool, lay.k_pool, lay.row_max, lay.counts, lay.indices, lay.v_t, lay.k_c, lay.meta, lay.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.k_pool - lay.q_pool >= 8 * NB * 128 * 4
    assert lay.v_t - lay.indices >= 8 * sum(n * (n + 1) // 2 for n in nbs) * 4
    assert lay.k_c - lay.v_t >= 2 * 128 * NB * 128 * 2
    assert lay.meta - lay.k_c >= 2 * NB * 128 * 128 * 2
    assert lay.total - lay.meta >= NB * 16 + len(lens) * 16
    fake = 1 << 22
    p.q, p.k, p.v, p.out = fake, fake, fake, fake
    # cu_seqlens must start at 0, end at seq_len and not decrease
    for bad in ([0, 300, 200, 1429], [1, 300, 429, 1429], [0, 300, 429, 1428]):
        a = (ctypes.c_int32 * len(bad))(*bad)
        v2, _, _ = _varlen([1])
        v2.num_seqs, v2.cu_seqlens = len(bad) - 1, a
        with pytest.raises(fp.FlashPrefillError) as e:
            fp.fp_workspace_layout_varlen(prob(seq_len=1429), v2)
        assert e.value.code == fp.FP_ERR_INVALID
    # only the matrix-core shapes
    for kw in (dict(dtype=fp.FP_F32), dict(head_dim=64), dict(block_size=64)):
        with pytest.raises(fp.FlashPrefillError) as e:
            fp.fp_workspace_layout_varlen(prob(seq_len=T, **kw), vl)
        assert e.value.code == fp.FP_ERR_UNSUPPORTED
    # paged: the block table must cover every sequence, strides must be aligned
    vp, _, _ = _varlen(lens, table=True, max_blocks=7, num_pages=20, kps=128 * 2 * 128, vps=128 * 2 * 128)
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_workspace_layout_varlen(p, vp)
    assert e.value.code == fp.FP_ERR_INVALID
    vp.max_blocks = 8
    fp.fp_workspace_layout_varlen(p, vp)
    vp.k_page_stride = 3
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_workspace_layout_varlen(p, vp)
    assert e.value.code == fp.FP_ERR_INVALID
    # workspace checks before any launch
    for fn in (fp.fp_block_pool_varlen, fp.fp_block_select_varlen, fp.fp_sparse_prefill_varlen):
        with pytest.raises(fp.FlashPrefillError) as e:
            fn(p, vl, fake, lay.total - 1, 0)
        assert e.value.code == fp.FP_ERR_WORKSPACE
    # an empty batch is a no-op
    ve, _, _ = _varlen([0, 0])
    for fn in (fp.fp_block_pool_varlen, fp.fp_block_select_varlen, fp.fp_sparse_prefill_varlen):
        fn(prob(seq_len=0), ve, 0, 0, 0)


def test_probe_selection_shapes_checked_before_launch():
    fake = 1 << 20
    for kw, code in ((dict(dtype=fp.FP_F32), fp.FP_ERR_UNSUPPORTED), (dict(head_dim=64), fp.FP_ERR_UNSUPPORTED),
                     (dict(seq_len=1025 * 128), fp.FP_ERR_UNSUPPORTED)):
        p = prob(**kw)
        p.q, p.k, p.v, p.out = fake, fake, fake, fake
        with pytest.raises(fp.FlashPrefillError) as e:
            fp.fp_block_select_probe(p, fake, 1 << 40, 0)
        assert e.value.code == code, kw
    p = prob()
    lay = fp.fp_workspace_layout(p)
    p.q, p.k, p.v, p.out = fake, fake, fake, fake
    with pytest.raises(fp.FlashPrefillError) as e:
        fp.fp_block_select_probe(p, fake, lay.total - 1, 0)
    assert e.value.code == fp.FP_ERR_WORKSPACE
    fp.fp_block_select_probe(prob(seq_len=0), 0, 0, 0)


def test_binding_fails_loudly_without_the_library(tmp_path):
    # a fresh interpreter pointed at a missing library: loading raises, and
    # there is no fallback path that would compute anything on the host
    code = (
        "import sys\n"
        "from block_sparse_long_04_amd import _lib\n"
        "try:\n"
        f"    _lib.load_library({str(tmp_path / 'absent.so')!r})\n"
        "except FileNotFoundError as e:\n"
        "    print('raised', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(1)\n"
    )
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "raised" in r.stdout


def _valid_lists(Hq, nb, seed=0):
    import numpy as np
    rng = np.random.default_rng(seed)
    tri = nb * (nb + 1) // 2
    counts = np.zeros((Hq, nb), np.int32)
    idx = np.full(Hq * tri, -7, np.int32)  # unused slots hold garbage on purpose
    for h in range(Hq):
        for i in range(nb):
            lst = sorted(set(rng.choice(i + 1, size=rng.integers(0, i + 1), replace=False).tolist()) | {i})
            counts[h, i] = len(lst)
            off = h * tri + i * (i + 1) // 2
            idx[off: off + len(lst)] = lst
    return counts, idx


def test_list_validation_rejects_bad_lists_before_any_write():
    """Caller-made lists are checked on the host (count in [1, i+1],
    ascending, inside [0, i], ending with i) before they reach the
    workspace; a bad list leaves the workspace untouched.  The workspace here
    is host memory: no GPU is involved."""
    import numpy as np
    import torch
    Hq, nb = 3, 9
    p = prob(seq_len=nb * 128 - 50, num_q_heads=Hq, num_kv_heads=1)
    ws = _lib.alloc_workspace(p, "cpu")
    ws.buf.fill_(0)
    counts, idx = _valid_lists(Hq, nb)
    _lib.validate_lists(counts, idx, nb)
    tri = nb * (nb + 1) // 2

    def row_off(h, i):
        return h * tri + i * (i + 1) // 2

    bad = []
    c = counts.copy(); c[1, 4] = 0; bad.append((c, idx))                       # empty list
    c = counts.copy(); c[2, 3] = 5; bad.append((c, idx))                       # count > i + 1
    x = idx.copy(); x[row_off(0, 6) + counts[0, 6] - 1] = 7; bad.append((counts, x))  # past i
    x = idx.copy(); x[row_off(1, 8)] = -1; bad.append((counts, x))            # negative
    h, i = 2, 8
    c = counts.copy(); x = idx.copy()
    lst = list(range(0, i + 1))
    c[h, i] = len(lst); x[row_off(h, i): row_off(h, i) + len(lst)] = lst
    _lib.validate_lists(c, x, nb)                                              # dense row is fine
    y = x.copy(); y[row_off(h, i) + 3] = y[row_off(h, i) + 2]; bad.append((c, y))  # repeated entry
    y = x.copy(); y[row_off(h, i) + 3], y[row_off(h, i) + 4] = 4, 3; bad.append((c, y))  # not ascending
    c2 = c.copy(); c2[h, i] = i; bad.append((c2, x))                           # does not end with i
    for cb, xb in bad:
        with pytest.raises(_lib.FlashPrefillError) as e:
            ws.set_lists(cb, xb)
        assert e.value.code == _lib.FP_ERR_INVALID
        assert int(ws.buf.sum()) == 0
    ws.set_lists(counts, idx)
    assert np.array_equal(ws.counts().numpy(), counts)
    assert np.array_equal(ws.indices().numpy(), idx)


def test_noalloc_rejects_problems_larger_than_its_buffer_before_any_gpu_call():
    """fp_prefill_noalloc checks the problem and its workspace size against
    the fixed scratch buffer on the host first: a 32K-token, 32 / 8-head
    layer needs more and is refused with FP_ERR_SCRATCH, and a bad problem
    with FP_ERR_INVALID, without touching a GPU (none is visible here)."""
    p = prob(seq_len=32768, num_q_heads=32, num_kv_heads=8)
    assert _lib.fp_workspace_layout(p).total > _lib.FP_NOALLOC_SCRATCH_BYTES
    p.q = p.k = p.v = p.out = 1 << 20  # aligned, non-null: only the size check refuses
    with pytest.raises(_lib.FlashPrefillError) as e:
        _lib.fp_prefill_noalloc(p, 0)
    assert e.value.code == _lib.FP_ERR_SCRATCH
    small = prob(seq_len=4096, num_q_heads=32, num_kv_heads=8)
    assert _lib.fp_workspace_layout(small).total <= _lib.FP_NOALLOC_SCRATCH_BYTES
    with pytest.raises(_lib.FlashPrefillError) as e:  # null pointers
        _lib.fp_prefill_noalloc(small, 0)
    assert e.value.code == _lib.FP_ERR_INVALID
