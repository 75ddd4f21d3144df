"""ctypes binding of libflashprefill.so (argument marshalling only).

Every step of the computation runs in the HIP library; this module only turns
torch tensors into the fp_problem struct of include/flashprefill.h (device
pointers, element strides, dtype, scales), hands over torch's current HIP
stream, and allocates the caller-owned workspace and output with torch.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libflashprefill.so")

FP_F32, FP_BF16, FP_FP8_E4M3 = 0, 1, 2
FP_OK, FP_ERR_INVALID, FP_ERR_UNSUPPORTED, FP_ERR_WORKSPACE, FP_ERR_HIP, FP_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
FP_NOALLOC_SCRATCH_BYTES = 64 << 20

FP_SELECT_TOPK, FP_SELECT_TOPP = 1, 2

EXPORTED = ("fp_workspace_layout", "fp_block_pool", "fp_block_select", "fp_block_select_group",
            "fp_block_select_sorted",
            "fp_block_select_probe", "fp_sparse_prefill", "fp_workspace_layout_varlen", "fp_block_pool_varlen",
            "fp_block_select_varlen", "fp_sparse_prefill_varlen", "fp_prefill_noalloc",
            "fp_sparse_prefill_pack", "fp_strerror")


class FpProblem(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("seq_len", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("k_stride_tok", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("v_stride_tok", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
        ("o_stride_tok", ctypes.c_int64), ("o_stride_head", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("q_scale", ctypes.c_float), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("sm_scale", ctypes.c_float), ("threshold", ctypes.c_float),
        ("causal", ctypes.c_int32),
    ]


class FpVarlen(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("cu_seqlens", ctypes.POINTER(ctypes.c_int32)),
                ("cu_seqlens_dev", ctypes.c_void_p), ("block_table_dev", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("k_page_stride", ctypes.c_int64), ("v_page_stride", ctypes.c_int64)]


class FpWsLayoutVarlen(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("q_pool", "k_pool", "row_max", "counts", "indices", "v_t", "k_c", "meta", "total")]


class FpWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("q_pool", "k_pool", "row_max", "counts", "indices", "v_t", "total")]


class FlashPrefillError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


_LIB = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once.  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m block_sparse_long_04_amd.build`")
    lib = ctypes.CDLL(path)
    P, W = ctypes.POINTER(FpProblem), ctypes.POINTER(FpWsLayout)
    lib.fp_workspace_layout.argtypes = [P, W]
    lib.fp_workspace_layout.restype = ctypes.c_int
    for name in ("fp_block_pool", "fp_block_select", "fp_block_select_group", "fp_block_select_probe",
                 "fp_sparse_prefill", "fp_sparse_prefill_pack"):
        fn = getattr(lib, name)
        fn.argtypes = [P, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.fp_block_select_sorted.argtypes = [P, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p]
    lib.fp_block_select_sorted.restype = ctypes.c_int
    VL = ctypes.POINTER(FpVarlen)
    lib.fp_workspace_layout_varlen.argtypes = [P, VL, ctypes.POINTER(FpWsLayoutVarlen)]
    lib.fp_workspace_layout_varlen.restype = ctypes.c_int
    for name in ("fp_block_pool_varlen", "fp_block_select_varlen", "fp_sparse_prefill_varlen"):
        fn = getattr(lib, name)
        fn.argtypes = [P, VL, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.fp_prefill_noalloc.argtypes = [P, ctypes.c_void_p]
    lib.fp_prefill_noalloc.restype = ctypes.c_int
    lib.fp_strerror.argtypes = [ctypes.c_int]
    lib.fp_strerror.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def strerror(code: int) -> str:
    return load_library().fp_strerror(code).decode()


def _check(code: int, where: str):
    if code != FP_OK:
        raise FlashPrefillError(code, where)


# ----------------------------------------------------------------------------
# Raw entry points (same names as the C ABI)
# ----------------------------------------------------------------------------

def fp_workspace_layout(prob: FpProblem) -> FpWsLayout:
    lay = FpWsLayout()
    _check(load_library().fp_workspace_layout(ctypes.byref(prob), ctypes.byref(lay)),
           "fp_workspace_layout")
    return lay


def fp_block_pool(prob: FpProblem, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(load_library().fp_block_pool(ctypes.byref(prob), ws_ptr, ws_bytes, stream),
           "fp_block_pool")


def fp_block_select(prob: FpProblem, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(load_library().fp_block_select(ctypes.byref(prob), ws_ptr, ws_bytes, stream),
           "fp_block_select")


def fp_block_select_group(prob: FpProblem, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(load_library().fp_block_select_group(ctypes.byref(prob), ws_ptr, ws_bytes, stream),
           "fp_block_select_group")


def fp_block_select_sorted(prob: FpProblem, rule: int, param: float, ws_ptr: int, ws_bytes: int,
                           stream: int) -> None:
    _check(load_library().fp_block_select_sorted(ctypes.byref(prob), rule, param, ws_ptr, ws_bytes,
                                                 stream), "fp_block_select_sorted")


def fp_block_select_probe(prob: FpProblem, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(load_library().fp_block_select_probe(ctypes.byref(prob), ws_ptr, ws_bytes, stream),
           "fp_block_select_probe")


def fp_sparse_prefill(prob: FpProblem, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(load_library().fp_sparse_prefill(ctypes.byref(prob), ws_ptr, ws_bytes, stream),
           "fp_sparse_prefill")


def fp_sparse_prefill_pack(prob: FpProblem, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(load_library().fp_sparse_prefill_pack(ctypes.byref(prob), ws_ptr, ws_bytes, stream),
           "fp_sparse_prefill_pack")


def fp_prefill_noalloc(prob: FpProblem, stream: int) -> None:
    _check(load_library().fp_prefill_noalloc(ctypes.byref(prob), stream), "fp_prefill_noalloc")


def fp_workspace_layout_varlen(prob: FpProblem, vl: FpVarlen) -> FpWsLayoutVarlen:
    lay = FpWsLayoutVarlen()
    _check(load_library().fp_workspace_layout_varlen(ctypes.byref(prob), ctypes.byref(vl), ctypes.byref(lay)),
           "fp_workspace_layout_varlen")
    return lay


def fp_block_pool_varlen(prob, vl, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(load_library().fp_block_pool_varlen(ctypes.byref(prob), ctypes.byref(vl), ws_ptr, ws_bytes, stream),
           "fp_block_pool_varlen")


def fp_block_select_varlen(prob, vl, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(load_library().fp_block_select_varlen(ctypes.byref(prob), ctypes.byref(vl), ws_ptr, ws_bytes, stream),
           "fp_block_select_varlen")


def fp_sparse_prefill_varlen(prob, vl, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(load_library().fp_sparse_prefill_varlen(ctypes.byref(prob), ctypes.byref(vl), ws_ptr, ws_bytes,
                                                   stream), "fp_sparse_prefill_varlen")


# ----------------------------------------------------------------------------
# torch-facing helpers
# ----------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FP_F32
    if t.dtype == torch.bfloat16:
        return FP_BF16
    if t.dtype == torch.float8_e4m3fn:
        return FP_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_problem(q, k, v, out, block_size: int, threshold: float, sm_scale: float = 0.0,
                 q_scale: float = 1.0, k_scale: float = 1.0, v_scale: float = 1.0,
                 seq_len: Optional[int] = None, num_q_heads: Optional[int] = None,
                 num_kv_heads: Optional[int] = None, head_dim: Optional[int] = None,
                 dtype: Optional[int] = None) -> FpProblem:
    """fp_problem for [L, H, d] tensors (any of them may be None: pointer 0;
    shapes then come from the keyword overrides)."""
    p = FpProblem()
    ref_q = q if q is not None else None
    p.q = q.data_ptr() if q is not None else 0
    p.k = k.data_ptr() if k is not None else 0
    p.v = v.data_ptr() if v is not None else 0
    p.out = out.data_ptr() if out is not None else 0
    p.seq_len = seq_len if seq_len is not None else ref_q.shape[0]
    p.num_q_heads = num_q_heads if num_q_heads is not None else ref_q.shape[1]
    p.num_kv_heads = num_kv_heads if num_kv_heads is not None else k.shape[1]
    p.head_dim = head_dim if head_dim is not None else ref_q.shape[2]
    p.block_size = block_size

    def strides(t, H, d):
        if t is None:  # contiguous default
            return H * d, d
        assert t.stride(2) == 1, "last dim must be contiguous"
        return t.stride(0), t.stride(1)

    p.q_stride_tok, p.q_stride_head = strides(q, p.num_q_heads, p.head_dim)
    p.k_stride_tok, p.k_stride_head = strides(k, p.num_kv_heads, p.head_dim)
    p.v_stride_tok, p.v_stride_head = strides(v, p.num_kv_heads, p.head_dim)
    p.o_stride_tok, p.o_stride_head = strides(out, p.num_q_heads, p.head_dim)
    p.dtype = dtype if dtype is not None else _dtype_code(q)
    p.q_scale, p.k_scale, p.v_scale = q_scale, k_scale, v_scale
    p.sm_scale = sm_scale
    p.threshold = threshold
    p.causal = 1
    return p


@dataclass
class Workspace:
    """Caller-owned workspace (a torch uint8 device tensor) plus typed views of
    its sections (see fp_ws_layout)."""

    buf: "object"
    layout: FpWsLayout
    nb: int
    Hq: int
    Hkv: int
    d: int

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()

    @property
    def nbytes(self) -> int:
        return self.buf.numel()

    def _view(self, off, count, dtype):
        import torch
        esz = torch.empty((), dtype=dtype).element_size()
        return self.buf[off: off + count * esz].view(dtype)

    def q_pool(self):
        import torch
        return self._view(self.layout.q_pool, self.Hq * self.nb * self.d, torch.float32).view(
            self.Hq, self.nb, self.d)

    def k_pool(self):
        import torch
        return self._view(self.layout.k_pool, self.Hkv * self.nb * self.d, torch.float32).view(
            self.Hkv, self.nb, self.d)

    def row_max(self):
        import torch
        return self._view(self.layout.row_max, self.Hq * self.nb, torch.float32).view(self.Hq, self.nb)

    def counts(self):
        import torch
        return self._view(self.layout.counts, self.Hq * self.nb, torch.int32).view(self.Hq, self.nb)

    def indices(self):
        import torch
        return self._view(self.layout.indices, self.Hq * self.nb * (self.nb + 1) // 2, torch.int32)

    def set_lists(self, counts, indices) -> None:
        """Write caller-made lists (host arrays: counts [Hq, nb], flat
        triangular indices) into the workspace, after validate_lists."""
        import numpy as np
        import torch
        validate_lists(counts, indices, self.nb)
        tri = self.Hq * self.nb * (self.nb + 1) // 2
        self.counts().copy_(torch.from_numpy(np.ascontiguousarray(counts, dtype=np.int32)))
        self.indices().copy_(torch.from_numpy(np.ascontiguousarray(np.asarray(indices).reshape(-1)[:tri],
                                                                   dtype=np.int32)))


def validate_lists(counts, indices, nb: int) -> None:
    """Host-side check of caller-written block lists before they go into a
    workspace: for every (h, i), 1 <= counts[h, i] <= i + 1 and the entries
    at indices[h*nb(nb+1)/2 + i(i+1)/2 ...] are strictly ascending, inside
    [0, i] and end with i (the diagonal).  The attention kernels trust the
    lists they are given, so a list that breaks these rules must never reach
    them.  counts: [Hq, nb] int array; indices: the flat triangular array (or
    at least its used entries).  Raises FlashPrefillError(FP_ERR_INVALID)."""
    import numpy as np
    counts = np.asarray(counts)
    indices = np.asarray(indices).reshape(-1)
    if counts.ndim != 2 or counts.shape[1] != nb:
        raise FlashPrefillError(FP_ERR_INVALID, "validate_lists: counts shape")
    Hq = counts.shape[0]
    tri = nb * (nb + 1) // 2
    if indices.size < Hq * tri:
        raise FlashPrefillError(FP_ERR_INVALID, "validate_lists: indices too short")
    i = np.arange(nb)
    if (counts < 1).any() or (counts > i[None, :] + 1).any():
        raise FlashPrefillError(FP_ERR_INVALID, "validate_lists: count outside [1, i + 1]")
    row = np.repeat(i, i + 1)                        # row of every triangular slot
    off = np.arange(tri) - (i * (i + 1) // 2)[row]   # slot within its row
    for h in range(Hq):
        sec = indices[h * tri:(h + 1) * tri].astype(np.int64)
        used = off < counts[h][row]
        e, r, o = sec[used], row[used], off[used]
        if (e < 0).any() or (e > r).any():
            raise FlashPrefillError(FP_ERR_INVALID, f"validate_lists: entry outside [0, i] (head {h})")
        last = o == counts[h][r] - 1
        if (e[last] != r[last]).any():
            raise FlashPrefillError(FP_ERR_INVALID, f"validate_lists: list does not end with i (head {h})")
        nxt = ~last
        if (e[nxt] >= e[np.flatnonzero(nxt) + 1]).any():
            raise FlashPrefillError(FP_ERR_INVALID, f"validate_lists: entries not ascending (head {h})")


def alloc_workspace(prob: FpProblem, device) -> Workspace:
    import torch
    lay = fp_workspace_layout(prob)
    buf = torch.empty(max(int(lay.total), 256), dtype=torch.uint8, device=device)
    nb = (prob.seq_len + prob.block_size - 1) // prob.block_size
    return Workspace(buf, lay, nb, prob.num_q_heads, prob.num_kv_heads, prob.head_dim)


def current_stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


class Prefill:
    """One layer's prefill problem bound to tensors: the three C-ABI calls on
    torch's current stream.  Inputs q [L,Hq,d], k/v [L,Hkv,d] on one device
    (fp32, bf16 or float8_e4m3fn); out is allocated [L,Hq,d] (fp32 for fp32
    inputs, bf16 otherwise) unless given."""

    def __init__(self, q, k, v, block_size: int = 128, threshold: float = 0.1,
                 sm_scale: float = 0.0, q_scale: float = 1.0, k_scale: float = 1.0,
                 v_scale: float = 1.0, out=None):
        import torch
        if not q.is_cuda:
            raise ValueError("q/k/v must be device tensors")
        if out is None:
            odt = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
            out = torch.empty(q.shape, dtype=odt, device=q.device)
        self.q, self.k, self.v, self.out = q, k, v, out
        self.prob = make_problem(q, k, v, out, block_size, threshold, sm_scale,
                                 q_scale, k_scale, v_scale)
        self.ws = alloc_workspace(self.prob, q.device)
        self.device = q.device

    def stream(self) -> int:
        return current_stream(self.device)

    def pool(self):
        fp_block_pool(self.prob, self.ws.ptr, self.ws.nbytes, self.stream())

    def select(self):
        fp_block_select(self.prob, self.ws.ptr, self.ws.nbytes, self.stream())

    def select_group(self):
        """Group-shared selection (each head's own threshold, then the union
        over the heads of each kv group as every head's list) into the same
        workspace sections as select()."""
        fp_block_select_group(self.prob, self.ws.ptr, self.ws.nbytes, self.stream())

    def select_sorted(self, rule: int, param: float):
        """Top-k (rule FP_SELECT_TOPK, param = k) or top-p (FP_SELECT_TOPP,
        param = p) selection into the same workspace sections as select()."""
        fp_block_select_sorted(self.prob, rule, param, self.ws.ptr, self.ws.nbytes, self.stream())

    def select_probe(self):
        """Query-probe selection (token-level max per key block) into the same
        workspace sections as select()."""
        fp_block_select_probe(self.prob, self.ws.ptr, self.ws.nbytes, self.stream())

    def attend(self):
        fp_sparse_prefill(self.prob, self.ws.ptr, self.ws.nbytes, self.stream())

    def attend_pack(self):
        """Attention with two query heads per workgroup (fp_sparse_prefill_pack)."""
        fp_sparse_prefill_pack(self.prob, self.ws.ptr, self.ws.nbytes, self.stream())

    def run(self):
        self.pool()
        self.select()
        self.attend()
        return self.out


def prefill(q, k, v, threshold: float = 0.1, block_size: int = 128, **kw):
    """Block-sparse causal prefill of one layer; returns (out, Prefill)."""
    pf = Prefill(q, k, v, block_size=block_size, threshold=threshold, **kw)
    return pf.run(), pf


def default_sm_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


class PrefillVarlen:
    """A batch of sequences (varlen): q / out packed [T, Hq, d]; k / v packed
    [T, Hkv, d], or page caches [pages, B, Hkv, d] with a block table
    [S, max_blocks] of page ids.  cu_seqlens: S + 1 token offsets (host list).
    Same pool / select / attend steps as Prefill, over every sequence."""

    def __init__(self, q, k, v, cu_seqlens, block_size: int = 128, threshold: float = 0.1,
                 sm_scale: float = 0.0, q_scale: float = 1.0, k_scale: float = 1.0, v_scale: float = 1.0,
                 block_table=None, out=None):
        import torch
        if not (q.is_cuda and k.is_cuda and v.is_cuda):
            raise ValueError("q/k/v must be device tensors")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        self.q, self.k, self.v, self.out = q, k, v, out
        T, Hq, d = q.shape
        Hkv = k.shape[-2]
        self.prob = make_problem(q, None, None, out, block_size, threshold, sm_scale, q_scale, k_scale,
                                 v_scale, seq_len=T, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d)
        self.prob.k, self.prob.v = k.data_ptr(), v.data_ptr()
        paged = block_table is not None
        # inside a page (or the packed tensor) token / head strides
        self.prob.k_stride_tok, self.prob.k_stride_head = k.stride(-3), k.stride(-2)
        self.prob.v_stride_tok, self.prob.v_stride_head = v.stride(-3), v.stride(-2)
        self.cu_host = (ctypes.c_int32 * len(cu_seqlens))(*[int(x) for x in cu_seqlens])
        self.cu_dev = torch.tensor([int(x) for x in cu_seqlens], dtype=torch.int32, device=q.device)
        vl = FpVarlen()
        vl.num_seqs = len(cu_seqlens) - 1
        vl.cu_seqlens = self.cu_host
        vl.cu_seqlens_dev = self.cu_dev.data_ptr()
        if paged:
            self.table = block_table.to(device=q.device, dtype=torch.int32).contiguous()
            vl.block_table_dev = self.table.data_ptr()
            vl.max_blocks = self.table.shape[1]
            vl.num_pages = k.shape[0]
            vl.k_page_stride, vl.v_page_stride = k.stride(0), v.stride(0)
        else:
            vl.block_table_dev = None
        self.vl = vl
        self.layout = fp_workspace_layout_varlen(self.prob, vl)
        self.buf = torch.empty(max(int(self.layout.total), 256), dtype=torch.uint8, device=q.device)
        B = block_size
        self.nbs = [(int(cu_seqlens[s + 1]) - int(cu_seqlens[s]) + B - 1) // B for s in range(vl.num_seqs)]
        self.NB = sum(self.nbs)
        self.Hq, self.Hkv, self.d = Hq, Hkv, d
        self.device = q.device

    def stream(self) -> int:
        return current_stream(self.device)

    def pool(self):
        fp_block_pool_varlen(self.prob, self.vl, self.buf.data_ptr(), self.buf.numel(), self.stream())

    def select(self):
        fp_block_select_varlen(self.prob, self.vl, self.buf.data_ptr(), self.buf.numel(), self.stream())

    def attend(self):
        fp_sparse_prefill_varlen(self.prob, self.vl, self.buf.data_ptr(), self.buf.numel(), self.stream())

    def run(self):
        self.pool()
        self.select()
        self.attend()
        return self.out

    def _view(self, off, count, dtype):
        import torch
        esz = torch.empty((), dtype=dtype).element_size()
        return self.buf[off: off + count * esz].view(dtype)

    def counts(self):
        import torch
        return self._view(self.layout.counts, self.Hq * self.NB, torch.int32).view(self.Hq, self.NB)

    def row_max(self):
        import torch
        return self._view(self.layout.row_max, self.Hq * self.NB, torch.float32).view(self.Hq, self.NB)

    def q_pool(self):
        import torch
        return self._view(self.layout.q_pool, self.Hq * self.NB * self.d, torch.float32).view(
            self.Hq, self.NB, self.d)

    def k_pool(self):
        import torch
        return self._view(self.layout.k_pool, self.Hkv * self.NB * self.d, torch.float32).view(
            self.Hkv, self.NB, self.d)

    def lists(self):
        """Host lists [s][h][i] (local block indices) from the workspace."""
        import numpy as np
        counts = self.counts().cpu().numpy()
        total = sum(self.Hq * n * (n + 1) // 2 for n in self.nbs)
        idx = self._view(self.layout.indices, total, __import__("torch").int32).cpu().numpy()
        res, base, first = [], 0, 0
        for n in self.nbs:
            tri = n * (n + 1) // 2
            per_h = []
            for h in range(self.Hq):
                rows = []
                for i in range(n):
                    off = base + h * tri + i * (i + 1) // 2
                    rows.append(idx[off: off + int(counts[h, first + i])].astype(np.int32))
                per_h.append(rows)
            res.append(per_h)
            base += self.Hq * tri
            first += n
        return res
