"""Python binding of libfpv2.so: mean-corrected block-sparse causal prefill on MI355X.

Argument marshalling only: every step of the computation runs in the library's
HIP kernels. PyTorch supplies device memory and the current HIP stream. If the
library has not been built, importing the compute functions raises at call
time with a message that says so; there is no fallback path.

Entry points mirror the C ABI in include/fpv2.h:
  pool_blocks, pool_chunk_blocks, select_blocks, stage1, sparse_prefill, dense_prefill
plus the convenience ``prefill`` that allocates outputs and runs all three
stages, and the host-only ``index_shape`` / ``select_workspace_bytes`` /
``attn_workspace_bytes`` / ``validate``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfpv2.so")

FP_BF16, FP_FP8_E4M3 = 0, 1
FP_KV_CONTIGUOUS, FP_KV_PAGED = 0, 1
FP_MAX_SEQS = 128
FP_MAX_BLOCKS_PER_SEQ = 16384

STATUS_NAMES = {
    0: "FP_OK", 1: "FP_ERR_NULL", 2: "FP_ERR_SHAPE", 3: "FP_ERR_GQA", 4: "FP_ERR_BLOCK", 5: "FP_ERR_DTYPE",
    6: "FP_ERR_LAYOUT", 7: "FP_ERR_CAPACITY", 8: "FP_ERR_WORKSPACE", 9: "FP_ERR_ARG", 10: "FP_ERR_UNSUPPORTED",
    11: "FP_ERR_HIP",
}


class FpError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


class _Problem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("cu_seqlens", ctypes.POINTER(ctypes.c_int32)),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("descale_q", ctypes.c_void_p),
        ("descale_k", ctypes.c_void_p),
        ("descale_v", ctypes.c_void_p),
        ("kv_layout", ctypes.c_int32),
        ("page_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("cu_seqlens_k", ctypes.POINTER(ctypes.c_int32)),
        ("pooled_pitch", ctypes.c_int32),
        ("pooled_row_off", ctypes.POINTER(ctypes.c_int32)),
    ]


class _SelectArgs(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_float), ("sel_scale", ctypes.c_float), ("min_sparse_len", ctypes.c_int32),
                ("sink_blocks", ctypes.c_int32), ("window_blocks", ctypes.c_int32),
                ("last_n_blocks", ctypes.c_int32)]


class _AttnArgs(ctypes.Structure):
    _fields_ = [("sm_scale", ctypes.c_float), ("mean_correction", ctypes.c_int32), ("num_splits", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfpv2.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_long_fp_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(_Problem)
        vp, i64p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)
        L.fp_index_shape.argtypes = [P, i64p, i64p, i64p, i64p]
        L.fp_select_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        L.fp_validate.argtypes = [P, ctypes.POINTER(_SelectArgs), ctypes.POINTER(_AttnArgs)]
        L.fp_pool_blocks.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.fp_pool_chunk_blocks.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.fp_select_blocks.argtypes = [P, ctypes.POINTER(_SelectArgs), vp, vp, vp, vp, ctypes.c_int64, vp,
                                       ctypes.c_size_t, vp]
        L.fp_select_blocks_noalloc.argtypes = [P, ctypes.POINTER(_SelectArgs), vp, vp, vp, vp, ctypes.c_int64, vp]
        L.fp_stage1.argtypes = [P, ctypes.POINTER(_SelectArgs), ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp,
                                ctypes.c_int64, vp, ctypes.c_size_t, vp]
        L.fp_attn_workspace_bytes.argtypes = [P, ctypes.POINTER(_AttnArgs), ctypes.c_int32,
                                              ctypes.POINTER(ctypes.c_size_t)]
        L.fp_attn_num_splits.argtypes = [P, ctypes.POINTER(_AttnArgs), ctypes.POINTER(ctypes.c_int32)]
        L.fp_sparse_prefill.argtypes = [P, ctypes.POINTER(_AttnArgs), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        ctypes.c_size_t, vp]
        L.fp_dense_prefill.argtypes = [P, ctypes.POINTER(_AttnArgs), vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.fp_check_index.argtypes = [P, vp, vp, ctypes.c_int64, vp, vp]
        L.fp_workspace_bytes.argtypes = [P, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        for f in ("fp_index_shape", "fp_select_workspace_bytes", "fp_attn_workspace_bytes", "fp_attn_num_splits",
                  "fp_validate",
                  "fp_pool_blocks", "fp_pool_chunk_blocks", "fp_select_blocks", "fp_select_blocks_noalloc", "fp_stage1",
                  "fp_sparse_prefill",
                  "fp_dense_prefill", "fp_check_index", "fp_workspace_bytes"):
            getattr(L, f).restype = ctypes.c_int32
        L.fp_status_string.argtypes = [ctypes.c_int32]
        L.fp_status_string.restype = ctypes.c_char_p
        L.fp_last_error.argtypes = []
        L.fp_last_error.restype = ctypes.c_char_p
        L.fp_abi_version.argtypes = []
        L.fp_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def _check(code: int):
    if code != 0:
        raise FpError(code, lib().fp_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# --------------------------------------------------------------------------
# Argument checks of the binding. The C ABI takes raw pointers, so it cannot
# see a tensor's dtype, device, strides or size; these checks run before any
# library call and raise FpError with the status code the C side uses for
# the same class of mistake. Every operand is checked for dtype, shape and
# contiguity first, then all of them for being on one GPU.
# --------------------------------------------------------------------------

FP_ERR_NULL, FP_ERR_SHAPE, FP_ERR_DTYPE, FP_ERR_LAYOUT, FP_ERR_CAPACITY, FP_ERR_WORKSPACE = 1, 2, 5, 6, 7, 8
_ELEM = {FP_BF16: torch.bfloat16, FP_FP8_E4M3: torch.float8_e4m3fn}


def _tensor(t, name: str, dtype, shape=None, min_rows=None, flat_min: Optional[int] = None,
            shape_code: int = FP_ERR_SHAPE):
    """Raise FpError unless ``t`` is a contiguous tensor of ``dtype`` and of
    ``shape`` (a tuple; with ``min_rows`` the first dim may be larger), or
    with ``flat_min`` 1-D with at least that many elements."""
    if t is None:
        raise FpError(FP_ERR_NULL, f"{name} is None")
    if not isinstance(t, torch.Tensor):
        raise FpError(FP_ERR_LAYOUT, f"{name} is a {type(t).__name__}, not a torch.Tensor")
    if t.dtype != dtype:
        raise FpError(FP_ERR_DTYPE, f"{name} has dtype {t.dtype}, expected {dtype}")
    got = tuple(t.shape)
    if flat_min is not None:
        if t.dim() != 1 or t.numel() < flat_min:
            raise FpError(shape_code, f"{name} has shape {got}, expected 1-D with >= {flat_min} elements")
    elif shape is not None:
        if min_rows is not None:
            ok = len(got) == len(shape) and got[0] >= min_rows and got[1:] == tuple(shape[1:])
        else:
            ok = got == tuple(shape)
        if not ok:
            want = ("(>= %d, %s)" % (min_rows, ", ".join(map(str, shape[1:])))) if min_rows is not None else shape
            raise FpError(shape_code, f"{name} has shape {got}, expected {want}")
    if not t.is_contiguous():
        raise FpError(FP_ERR_LAYOUT, f"{name} is not contiguous (strides {tuple(t.stride())})")
    return t


def _one_gpu(named):
    """All tensors of ``named`` (name -> tensor or None) on one GPU; returns it."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise FpError(FP_ERR_LAYOUT, f"{name} is on {t.device}, not on a GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise FpError(FP_ERR_LAYOUT, f"{name} is on {t.device}, the other operands on {dev}")
    return dev


def _qkv_checks(prob: "Problem", q, k, v):
    """Q [Tq, Hq, d]; K, V [Tk, Hkv, d] or page pools [pages, page_size, Hkv, d];
    all of the problem's element type; FP8 descales and the page table.
    Returns the (name, tensor) pairs checked."""
    s = prob.s
    d = s.head_dim
    el = _ELEM.get(s.dtype)
    if el is None:
        raise FpError(FP_ERR_DTYPE, f"unknown dtype code {s.dtype}")
    # Inputs may hold more leading rows than the call reads (a buffer sized for
    # a whole prompt, a page pool with spare pages); the kernels read rows
    # below Tq / Tk / num_pages only.
    if s.kv_layout == FP_KV_PAGED:
        kv_shape = (s.num_pages, s.page_size, s.num_kv_heads, d)
    else:
        kv_shape = (prob.Tk, s.num_kv_heads, d)
    named = [("q", _tensor(q, "q", el, (prob.Tq, s.num_q_heads, d), min_rows=prob.Tq)),
             ("k", _tensor(k, "k", el, kv_shape, min_rows=kv_shape[0])),
             ("v", _tensor(v, "v", el, kv_shape, min_rows=kv_shape[0]))]
    if s.dtype == FP_FP8_E4M3:
        if prob.descales is None:
            raise FpError(FP_ERR_DTYPE, "FP8 inputs need descale_q, descale_k and descale_v")
        for name, t in zip(("descale_q", "descale_k", "descale_v"), prob.descales):
            named.append((name, _tensor(t, name, torch.float32, (1,))))
    if s.kv_layout == FP_KV_PAGED:
        named.append(("page_table", _tensor(prob.page_table, "page_table", torch.int32,
                                            (prob.num_seqs, s.max_pages_per_seq), min_rows=prob.num_seqs)))
    return named


def _pooled_checks(prob: "Problem", q_bar=None, k_bar=None, v_bar=None):
    """Returns (CSR rows, checked pairs)."""
    rows, nnz, nbq, nbk = index_shape(prob)
    pitch = prob.s.pooled_pitch or nbk
    Hkv, d = prob.s.num_kv_heads, prob.s.head_dim
    named = []
    if q_bar is not None:
        named.append(("q_bar", _tensor(q_bar, "q_bar", torch.float32, (Hkv, nbq, d))))
    for name, t in (("k_bar", k_bar), ("v_bar", v_bar)):
        if t is not None:
            named.append((name, _tensor(t, name, torch.float32, (Hkv, pitch, d))))
    return rows, named


def _out_checks(prob: "Problem", out, lse):
    s = prob.s
    named = [("out", _tensor(out, "out", torch.bfloat16, (prob.Tq, s.num_q_heads, s.head_dim)))]
    if lse is not None:
        named.append(("lse", _tensor(lse, "lse", torch.float32, (s.num_q_heads, prob.Tq))))
    return named


def _workspace_check(ws, name="workspace"):
    return [(name, _tensor(ws, name, torch.uint8, flat_min=1, shape_code=FP_ERR_WORKSPACE))]


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Problem:
    """Holds an fp_problem and keeps its host arrays alive.

    ``cu_seqlens`` are the query offsets; ``cu_seqlens_k`` (None: the same) the
    key offsets. In chunked prefill request r's queries are the last
    Lq_r = cu_seqlens[r+1] - cu_seqlens[r] of its Lk_r keys. ``pooled_pitch``:
    rows per KV head of k_bar / v_bar (0: the problem's key-block count)."""

    def __init__(self, cu_seqlens: Sequence[int], num_q_heads: int, num_kv_heads: int, block_size: int,
                 head_dim: int = 128, dtype: int = FP_BF16, descales: Optional[Sequence[torch.Tensor]] = None,
                 page_table: Optional[torch.Tensor] = None, page_size: int = 0, num_pages: int = 0,
                 cu_seqlens_k: Optional[Sequence[int]] = None, pooled_pitch: int = 0,
                 pooled_row_off: Optional[Sequence[int]] = None):
        cu = [int(x) for x in cu_seqlens]
        self.cu_seqlens = cu
        self.cu_seqlens_k = cu if cu_seqlens_k is None else [int(x) for x in cu_seqlens_k]
        self._cu = (ctypes.c_int32 * len(cu))(*cu)
        self._keep = []
        s = _Problem()
        s.num_seqs = len(cu) - 1
        s.cu_seqlens = ctypes.cast(self._cu, ctypes.POINTER(ctypes.c_int32))
        if cu_seqlens_k is not None:
            self._cuk = (ctypes.c_int32 * len(self.cu_seqlens_k))(*self.cu_seqlens_k)
            s.cu_seqlens_k = ctypes.cast(self._cuk, ctypes.POINTER(ctypes.c_int32))
        s.pooled_pitch = pooled_pitch
        if pooled_row_off is not None:
            self._prow = (ctypes.c_int32 * len(pooled_row_off))(*[int(x) for x in pooled_row_off])
            s.pooled_row_off = ctypes.cast(self._prow, ctypes.POINTER(ctypes.c_int32))
        self.descales = list(descales) if descales is not None else None
        self.page_table = page_table
        s.num_q_heads, s.num_kv_heads, s.head_dim, s.block_size = num_q_heads, num_kv_heads, head_dim, block_size
        s.dtype = dtype
        if descales is not None:
            self._keep.extend(descales)
            s.descale_q, s.descale_k, s.descale_v = (t.data_ptr() for t in descales)
        if page_table is not None:
            self._keep.append(page_table)
            s.kv_layout = FP_KV_PAGED
            s.page_table = page_table.data_ptr()
            s.page_size = page_size
            s.max_pages_per_seq = page_table.shape[1]
            s.num_pages = num_pages
        else:
            s.kv_layout = FP_KV_CONTIGUOUS
        self.s = s

    @property
    def ref(self):
        return ctypes.byref(self.s)

    @property
    def num_seqs(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def Tq(self) -> int:
        return self.cu_seqlens[-1]

    @property
    def Tk(self) -> int:
        return self.cu_seqlens_k[-1]


def index_shape(prob: Problem):
    """(CSR rows, worst-case nnz, query blocks NBq_tot, key blocks NBk_tot)."""
    rows, nnz, nbq, nbk = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().fp_index_shape(prob.ref, ctypes.byref(rows), ctypes.byref(nnz), ctypes.byref(nbq),
                                ctypes.byref(nbk)))
    return rows.value, nnz.value, nbq.value, nbk.value


def select_workspace_bytes(prob: Problem) -> int:
    n = ctypes.c_size_t()
    _check(lib().fp_select_workspace_bytes(prob.ref, ctypes.byref(n)))
    return n.value


def attn_workspace_bytes(prob: Problem, sparse: bool = True, attn: Optional["_AttnArgs"] = None) -> int:
    """Attention workspace bytes for these args (None: defaults, automatic split)."""
    n = ctypes.c_size_t()
    _check(lib().fp_attn_workspace_bytes(prob.ref, ctypes.byref(attn) if attn is not None else None,
                                         1 if sparse else 0, ctypes.byref(n)))
    return n.value


FP_CALL_SELECT, FP_CALL_SPARSE, FP_CALL_DENSE = 0, 1, 2


def workspace_bytes(prob: Problem, which_call: int) -> int:
    """fp_workspace_bytes: the workspace of FP_CALL_SELECT, FP_CALL_SPARSE or
    FP_CALL_DENSE (attention with the default arguments)."""
    n = ctypes.c_size_t()
    _check(lib().fp_workspace_bytes(prob.ref, which_call, ctypes.byref(n)))
    return n.value


def attn_num_splits(prob: Problem, attn: Optional["_AttnArgs"] = None) -> int:
    """The split-KV part count the attention calls use for these args."""
    n = ctypes.c_int32()
    _check(lib().fp_attn_num_splits(prob.ref, ctypes.byref(attn) if attn is not None else None, ctypes.byref(n)))
    return n.value


def _attn_workspace(prob: Problem, sparse: bool, workspace, device, attn=None):
    """The caller's workspace, or a fresh torch allocation of the needed size."""
    if workspace is None:
        n = attn_workspace_bytes(prob, sparse, attn)
        if n > 0:
            workspace = torch.empty(n, dtype=torch.uint8, device=device)
    return workspace


def select_args(alpha: float, sel_scale: float = 1.0, min_sparse_len: int = 0, sink: int = 0, window: int = 0,
                last_n: int = 0) -> _SelectArgs:
    """fp_select_args; sink / window / last_n are the forced keeps, in blocks."""
    return _SelectArgs(alpha, sel_scale, min_sparse_len, sink, window, last_n)


def attn_args(sm_scale: float = 0.0, mean_correction: bool = True, num_splits: int = 0) -> _AttnArgs:
    """fp_attn_args; num_splits 0 = automatic split-KV, 1 = none, k = k parts."""
    return _AttnArgs(sm_scale, 1 if mean_correction else 0, num_splits)


def validate(prob: Problem, sel: Optional[_SelectArgs] = None, attn: Optional[_AttnArgs] = None):
    _check(lib().fp_validate(prob.ref, ctypes.byref(sel) if sel is not None else None,
                             ctypes.byref(attn) if attn is not None else None))


def pool_blocks(prob: Problem, q, k, v, q_bar, k_bar, v_bar, stream=None):
    _one_gpu(_qkv_checks(prob, q, k, v) + _pooled_checks(prob, q_bar, k_bar, v_bar)[1])
    _check(lib().fp_pool_blocks(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(q_bar), _ptr(k_bar), _ptr(v_bar),
                                _stream(stream)))


def pool_chunk_blocks(prob: Problem, q, k, v, q_bar, k_bar, v_bar, stream=None):
    """fp_pool_chunk_blocks: pools q_bar and only the key blocks the chunk
    adds; k_bar / v_bar rows of earlier blocks must hold earlier calls' values."""
    _one_gpu(_qkv_checks(prob, q, k, v) + _pooled_checks(prob, q_bar, k_bar, v_bar)[1])
    _check(lib().fp_pool_chunk_blocks(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(q_bar), _ptr(k_bar),
                                      _ptr(v_bar), _stream(stream)))


def select_blocks(prob: Problem, sel: _SelectArgs, q_bar, k_bar, row_ptr, col_idx, workspace, stream=None):
    rows, named = _pooled_checks(prob, q_bar, k_bar)
    if q_bar is None or k_bar is None:
        raise FpError(FP_ERR_NULL, "q_bar and k_bar are required")
    named += [("row_ptr", _tensor(row_ptr, "row_ptr", torch.int32, (rows + 1,))),
              ("col_idx", _tensor(col_idx, "col_idx", torch.int32, flat_min=1))]
    _one_gpu(named + _workspace_check(workspace))
    _check(lib().fp_select_blocks(prob.ref, ctypes.byref(sel), _ptr(q_bar), _ptr(k_bar), _ptr(row_ptr),
                                  _ptr(col_idx), col_idx.numel(), _ptr(workspace), workspace.numel(),
                                  _stream(stream)))


def select_blocks_noalloc(prob: Problem, sel: _SelectArgs, q_bar, k_bar, row_ptr, col_idx, stream=None):
    """fp_select_blocks_noalloc: select_blocks with the workspace in the
    library's fixed per-GPU array (no allocation; calls on one GPU must not
    overlap)."""
    rows, named = _pooled_checks(prob, q_bar, k_bar)
    if q_bar is None or k_bar is None:
        raise FpError(FP_ERR_NULL, "q_bar and k_bar are required")
    named += [("row_ptr", _tensor(row_ptr, "row_ptr", torch.int32, (rows + 1,))),
              ("col_idx", _tensor(col_idx, "col_idx", torch.int32, flat_min=1))]
    _one_gpu(named)
    _check(lib().fp_select_blocks_noalloc(prob.ref, ctypes.byref(sel), _ptr(q_bar), _ptr(k_bar), _ptr(row_ptr),
                                          _ptr(col_idx), col_idx.numel(), _stream(stream)))


def stage1(prob: Problem, sel: _SelectArgs, q, k, v, q_bar, k_bar, v_bar, row_ptr, col_idx, workspace,
           chunk_only: bool = False, stream=None):
    """fp_stage1: pooling (all key blocks, or with ``chunk_only`` only the ones
    the chunk adds) and selection in two kernels."""
    rows, named = _pooled_checks(prob, q_bar, k_bar, v_bar)
    named += _qkv_checks(prob, q, k, v)
    named += [("row_ptr", _tensor(row_ptr, "row_ptr", torch.int32, (rows + 1,))),
              ("col_idx", _tensor(col_idx, "col_idx", torch.int32, flat_min=1))]
    _one_gpu(named + _workspace_check(workspace))
    _check(lib().fp_stage1(prob.ref, ctypes.byref(sel), 1 if chunk_only else 0, _ptr(q), _ptr(k), _ptr(v),
                           _ptr(q_bar), _ptr(k_bar), _ptr(v_bar), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                           _ptr(workspace), workspace.numel(), _stream(stream)))


def sparse_prefill(prob: Problem, attn: _AttnArgs, q, k, v, k_bar, v_bar, row_ptr, col_idx, out, lse=None,
                   workspace=None, stream=None):
    """fp_sparse_prefill; ``workspace`` (uint8 device tensor of at least
    attn_workspace_bytes(prob, True) bytes) is allocated here when None."""
    named = _qkv_checks(prob, q, k, v)
    rows, pooled = _pooled_checks(prob, None, k_bar, v_bar)
    if attn.mean_correction and (k_bar is None or v_bar is None):
        raise FpError(FP_ERR_NULL, "mean correction needs k_bar and v_bar")
    named += pooled + [("row_ptr", _tensor(row_ptr, "row_ptr", torch.int32, (rows + 1,))),
                       ("col_idx", _tensor(col_idx, "col_idx", torch.int32, flat_min=1))]
    named += _out_checks(prob, out, lse)
    if workspace is not None:
        named += _workspace_check(workspace)
    _one_gpu(named)
    workspace = _attn_workspace(prob, True, workspace, out.device, attn)
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib().fp_sparse_prefill(prob.ref, ctypes.byref(attn), _ptr(q), _ptr(k), _ptr(v), _ptr(k_bar),
                                   _ptr(v_bar), _ptr(row_ptr), _ptr(col_idx), _ptr(out), _ptr(lse),
                                   _ptr(workspace), nbytes, _stream(stream)))


def dense_prefill(prob: Problem, attn: _AttnArgs, q, k, v, out, lse=None, workspace=None, stream=None):
    """fp_dense_prefill; ``workspace`` as in sparse_prefill (only FP8 needs one)."""
    named = _qkv_checks(prob, q, k, v) + _out_checks(prob, out, lse)
    if workspace is not None:
        named += _workspace_check(workspace)
    _one_gpu(named)
    workspace = _attn_workspace(prob, False, workspace, out.device, attn)
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib().fp_dense_prefill(prob.ref, ctypes.byref(attn), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                  _ptr(workspace), nbytes, _stream(stream)))


FP_CHECK_ROWPTR, FP_CHECK_ORDER, FP_CHECK_RANGE, FP_CHECK_DIAG, FP_CHECK_PAGE = 1, 2, 4, 8, 16


def check_index(prob: Problem, row_ptr=None, col_idx=None, err=None, stream=None):
    """fp_check_index: device check of a CSR index (and, for paged K / V, the
    page table) before fp_sparse_prefill, which trusts both. Returns ``err``
    (an int32 device tensor of one element, allocated here if None), which
    holds the OR of the FP_CHECK_* bits found once the stream reaches it."""
    named = []
    if (row_ptr is None) != (col_idx is None):
        raise FpError(FP_ERR_NULL, "give both row_ptr and col_idx, or neither")
    if row_ptr is not None:
        rows, nnz, nbq, nbk = index_shape(prob)
        named += [("row_ptr", _tensor(row_ptr, "row_ptr", torch.int32, (rows + 1,))),
                  ("col_idx", _tensor(col_idx, "col_idx", torch.int32, flat_min=1))]
    if prob.s.kv_layout == FP_KV_PAGED:
        named.append(("page_table", _tensor(prob.page_table, "page_table", torch.int32,
                                            (prob.num_seqs, prob.s.max_pages_per_seq), min_rows=prob.num_seqs)))
    if err is None:
        dev = _one_gpu(named)
        if dev is None:
            raise FpError(FP_ERR_NULL, "nothing to check on a GPU (no CSR, and K / V are not paged)")
        err = torch.empty(1, dtype=torch.int32, device=dev)
    named.append(("err", _tensor(err, "err", torch.int32, flat_min=1)))
    _one_gpu(named)
    cap = 0 if col_idx is None else col_idx.numel()
    _check(lib().fp_check_index(prob.ref, _ptr(row_ptr), _ptr(col_idx), cap, _ptr(err), _stream(stream)))
    return err


class Buffers:
    """Device buffers of one prefill problem (allocated with torch)."""

    def __init__(self, prob: Problem, device, head_dim: int = 128, attn: Optional[_AttnArgs] = None):
        rows, nnz, nbq, nbk = index_shape(prob)
        Hkv = prob.s.num_kv_heads
        T = prob.cu_seqlens[-1]
        Hq = prob.s.num_q_heads
        f32 = dict(dtype=torch.float32, device=device)
        kp = prob.s.pooled_pitch or nbk
        self.q_bar = torch.empty((Hkv, nbq, head_dim), **f32)
        self.k_bar = torch.empty((Hkv, kp, head_dim), **f32)
        self.v_bar = torch.empty((Hkv, kp, head_dim), **f32)
        self.row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=device)
        self.col_idx = torch.empty(max(nnz, 1), dtype=torch.int32, device=device)
        self.workspace = torch.empty(select_workspace_bytes(prob), dtype=torch.uint8, device=device)
        self.attn_workspace = torch.empty(max(attn_workspace_bytes(prob, True, attn), 1), dtype=torch.uint8,
                                          device=device)
        self.out = torch.empty((T, Hq, head_dim), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((Hq, T), **f32)


def run_prefill(prob: Problem, bufs: Buffers, q, k, v, alpha: float, sel_scale: float = 1.0,
                min_sparse_len: int = 0, sm_scale: float = 0.0, mean_correction: bool = True, stream=None,
                sink: int = 0, window: int = 0, last_n: int = 0, num_splits: int = 0, fused_stage1: bool = True):
    """All three stages on preallocated buffers (nothing allocated here; the
    buffers must have been sized with the same num_splits). Stage 1 runs as
    fp_stage1 (two kernels), or with ``fused_stage1=False`` as the separate
    fp_pool_blocks and fp_select_blocks calls."""
    sel = select_args(alpha, sel_scale, min_sparse_len, sink, window, last_n)
    if fused_stage1:
        stage1(prob, sel, q, k, v, bufs.q_bar, bufs.k_bar, bufs.v_bar, bufs.row_ptr, bufs.col_idx, bufs.workspace,
               stream=stream)
    else:
        pool_blocks(prob, q, k, v, bufs.q_bar, bufs.k_bar, bufs.v_bar, stream)
        select_blocks(prob, sel, bufs.q_bar, bufs.k_bar, bufs.row_ptr, bufs.col_idx, bufs.workspace, stream)
    sparse_prefill(prob, attn_args(sm_scale, mean_correction, num_splits), q, k, v, bufs.k_bar, bufs.v_bar,
                   bufs.row_ptr, bufs.col_idx, bufs.out, bufs.lse, bufs.attn_workspace, stream)
    return bufs


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: Sequence[int], block_size: int,
            alpha: float, sel_scale: float = 1.0, min_sparse_len: int = 0, sm_scale: float = 0.0,
            mean_correction: bool = True, descales: Optional[Sequence[torch.Tensor]] = None,
            page_table: Optional[torch.Tensor] = None, page_size: int = 0, sink: int = 0, window: int = 0,
            last_n: int = 0, cu_seqlens_k: Optional[Sequence[int]] = None):
    """Mean-corrected block-sparse causal prefill of a ragged batch.

    q [Tq, Hq, 128]; k, v [Tk, Hkv, 128] (contiguous) or page pools
    [num_pages, page_size, Hkv, 128] with ``page_table`` [R, max_pages]
    (int32, device). bf16, or float8_e4m3fn with ``descales`` = three
    one-element fp32 device tensors. ``sink`` / ``window`` / ``last_n`` are
    the forced keeps, in blocks. ``cu_seqlens_k`` (chunked prefill): key
    offsets; each request's queries are its last positions. Returns a
    ``Buffers`` with out, lse, row_ptr, col_idx and the pooled statistics.
    """
    Hq = q.shape[1]
    Hkv = k.shape[-2]
    if q.dtype == torch.bfloat16:
        dtype = FP_BF16
    elif q.dtype == torch.float8_e4m3fn:
        dtype = FP_FP8_E4M3
    else:
        raise FpError(FP_ERR_DTYPE, f"q has dtype {q.dtype}; the kernels take bfloat16 or float8_e4m3fn")
    prob = Problem(cu_seqlens, Hq, Hkv, block_size, q.shape[-1], dtype, descales, page_table, page_size,
                   k.shape[0] if page_table is not None else 0, cu_seqlens_k)
    bufs = Buffers(prob, q.device, q.shape[-1])
    return run_prefill(prob, bufs, q, k, v, alpha, sel_scale, min_sparse_len, sm_scale, mean_correction,
                       sink=sink, window=window, last_n=last_n)
