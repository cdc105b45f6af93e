"""GPU tests of fp_check_index, the device check of the CSR index and the page
table that fp_sparse_prefill trusts.

The malformed indexes are built on the host from a valid one and handed to the
checker only (never to the attention kernel); the checker bounds every read
by the problem's sizes and the column capacity.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_common import upload

pytestmark = pytest.mark.gpu

import block_sparse_long_fp_amd as fp


def _valid_index():
    """A small ragged GQA-4 problem and the CSR its selection writes."""
    wl = synth.make_workload("llama_32k", L=5000, Hq=8, Hkv=2, B=128, n_planted=3)
    prob, q, k, v = upload(wl)
    bufs = fp.Buffers(prob, "cuda:0")
    fp.stage1(prob, fp.select_args(0.3), q, k, v, bufs.q_bar, bufs.k_bar, bufs.v_bar, bufs.row_ptr,
              bufs.col_idx, bufs.workspace)
    torch.cuda.synchronize()
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    ci = bufs.col_idx.cpu().numpy().astype(np.int64)
    return prob, bufs, rp, ci


def _check(prob, rp, ci, cap=None):
    dev = "cuda:0"
    cap = len(ci) if cap is None else cap
    row_ptr = torch.tensor(rp, dtype=torch.int32, device=dev)
    col_idx = torch.tensor(np.resize(ci, cap), dtype=torch.int32, device=dev)
    err = fp.check_index(prob, row_ptr, col_idx)
    torch.cuda.synchronize()
    return int(err.item())


def test_check_index_flags_each_kind_of_damage():
    prob, bufs, rp, ci = _valid_index()
    NBq = len(rp) - 1
    print(f"[check] rows={NBq} nnz={rp[-1]}", flush=True)
    assert _check(prob, rp, ci) == 0
    counts = np.diff(rp)
    # Rows in the problem's own numbering: row g is query block g % NBq_h of its KV head.
    nbq_h = NBq // 2
    def diag(g):
        return g % nbq_h  # one request: the row's own key block
    multi = [g for g in range(NBq) if counts[g] >= 2]
    assert multi, "need rows with at least two kept blocks"
    g = multi[len(multi) // 2]
    a = rp[g]

    swapped = ci.copy()
    swapped[a], swapped[a + 1] = swapped[a + 1], swapped[a]
    assert _check(prob, rp, swapped) & fp.FP_CHECK_ORDER

    out_of_range = ci.copy()
    out_of_range[a] = diag(g) + 1
    assert _check(prob, rp, out_of_range) & fp.FP_CHECK_RANGE

    # A row whose last column becomes I - 1 while staying ascending: only
    # the missing diagonal is wrong.
    no_diag = [h for h in multi if ci[rp[h + 1] - 2] < diag(h) - 1]
    assert no_diag, "need a row that does not keep its block I - 1"
    h = no_diag[len(no_diag) // 2]
    missing = ci.copy()
    missing[rp[h + 1] - 1] = diag(h) - 1
    assert _check(prob, rp, missing) == fp.FP_CHECK_DIAG

    empty = rp.copy()
    empty[g + 1] = empty[g]
    assert _check(prob, empty, ci) & fp.FP_CHECK_DIAG

    falling = rp.copy()
    falling[g + 1] = rp[g] - 1
    assert _check(prob, falling, ci) & fp.FP_CHECK_ROWPTR

    shifted = rp.copy()
    shifted[0] = 1
    assert _check(prob, shifted, ci) & fp.FP_CHECK_ROWPTR

    assert _check(prob, rp, ci, cap=int(rp[-1]) - 1) & fp.FP_CHECK_ROWPTR
    print("[check] ok", flush=True)


def test_check_index_of_a_paged_batch():
    """Page ids of a varlen paged batch: the valid table passes (with and
    without its CSR), one id at num_pages or below zero is flagged."""
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[700, 2900, 1500], Hq=8, Hkv=2, min_sparse_len=0,
                             page_size=16, n_planted=2)
    prob, q, k, v = upload(wl)
    bufs = fp.Buffers(prob, "cuda:0")
    fp.stage1(prob, fp.select_args(wl.alpha), q, k, v, bufs.q_bar, bufs.k_bar, bufs.v_bar, bufs.row_ptr,
              bufs.col_idx, bufs.workspace)
    err = fp.check_index(prob, bufs.row_ptr, bufs.col_idx)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert int(fp.check_index(prob).item()) == 0
    table = wl.page_table.clone()
    num_pages = k.shape[0]
    for bad in (num_pages, -1):
        t = table.clone()
        t[1, 3] = bad  # request 1 uses more than 3 pages of 16 tokens
        pb = fp.Problem(wl.cu_seqlens, wl.num_q_heads, wl.num_kv_heads, wl.block_size, wl.head_dim, fp.FP_BF16,
                        None, t.to("cuda:0"), wl.page_size, num_pages, wl.cu_seqlens_k)
        e = fp.check_index(pb)
        torch.cuda.synchronize()
        assert int(e.item()) == fp.FP_CHECK_PAGE, bad
    print("[check] paged ok", flush=True)
