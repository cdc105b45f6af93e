"""fp_select_blocks_noalloc (the selection with its workspace in the
library's fixed per-GPU array, for callers that cannot allocate) against
fp_select_blocks with a caller workspace: the same CSR bit for bit, on two
calls in a row, the second with a smaller problem (fewer tiles than the
first left in the array)."""
import numpy as np
import pytest
import torch

import block_sparse_long_fp_amd as fp
import synth
from gpu_common import upload

pytestmark = pytest.mark.gpu


def _select(wl, noalloc: bool):
    prob, q, k, v = upload(wl)
    bufs = fp.Buffers(prob, "cuda:0")
    fp.pool_blocks(prob, q, k, v, bufs.q_bar, bufs.k_bar, bufs.v_bar)
    sel = fp.select_args(wl.alpha, wl.sel_scale, wl.min_sparse_len, 1, 1, 0)
    bufs.row_ptr.fill_(-3)
    bufs.col_idx.fill_(-3)
    if noalloc:
        fp.select_blocks_noalloc(prob, sel, bufs.q_bar, bufs.k_bar, bufs.row_ptr, bufs.col_idx)
    else:
        fp.select_blocks(prob, sel, bufs.q_bar, bufs.k_bar, bufs.row_ptr, bufs.col_idx, bufs.workspace)
    torch.cuda.synchronize()
    rp = bufs.row_ptr.cpu().numpy()
    return rp, bufs.col_idx[: int(rp[-1])].cpu().numpy()


def test_noalloc_selection_equals_the_workspace_call():
    # 4384 CSR rows (tiles of 16 query blocks, 280 tiles), then 60 rows (tiles of 4)
    big = synth.make_workload("llama_32k", lengths=[40000, 30000], Hq=8, Hkv=8, n_planted=8, kind="varlen",
                              seeds_base=40, page_size=0, min_sparse_len=0)
    small = synth.make_workload("llama_32k", lengths=[2100, 1700], Hq=8, Hkv=2, n_planted=3, kind="varlen",
                                seeds_base=50, page_size=0, min_sparse_len=0)
    for wl in (big, small):
        print(f"[no-alloc] lengths={wl.seqlens} Hkv={wl.num_kv_heads}", flush=True)
        a_rp, a_ci = _select(wl, True)
        b_rp, b_ci = _select(wl, False)
        assert np.array_equal(a_rp, b_rp)
        assert np.array_equal(a_ci, b_ci)
        assert a_rp[-1] > len(a_rp) - 1  # more than the diagonals: real selections
