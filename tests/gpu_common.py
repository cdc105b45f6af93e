"""Shared helpers of the GPU parity tests: upload a workload, run the HIP path
through the C ABI, run the oracle on the same bytes, and compare."""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
import torch

import block_sparse_long_fp_amd as fp
import oracle

O_TOL = {"bf16": 2e-2, "fp8": 6e-2}
LSE_REL = 1e-3


def upload(wl, device="cuda:0", paged: Optional[bool] = None):
    """Device tensors and the fp_problem of a workload."""
    paged = wl.paged if paged is None else paged
    q = wl.q.to(device)
    if paged:
        k, v = wl.k_pages.to(device), wl.v_pages.to(device)
        table = wl.page_table.to(device)
    else:
        k, v = wl.k.to(device), wl.v.to(device)
        table = None
    descales = None
    if wl.dtype == "fp8":
        descales = [torch.tensor([s], dtype=torch.float32, device=device)
                    for s in (wl.descale_q, wl.descale_k, wl.descale_v)]
    prob = fp.Problem(wl.cu_seqlens, wl.num_q_heads, wl.num_kv_heads, wl.block_size, wl.head_dim,
                      fp.FP_FP8_E4M3 if wl.dtype == "fp8" else fp.FP_BF16, descales, table,
                      wl.page_size if paged else 0, k.shape[0] if paged else 0, wl.cu_seqlens_k)
    return prob, q, k, v


def run_gpu(wl, alpha=None, mean_correction=True, paged=None, dense=False, min_sparse_len=None,
            device="cuda:0", forced=None, num_splits=0, fused_stage1=True, sm_scale=0.0):
    """Run pool -> select -> attention (or the dense kernel); return CPU results.
    ``forced``: dict(sink=, window=, last_n=) forced keeps, in blocks.
    ``num_splits``: split-KV parts (0 = the library's automatic choice).
    ``fused_stage1``: Stage 1 through fp_stage1 (else fp_pool_blocks and
    fp_select_blocks). ``sm_scale``: softmax scale (0 = 1 / sqrt(d))."""
    alpha = wl.alpha if alpha is None else alpha
    msl = wl.min_sparse_len if min_sparse_len is None else min_sparse_len
    prob, q, k, v = upload(wl, device, paged)
    att = fp.attn_args(sm_scale, mean_correction, num_splits)
    print(f"[gpu] splits={fp.attn_num_splits(prob, att)}", flush=True)
    bufs = fp.Buffers(prob, device, attn=att)
    if dense:
        fp.dense_prefill(prob, att, q, k, v, bufs.out, bufs.lse)
    else:
        fp.run_prefill(prob, bufs, q, k, v, alpha, wl.sel_scale, msl, sm_scale, mean_correction, **(forced or {}),
                       num_splits=num_splits, fused_stage1=fused_stage1)
    torch.cuda.synchronize()
    res = dict(out=bufs.out.float().cpu().numpy(), lse=bufs.lse.cpu().numpy())
    if not dense:
        nnz = int(bufs.row_ptr[-1].item())
        res.update(q_bar=bufs.q_bar.cpu().numpy(), k_bar=bufs.k_bar.cpu().numpy(), v_bar=bufs.v_bar.cpu().numpy(),
                   row_ptr=bufs.row_ptr.cpu().numpy().astype(np.int64),
                   col_idx=bufs.col_idx[:nnz].cpu().numpy().astype(np.int64))
    return res


def host_values(wl):
    """fp64 numpy Q, K, V (dequantised for FP8): exactly what the GPU reads."""
    def deq(t, s):
        x = t.to(torch.float64) if t.dtype != torch.float8_e4m3fn else t.to(torch.float32).to(torch.float64)
        return (x * s if s is not None else x).numpy()
    Q = deq(wl.q, wl.descale_q)
    K = deq(wl.k, wl.descale_k)
    V = deq(wl.v, wl.descale_v)
    return Q, K, V


def run_oracle(wl, alpha=None, mean_correction=True, do_attend=True, rows=None, paged=None,
               min_sparse_len=None, Qkv=None, forced=None):
    alpha = wl.alpha if alpha is None else alpha
    msl = wl.min_sparse_len if min_sparse_len is None else min_sparse_len
    Q, K, V = host_values(wl) if Qkv is None else Qkv
    paged = wl.paged if paged is None else paged
    kw = {}
    if paged:
        kp = wl.k_pages.to(torch.float32).to(torch.float64).numpy() * (wl.descale_k or 1.0)
        vp = wl.v_pages.to(torch.float32).to(torch.float64).numpy() * (wl.descale_v or 1.0)
        kw = dict(K_pages=kp, V_pages=vp, page_table=wl.page_table.numpy(), page_size=wl.page_size)
        K = V = None
    return oracle.prefill(Q, K, V, wl.cu_seqlens, wl.num_kv_heads, wl.block_size, alpha, wl.sel_scale, msl,
                          1.0 / math.sqrt(wl.head_dim), mean_correction, do_attend, rows, **kw, **(forced or {}),
                          cu_seqlens_k=wl.cu_seqlens_k)


def csr_rows(row_ptr, col_idx):
    return [col_idx[row_ptr[i]:row_ptr[i + 1]] for i in range(len(row_ptr) - 1)]


def compare_csr(gpu, orc):
    """Bit-exact CSR outside the near-threshold band; returns #rows touched by it."""
    near = {}
    for gr, J in orc.near:
        near.setdefault(gr, set()).add(J)
    g_rows = csr_rows(gpu["row_ptr"], gpu["col_idx"])
    o_rows = csr_rows(orc.row_ptr, orc.col_idx)
    assert len(g_rows) == len(o_rows)
    for i, (a, b) in enumerate(zip(g_rows, o_rows)):
        assert np.all(np.diff(a) > 0), f"row {i} not strictly ascending"
        if i in near:
            sa, sb = set(a.tolist()) - near[i], set(b.tolist()) - near[i]
            assert sa == sb, f"row {i}: {sorted(sa ^ sb)} differ outside the threshold band"
        else:
            assert np.array_equal(a, b), f"row {i}: gpu {a.tolist()} oracle {b.tolist()}"
    if not near:
        assert np.array_equal(gpu["row_ptr"], orc.row_ptr)
        assert np.array_equal(gpu["col_idx"], orc.col_idx)
    return len(near)


def sets_from_csr(row_ptr, col_idx, blk_off, Hkv):
    """Per request, per head, per query block selected-set lists from a CSR."""
    NBt = blk_off[-1]
    out = []
    for r in range(len(blk_off) - 1):
        per_h = []
        for h in range(Hkv):
            rows = []
            for I in range(blk_off[r + 1] - blk_off[r]):
                gr = h * NBt + blk_off[r] + I
                rows.append(col_idx[row_ptr[gr]:row_ptr[gr + 1]])
            per_h.append(rows)
        out.append(per_h)
    return out


def compare_pooled(gpu, orc, rtol=1e-5, atol=1e-5):
    for name in ("q_bar", "k_bar", "v_bar"):
        a, b = gpu[name], getattr(orc, name.replace("_", ""))
        assert a.shape == b.shape, name
        err = np.abs(a - b) - rtol * np.abs(b)
        assert err.max() <= atol, f"{name}: max err {err.max()}"


# The log-sum-exp bound is relative (fp32 LSE within 1e-3 of the oracle's,
# relative). An LSE within LSE_FLOOR of zero (the first keys of a request,
# whose single logit can be arbitrarily close to 0) has no meaningful
# relative error, so there the bound is taken against LSE_FLOOR: an
# absolute 1e-5.
LSE_FLOOR = 1e-2


def compare_outputs(gpu_out, gpu_lse, o_ref, lse_ref, tol, where: Optional[np.ndarray] = None):
    """Max-abs O error and relative LSE error over positions the oracle
    computed; returns (O max-abs, LSE relative, LSE absolute)."""
    mask = ~np.isnan(lse_ref)
    assert mask.any()
    do = np.abs(gpu_out - o_ref)
    do = do[~np.isnan(o_ref)]
    assert np.isfinite(gpu_out[~np.isnan(o_ref)]).all()
    o_err = float(do.max())
    dabs = np.abs(gpu_lse[mask] - lse_ref[mask])
    lse_rel = float((dabs / np.maximum(LSE_FLOOR, np.abs(lse_ref[mask]))).max())
    assert o_err <= tol, f"O max-abs error {o_err} > {tol}"
    assert lse_rel <= LSE_REL, f"LSE relative error {lse_rel} > {LSE_REL}"
    return o_err, lse_rel, float(dabs.max())


def rows_for_sample(wl, n_random=8, seed=0, row_ptr=None, near=None, n_near=8):
    """Global CSR rows to check at full size: the first, second, middle and
    last query block of the first and last KV head of every request; with
    ``row_ptr`` (the GPU's CSR) also each KV head's row with the most kept
    blocks; with ``near`` (the oracle's near-threshold pairs) up to
    ``n_near`` of the rows they touch; plus ``n_random`` random rows."""
    NBs = [-(-L // wl.block_size) for L in wl.seqlens]
    blk_off = np.concatenate([[0], np.cumsum(NBs)])
    NBt = int(blk_off[-1])
    rng = np.random.default_rng(seed)
    rows = set()
    for r, nb in enumerate(NBs):
        for h in (0, wl.num_kv_heads - 1):
            for I in (0, 1, nb // 2, nb - 1):
                rows.add(h * NBt + int(blk_off[r]) + I)
    if row_ptr is not None:
        counts = np.diff(np.asarray(row_ptr, dtype=np.int64))
        for h in range(wl.num_kv_heads):
            rows.add(h * NBt + int(np.argmax(counts[h * NBt:(h + 1) * NBt])))
    if near:
        touched = sorted({int(gr) for gr, _ in near})
        pick = rng.permutation(len(touched))[:n_near]
        rows.update(touched[i] for i in pick)
    for _ in range(n_random):
        rows.add(int(rng.integers(0, wl.num_kv_heads * NBt)))
    return sorted(rows)
