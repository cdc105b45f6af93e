"""The Python binding's argument checks, on the CPU.

The C ABI takes raw pointers, so the binding checks every tensor before a
library call: dtype (FP_ERR_DTYPE), shape against the problem (FP_ERR_SHAPE),
contiguity and device (FP_ERR_LAYOUT), workspace type (FP_ERR_WORKSPACE). The
checks run in that order, so CPU tensors reach each of them: a CPU tensor that
is right in every other respect is rejected for its device. No kernel is
launched here.
"""
import os

import pytest
import torch

import block_sparse_long_fp_amd as fp

pytestmark = pytest.mark.skipif(not os.path.exists(fp.LIB_PATH), reason="libfpv2.so not built")

T, HQ, HKV, D, B = 300, 8, 2, 128, 64
NB = -(-T // B)


def _prob(**kw):
    base = dict(cu_seqlens=[0, T], num_q_heads=HQ, num_kv_heads=HKV, block_size=B)
    base.update(kw)
    return fp.Problem(**base)


def _qkv(dtype=torch.bfloat16):
    return (torch.zeros(T, HQ, D, dtype=dtype), torch.zeros(T, HKV, D, dtype=dtype),
            torch.zeros(T, HKV, D, dtype=dtype))


def _pooled():
    return (torch.zeros(HKV, NB, D), torch.zeros(HKV, NB, D), torch.zeros(HKV, NB, D))


def _code(fn, *a, **kw):
    with pytest.raises(fp.FpError) as e:
        fn(*a, **kw)
    return e.value.code, str(e.value)


def test_pool_blocks_checks_in_order():
    p = _prob()
    q, k, v = _qkv()
    qb, kb, vb = _pooled()
    # dtype: fp16 / fp32 inputs are not read as bf16
    assert _code(fp.pool_blocks, p, q.half(), k, v, qb, kb, vb)[0] == fp.FP_ERR_DTYPE
    assert _code(fp.pool_blocks, p, q, k.float(), v, qb, kb, vb)[0] == fp.FP_ERR_DTYPE
    assert _code(fp.pool_blocks, p, q, k, v, qb.double(), kb, vb)[0] == fp.FP_ERR_DTYPE
    # shape against the problem
    assert _code(fp.pool_blocks, p, q[:-1], k, v, qb, kb, vb)[0] == fp.FP_ERR_SHAPE
    assert _code(fp.pool_blocks, p, q, k[:, :1], v, qb, kb, vb)[0] == fp.FP_ERR_SHAPE
    assert _code(fp.pool_blocks, p, q, k, v, qb[:, :-1], kb, vb)[0] == fp.FP_ERR_SHAPE
    assert _code(fp.pool_blocks, p, q, k, v, qb, kb, vb[:1])[0] == fp.FP_ERR_SHAPE
    # contiguity: a transposed view of the right shape
    qt = torch.zeros(HQ, T, D, dtype=torch.bfloat16).transpose(0, 1)
    assert qt.shape == q.shape
    assert _code(fp.pool_blocks, p, qt, k, v, qb, kb, vb)[0] == fp.FP_ERR_LAYOUT
    # device: everything right but on the CPU
    code, msg = _code(fp.pool_blocks, p, q, k, v, qb, kb, vb)
    assert code == fp.FP_ERR_LAYOUT and "not on a GPU" in msg
    assert _code(fp.pool_blocks, p, None, k, v, qb, kb, vb)[0] == fp.FP_ERR_NULL
    assert _code(fp.pool_blocks, p, [1, 2], k, v, qb, kb, vb)[0] == fp.FP_ERR_LAYOUT


def test_fp8_inputs_need_fp8_tensors_and_descales():
    ds = [torch.ones(1) for _ in range(3)]
    p = _prob(dtype=fp.FP_FP8_E4M3, descales=ds)
    q8, k8, v8 = _qkv(torch.float8_e4m3fn)
    qb, kb, vb = _pooled()
    q, k, v = _qkv()
    assert _code(fp.pool_blocks, p, q, k, v, qb, kb, vb)[0] == fp.FP_ERR_DTYPE       # bf16 for an FP8 problem
    assert _code(fp.pool_blocks, _prob(), q8, k8, v8, qb, kb, vb)[0] == fp.FP_ERR_DTYPE
    bad = fp.Problem([0, T], HQ, HKV, B, dtype=fp.FP_FP8_E4M3, descales=[torch.ones(1, dtype=torch.float64)] * 3)
    assert _code(fp.pool_blocks, bad, q8, k8, v8, qb, kb, vb)[0] == fp.FP_ERR_DTYPE
    two = fp.Problem([0, T], HQ, HKV, B, dtype=fp.FP_FP8_E4M3, descales=[torch.ones(2)] * 3)
    assert _code(fp.pool_blocks, two, q8, k8, v8, qb, kb, vb)[0] == fp.FP_ERR_SHAPE
    # right in every respect but the device
    assert _code(fp.pool_blocks, p, q8, k8, v8, qb, kb, vb)[0] == fp.FP_ERR_LAYOUT


def test_prefill_rejects_other_dtypes():
    q, k, v = (t.float() for t in _qkv())
    assert _code(fp.prefill, q, k, v, [0, T], B, 0.3)[0] == fp.FP_ERR_DTYPE
    assert _code(fp.prefill, q.half(), k.half(), v.half(), [0, T], B, 0.3)[0] == fp.FP_ERR_DTYPE


def test_paged_pools_and_page_table():
    ps, pages = 16, 40
    table = torch.zeros(1, -(-T // ps), dtype=torch.int32)
    p = _prob(page_table=table, page_size=ps, num_pages=pages)
    q = torch.zeros(T, HQ, D, dtype=torch.bfloat16)
    kp = torch.zeros(pages, ps, HKV, D, dtype=torch.bfloat16)
    qb, kb, vb = _pooled()
    k, v = _qkv()[1:]
    assert _code(fp.pool_blocks, p, q, k, v, qb, kb, vb)[0] == fp.FP_ERR_SHAPE          # contiguous K for paged
    assert _code(fp.pool_blocks, p, q, kp[:-1], kp, qb, kb, vb)[0] == fp.FP_ERR_SHAPE   # fewer pages than declared
    p64 = _prob(page_table=table.long(), page_size=ps, num_pages=pages)
    assert _code(fp.pool_blocks, p64, q, kp, kp, qb, kb, vb)[0] == fp.FP_ERR_DTYPE      # int64 page table
    assert _code(fp.pool_blocks, p, q, kp, kp, qb, kb, vb)[0] == fp.FP_ERR_LAYOUT       # CPU


def test_select_blocks_checks():
    p = _prob()
    rows, nnz, nbq, nbk = fp.index_shape(p)
    qb, kb, _ = _pooled()
    rp = torch.zeros(rows + 1, dtype=torch.int32)
    ci = torch.zeros(nnz, dtype=torch.int32)
    ws = torch.zeros(fp.select_workspace_bytes(p), dtype=torch.uint8)
    sel = fp.select_args(0.3)
    assert _code(fp.select_blocks, p, sel, qb, kb, rp.long(), ci, ws)[0] == fp.FP_ERR_DTYPE
    assert _code(fp.select_blocks, p, sel, qb, kb, rp[:-1], ci, ws)[0] == fp.FP_ERR_SHAPE
    assert _code(fp.select_blocks, p, sel, qb, kb, rp, ci.view(-1, 1), ws)[0] == fp.FP_ERR_SHAPE
    assert _code(fp.select_blocks, p, sel, qb, kb, rp, ci, ws.float())[0] == fp.FP_ERR_DTYPE
    assert _code(fp.select_blocks, p, sel, qb, kb, rp, ci, ws[:0])[0] == fp.FP_ERR_WORKSPACE
    assert _code(fp.select_blocks, p, sel, qb, kb, rp, ci, ws)[0] == fp.FP_ERR_LAYOUT


def test_attention_checks():
    p = _prob()
    rows, nnz, nbq, nbk = fp.index_shape(p)
    q, k, v = _qkv()
    _, kb, vb = _pooled()
    rp = torch.zeros(rows + 1, dtype=torch.int32)
    ci = torch.zeros(nnz, dtype=torch.int32)
    out = torch.zeros(T, HQ, D, dtype=torch.bfloat16)
    lse = torch.zeros(HQ, T)
    ws = torch.zeros(fp.attn_workspace_bytes(p, True), dtype=torch.uint8)
    a = fp.attn_args()
    assert _code(fp.sparse_prefill, p, a, q, k, v, kb, vb, rp, ci, out.float(), lse, ws)[0] == fp.FP_ERR_DTYPE
    assert _code(fp.sparse_prefill, p, a, q, k, v, kb, vb, rp, ci, out, lse.T, ws)[0] == fp.FP_ERR_SHAPE
    assert _code(fp.sparse_prefill, p, a, q, k, v, kb, vb, rp, ci, out, lse.T.contiguous().T, ws)[0] == \
        fp.FP_ERR_LAYOUT
    assert _code(fp.sparse_prefill, p, a, q, k, v, None, vb, rp, ci, out, lse, ws)[0] == fp.FP_ERR_NULL
    assert _code(fp.sparse_prefill, p, a, q, k, v, kb, vb, rp, ci, out, lse, ws.view(2, -1))[0] == \
        fp.FP_ERR_WORKSPACE
    assert _code(fp.sparse_prefill, p, a, q, k, v, kb, vb, rp, ci, out, lse, ws)[0] == fp.FP_ERR_LAYOUT
    assert _code(fp.dense_prefill, p, a, q, k, v, out[:, :1], lse)[0] == fp.FP_ERR_SHAPE
    assert _code(fp.dense_prefill, p, a, q, k, v, out, None)[0] == fp.FP_ERR_LAYOUT


def test_pooled_row_offsets_validation():
    # two requests of 3 and 2 key blocks (block 64) in a pooled buffer of pitch 10
    cu = [0, 150, 250]
    ok = fp.Problem(cu, HQ, HKV, B, pooled_pitch=10, pooled_row_off=[5, 0])
    fp.validate(ok)
    assert fp.index_shape(ok)[3] == 5
    for off, pitch in (([0, 2], 10), ([8, 0], 10), ([-1, 4], 10), ([0, 3], 4)):
        with pytest.raises(fp.FpError) as e:
            fp.validate(fp.Problem(cu, HQ, HKV, B, pooled_pitch=pitch, pooled_row_off=off))
        assert e.value.code == fp.FP_ERR_SHAPE, (off, pitch)
    # without a pitch the rows must fit in the call's own key-block count
    fp.validate(fp.Problem(cu, HQ, HKV, B, pooled_row_off=[2, 0]))
    with pytest.raises(fp.FpError):
        fp.validate(fp.Problem(cu, HQ, HKV, B, pooled_row_off=[0, 4]))
