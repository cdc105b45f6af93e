"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before touching any device pointer.

None of these calls launch a kernel, so they run without a GPU.
"""
import ctypes
import os
import re

import pytest
import torch

import block_sparse_long_fp_amd as fp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fpv2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fp.LIB_PATH), reason="libfpv2.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(fp_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"fp_pool_blocks", "fp_select_blocks", "fp_sparse_prefill", "fp_dense_prefill"} <= set(names)
    L = ctypes.CDLL(fp.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    ver = int(re.search(r"#define FPV2_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert fp.lib().fp_abi_version() == ver


ONE = fp.attn_args(num_splits=1) if os.path.exists(fp.LIB_PATH) else None   # no split-KV


def _prob(**kw):
    base = dict(cu_seqlens=[0, 1000, 3000], num_q_heads=32, num_kv_heads=8, block_size=128)
    base.update(kw)
    return fp.Problem(**base)


def test_attention_workspace_sizes():
    def a256(x):
        return (x + 255) // 256 * 256
    p = _prob()
    nb, T, Hkv, d = 24, 3000, 8, 128
    assert fp.attn_workspace_bytes(p, True, ONE) == 2 * a256(Hkv * nb * d * 2)
    assert fp.attn_workspace_bytes(p, False, ONE) == 0
    ds = [torch.ones(1) for _ in range(3)]
    p8 = _prob(dtype=fp.FP_FP8_E4M3, descales=ds)
    # FP8: plus one bf16 copy of the V codes (K is read as FP8).
    assert fp.attn_workspace_bytes(p8, True, ONE) == 2 * a256(Hkv * nb * d * 2) + a256(T * Hkv * d * 2)
    assert fp.attn_workspace_bytes(p8, False, ONE) == a256(T * Hkv * d * 2)


def test_index_shape_and_workspace():
    p = _prob()
    rows, nnz, nb, nbk = fp.index_shape(p)
    nbs = [8, 16]
    assert nb == 24 and rows == 8 * 24
    assert nnz == 8 * sum(n * (n + 1) // 2 for n in nbs)
    # selection workspace: a 256-byte ticket slot, then one 8-byte look-back
    # word per tile. Rows are tiled in 16-row blocks of about equal causal
    # area (at least one block per tile): here one tile per request and KV
    # head, 16 in all
    assert fp.select_workspace_bytes(p) == 256 + 256
    # 128K tokens, 8 KV heads: 256 tiles of about 16.7K score floats
    big = _prob(cu_seqlens=[0, 131072])
    assert fp.select_workspace_bytes(big) == 256 + 256 * 8
    # 32K tokens: 256 query blocks per KV head make too few 16-row blocks
    # for one tile per CU, so a tile holds the area of one widest block (8
    # per KV head, 64 in all); with about one matrix-core unit per wave
    # their key blocks are not split
    mid = _prob(cu_seqlens=[0, 32768])
    assert fp.select_workspace_bytes(mid) == 256 + 64 * 8
    # a 2048-token chunk after 129024 tokens: one 16-row block per KV head,
    # 64 units each, so each tile's 1024 key blocks go to 16 workgroups of
    # 64 (4 units, one per SIMD): the look-back words plus one arrival count
    # per tile, each part's row maxima (320 int32) and each tile's scores
    # (two widest blocks: 2 x 16 x (1024 + 3) floats)
    def a256(x):
        return (x + 255) // 256 * 256
    chunk = _prob(cu_seqlens=[0, 2048], cu_seqlens_k=[0, 131072])
    tiles, parts = 8, 16
    assert fp.select_workspace_bytes(chunk) == (256 + a256(2 * tiles * 8) + a256(tiles * parts * 320 * 4)
                                              + a256(tiles * 2 * 16 * 1027 * 4))


def test_chunked_index_shape():
    # Request 0: a 1000-token chunk after 2048 earlier tokens (qb0 = 16, 8
    # query blocks, 24 key blocks); request 1: a whole 640-token prefill.
    p = _prob(cu_seqlens=[0, 1000, 1640], cu_seqlens_k=[0, 3048, 3688])
    rows, nnz, nbq, nbk = fp.index_shape(p)
    assert (nbq, nbk) == (8 + 5, 24 + 5) and rows == 8 * 13
    assert nnz == 8 * (sum(16 + i + 1 for i in range(8)) + 5 * 6 // 2)
    def a256(x):
        return (x + 255) // 256 * 256
    assert fp.attn_workspace_bytes(p, True, ONE) == 2 * a256(8 * nbk * 128 * 2)
    ds = [torch.ones(1) for _ in range(3)]
    p8 = _prob(cu_seqlens=[0, 1000, 1640], cu_seqlens_k=[0, 3048, 3688], dtype=fp.FP_FP8_E4M3, descales=ds)
    # the FP8 V copy covers every key token (Tk = 3688), not only the chunk
    assert fp.attn_workspace_bytes(p8, False, ONE) == a256(3688 * 8 * 128 * 2)


def test_split_kv_choice_and_workspace():
    def a256(x):
        return (x + 255) // 256 * 256
    # 8 KV heads x 24 query blocks x 2 workgroups per row = 384 workgroups
    # fill the 256 CUs: no split. 2 KV heads: 96 workgroups, so 3 parts; the
    # workspace gains the parts' fp32 outputs and log-sum-exps
    assert fp.attn_num_splits(_prob()) == 1
    p = _prob(num_q_heads=8, num_kv_heads=2)
    assert fp.attn_num_splits(p) == 3 and fp.attn_num_splits(p, fp.attn_args(num_splits=5)) == 5
    T, Hq = 3000, 8
    base = fp.attn_workspace_bytes(p, True, ONE)
    assert base == 2 * a256(2 * 24 * 128 * 2)
    assert fp.attn_workspace_bytes(p, True) == base + a256(3 * T * Hq * 128 * 4) + a256(3 * T * Hq * 4)
    assert fp.attn_workspace_bytes(p, False) == a256(3 * T * Hq * 128 * 4) + a256(3 * T * Hq * 4)
    # a 128K prompt has enough rows: no split; a one-block problem cannot split
    assert fp.attn_num_splits(_prob(cu_seqlens=[0, 131072])) == 1
    assert fp.attn_num_splits(_prob(cu_seqlens=[0, 100])) == 1
    # 16 at most; out of range is rejected
    assert fp.attn_num_splits(_prob(cu_seqlens=[0, 4096], num_q_heads=1, num_kv_heads=1, block_size=64)) == 4
    assert fp.attn_num_splits(_prob(cu_seqlens=[0, 8192], num_q_heads=1, num_kv_heads=1)) == 4
    assert fp.attn_num_splits(_prob(cu_seqlens=[0, 4000], num_q_heads=1, num_kv_heads=1, block_size=64)) == 5
    assert fp.attn_num_splits(_prob(cu_seqlens=[0, 1024], num_q_heads=1, num_kv_heads=1, block_size=64)) == 16
    for bad in (-1, 17):
        with pytest.raises(fp.FpError) as e:
            fp.validate(p, None, fp.attn_args(num_splits=bad))
        assert e.value.code == 9


def test_pooled_pitch():
    # a pitch below the key-block count is rejected; a larger one sizes the
    # pooled copies of the attention workspace
    with pytest.raises(fp.FpError) as e:
        fp.validate(_prob(pooled_pitch=23))
    assert e.value.code == 2
    def a256(x):
        return (x + 255) // 256 * 256
    assert fp.attn_workspace_bytes(_prob(pooled_pitch=100), True, ONE) == 2 * a256(8 * 100 * 128 * 2)
    b = fp.Problem([0, 1000], 32, 8, 128, cu_seqlens_k=[0, 3048], pooled_pitch=40)
    assert fp.index_shape(b)[2:] == (8, 24)


@pytest.mark.parametrize("cuk", [
    [0, 999, 1640],     # fewer keys than queries
    [0, 1100, 1740],    # chunk offset 100 is not a multiple of 128
    [5, 1000, 1640],    # does not start at 0
])
def test_chunked_validation(cuk):
    with pytest.raises(fp.FpError) as e:
        fp.validate(_prob(cu_seqlens=[0, 1000, 1640], cu_seqlens_k=cuk))
    assert e.value.code == 2


def test_index_memory_matches_the_pages_order_of_magnitude():
    # Table 7 of the digest: at 128K with 32 query / 4 KV heads the CSR of
    # selected blocks takes about 6 MB at ~5% density, against 32 MB for a
    # dense per-query-head byte mask of 128-token tiles. Our worst case (every
    # causal block of 128 tokens, per KV head) times the density gives the
    # same order: 4 * 1024*1025/2 * 0.05 * 4 B ~ 0.4 MB, far under the mask.
    p = _prob(cu_seqlens=[0, 131072], num_q_heads=32, num_kv_heads=4, block_size=128)
    rows, nnz, nb, nbk = fp.index_shape(p)
    mask_bytes = 32 * 1024 * 1024
    assert mask_bytes == 32 * 2 ** 20
    assert nnz * 4 * 0.05 < 6e6 < mask_bytes


@pytest.mark.parametrize("kw,code", [
    (dict(num_kv_heads=5), 3),
    (dict(block_size=96), 4),
    (dict(head_dim=64), 10),
    (dict(cu_seqlens=[0, 10, 5]), 2),
    (dict(cu_seqlens=[1, 10]), 2),
    (dict(cu_seqlens=[0] + list(range(1, 130))), 10),
    (dict(dtype=1), 5),
    (dict(dtype=7), 5),
    (dict(num_q_heads=0), 2),
])
def test_problem_validation(kw, code):
    with pytest.raises(fp.FpError) as e:
        fp.validate(_prob(**kw))
    assert e.value.code == code
    assert fp.lib().fp_last_error().decode()


def test_paged_validation():
    class FakeTensor:
        def __init__(self, shape):
            self.shape = shape

        def data_ptr(self):
            return 0x1000

    p = fp.Problem([0, 1000], 8, 2, 128, page_table=FakeTensor((1, 10)), page_size=64, num_pages=100)
    with pytest.raises(fp.FpError) as e:
        fp.validate(p)  # 1000 tokens need 16 pages of 64, table has 10
    assert e.value.code == 6
    p = fp.Problem([0, 1000], 8, 2, 128, page_table=FakeTensor((1, 16)), page_size=0, num_pages=100)
    with pytest.raises(fp.FpError) as e:
        fp.validate(p)
    assert e.value.code == 6
    fp.validate(fp.Problem([0, 1000], 8, 2, 128, page_table=FakeTensor((1, 16)), page_size=64, num_pages=100))


def test_argument_validation():
    p = _prob()
    with pytest.raises(fp.FpError) as e:
        fp.validate(p, fp.select_args(float("nan")))
    assert e.value.code == 9
    for tau in (float("inf"), 0.0, -1.0, float("nan")):
        with pytest.raises(fp.FpError) as e:
            fp.validate(p, fp.select_args(0.3, tau))
        assert e.value.code == 9
    with pytest.raises(fp.FpError) as e:
        fp.validate(p, None, fp.attn_args(-1.0))
    assert e.value.code == 9
    with pytest.raises(fp.FpError) as e:
        fp.validate(p, None, fp._AttnArgs(0.1, 2))
    assert e.value.code == 9
    fp.validate(p, fp.select_args(0.3), fp.attn_args())
    fp.validate(p, fp.select_args(-1.0), fp.attn_args(0.0, False))


def test_compute_calls_reject_before_launch():
    """Null buffers, small capacity and small workspace fail on the host."""
    p = _prob()
    L = fp.lib()
    sel = fp.select_args(0.3)
    attn = fp.attn_args()
    vp = ctypes.c_void_p
    fake = vp(0x1000)
    assert L.fp_pool_blocks(p.ref, None, fake, fake, fake, fake, fake, None) == 1
    rows, nnz, nb, nbk = fp.index_shape(p)
    ws = fp.select_workspace_bytes(p)
    assert L.fp_select_blocks(p.ref, ctypes.byref(sel), fake, fake, fake, fake, nnz - 1, fake, ws, None) == 7
    assert L.fp_select_blocks(p.ref, ctypes.byref(sel), fake, fake, fake, fake, nnz, fake, ws - 1, None) == 8
    assert L.fp_select_blocks(p.ref, ctypes.byref(sel), fake, fake, fake, fake, nnz, None, ws, None) == 8
    aws = fp.attn_workspace_bytes(p, True, ONE)
    assert aws > 0 and fp.attn_workspace_bytes(p, False, ONE) == 0  # bf16: only the pooled copies
    assert L.fp_sparse_prefill(p.ref, ctypes.byref(attn), fake, fake, fake, None, fake, fake, fake, fake, None,
                               fake, aws, None) == 1
    assert L.fp_sparse_prefill(p.ref, ctypes.byref(attn), fake, fake, fake, fake, fake, None, fake, fake, None,
                               fake, aws, None) == 1
    assert L.fp_sparse_prefill(p.ref, ctypes.byref(attn), fake, fake, fake, fake, fake, fake, fake, fake, None,
                               fake, aws - 1, None) == 8
    assert L.fp_sparse_prefill(p.ref, ctypes.byref(attn), fake, fake, fake, fake, fake, fake, fake, fake, None,
                               None, aws, None) == 8
    assert L.fp_dense_prefill(p.ref, ctypes.byref(attn), fake, fake, fake, None, None, None, 0, None) == 1
    for code in range(12):
        assert L.fp_status_string(code)


def test_noalloc_selection_rejects_problems_beyond_its_array():
    """fp_select_blocks_noalloc holds the selection workspace of at most
    FP_NOALLOC_MAX_SELECT_TILES tiles; a larger problem (128 one-block
    requests x 1024 KV heads = 131072 tiles) is rejected on the host with
    FP_ERR_CAPACITY before any device call."""
    header = open(HEADER).read()
    cap = int(re.search(r"#define FP_NOALLOC_MAX_SELECT_TILES (\d+)", header).group(1))
    assert cap == 65536
    cu = [64 * i for i in range(129)]
    p = fp.Problem(cu, 1024, 1024, 64)
    rows, nnz, nbq, nbk = fp.index_shape(p)
    assert rows == 131072
    sel = fp.select_args(0.3)
    fake = ctypes.c_void_p(0x1000)
    code = fp.lib().fp_select_blocks_noalloc(p.ref, ctypes.byref(sel), fake, fake, fake, fake, nnz, None)
    assert code == fp.FP_ERR_CAPACITY
    assert b"no-alloc" in fp.lib().fp_last_error()


def test_check_index_rejects_bad_arguments_on_the_host():
    """fp_check_index validates before launching: a NULL error word, one of
    row_ptr / col_idx without the other, or a negative capacity (fake
    non-NULL device pointers; nothing is dereferenced)."""
    L = fp.lib()
    p = _prob()
    fake = ctypes.c_void_p(0x1000)
    assert L.fp_check_index(p.ref, fake, fake, 10, None, None) == fp.FP_ERR_NULL
    assert L.fp_check_index(p.ref, fake, None, 10, fake, None) == fp.FP_ERR_NULL
    assert L.fp_check_index(p.ref, None, fake, 10, fake, None) == fp.FP_ERR_NULL
    assert L.fp_check_index(p.ref, fake, fake, -1, fake, None) == 9  # FP_ERR_ARG
    bad = _prob(num_q_heads=30)  # GQA mismatch is caught by the problem check first
    assert L.fp_check_index(bad.ref, fake, fake, 10, fake, None) == 3


def test_workspace_bytes_by_call_matches_the_specific_sizes():
    """fp_workspace_bytes(which_call) returns what the per-call sizing
    functions return (attention with its default arguments), for a batch, a
    single long prompt, a chunk and an FP8 paged problem; an unknown call is
    FP_ERR_ARG."""
    ds = [torch.ones(1) for _ in range(3)]
    table = torch.zeros((2, 40), dtype=torch.int32)
    probs = [_prob(), _prob(cu_seqlens=[0, 131072]), _prob(cu_seqlens=[0, 2048], cu_seqlens_k=[0, 131072]),
             _prob(dtype=fp.FP_FP8_E4M3, descales=ds, page_table=table, page_size=128, num_pages=80)]
    for p in probs:
        assert fp.workspace_bytes(p, fp.FP_CALL_SELECT) == fp.select_workspace_bytes(p)
        assert fp.workspace_bytes(p, fp.FP_CALL_SPARSE) == fp.attn_workspace_bytes(p, True)
        assert fp.workspace_bytes(p, fp.FP_CALL_DENSE) == fp.attn_workspace_bytes(p, False)
    n = ctypes.c_size_t()
    assert fp.lib().fp_workspace_bytes(probs[0].ref, 7, ctypes.byref(n)) == 9  # FP_ERR_ARG
