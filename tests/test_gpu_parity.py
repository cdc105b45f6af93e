"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Sizes are small enough for the oracle to finish in seconds, yet span several
key blocks, several workgroups per (KV head, query block) and ragged tails.
Bar: bit-exact CSR outside the near-threshold band; O max-abs <= 2e-2 (bf16)
or 6e-2 (fp8); LSE relative error <= 1e-3 (against max(|LSE|, 1e-2)).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_common import (O_TOL, compare_csr, compare_outputs, compare_pooled, run_gpu, run_oracle,
                        sets_from_csr, host_values, upload)
import oracle

pytestmark = pytest.mark.gpu


def _check_full(wl, alpha=None, mean_correction=True, paged=None, min_sparse_len=None, forced=None, num_splits=0,
                sm_scale=0.0):
    print(f"[parity] {wl.name} L={wl.seqlens} Lk={wl.key_seqlens} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} B={wl.block_size} "
          f"dtype={wl.dtype} alpha={alpha if alpha is not None else wl.alpha} mc={mean_correction} "
          f"paged={paged if paged is not None else wl.paged} forced={forced}", flush=True)
    gpu = run_gpu(wl, alpha, mean_correction, paged, min_sparse_len=min_sparse_len, forced=forced,
                  num_splits=num_splits, sm_scale=sm_scale)
    orc = run_oracle(wl, alpha, mean_correction, do_attend=False, paged=paged, min_sparse_len=min_sparse_len,
                     forced=forced)
    compare_pooled(gpu, orc)
    n_near = compare_csr(gpu, orc)
    # Attention on the CSR the GPU chose (identical to the oracle's outside the band).
    Q, K, V = host_values(wl)
    sets = sets_from_csr(gpu["row_ptr"], gpu["col_idx"], orc.blk_off, wl.num_kv_heads)
    O = np.full_like(Q, np.nan)
    LSE = np.full((wl.num_q_heads, Q.shape[0]), np.nan)
    import math
    G = wl.num_q_heads // wl.num_kv_heads
    cuk = wl.cu_seqlens_k or wl.cu_seqlens
    for r in range(len(wl.seqlens)):
        s, e = wl.cu_seqlens[r], wl.cu_seqlens[r + 1]
        ks, ke = cuk[r], cuk[r + 1]
        a, b = orc.kblk_off[r], orc.kblk_off[r + 1]
        o, l = oracle.attend(Q[s:e], K[ks:ke], V[ks:ke], orc.kbar[:, a:b], orc.vbar[:, a:b], sets[r],
                             wl.block_size, G, sm_scale or 1.0 / math.sqrt(wl.head_dim), mean_correction,
                             q_off=(ke - ks) - (e - s))
        O[s:e], LSE[:, s:e] = o, l
    o_err, l_rel, l_abs = compare_outputs(gpu["out"], gpu["lse"], O, LSE, O_TOL[wl.dtype])
    print(f"[parity] ok: nnz={gpu['row_ptr'][-1]} near_rows={n_near} O_err={o_err:.2e} LSE_rel={l_rel:.2e} "
          f"LSE_abs={l_abs:.2e}", flush=True)
    return gpu


def test_tiny_needle_full():
    _check_full(synth.make_workload("tiny_4k"))


def test_gqa4_block128_ragged():
    wl = synth.make_workload("llama_32k", L=3000, Hq=8, Hkv=2, n_planted=6)
    _check_full(wl)


def test_gqa8_block64_ragged():
    wl = synth.make_workload("llama_32k", L=2500, Hq=16, Hkv=2, B=64, n_planted=8, alpha=0.4)
    _check_full(wl)


def test_gqa1_block128():
    wl = synth.make_workload("llama_32k", L=1500, Hq=2, Hkv=2, n_planted=3)
    _check_full(wl)


def test_mean_correction_off():
    wl = synth.make_workload("llama_32k", L=2200, Hq=8, Hkv=2, n_planted=5)
    _check_full(wl, mean_correction=False)


@pytest.mark.parametrize("sm_scale,fp8,mc", [(0.05, False, True), (0.2, False, True), (0.15, True, False)])
def test_softmax_scale_and_fp8_without_correction(sm_scale, fp8, mc):
    """A caller's softmax scale instead of 1 / sqrt(d) (on exact and pooled
    logits alike; the pooled logit's ln n_J does not scale), and FP8 inputs
    with the mean correction off. Ragged GQA-4 batch."""
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[1300, 500], Hq=8, Hkv=2, min_sparse_len=0,
                             n_planted=3, fp8=fp8, page_size=0)
    _check_full(wl, mean_correction=mc, sm_scale=sm_scale)


def test_fp8_gqa8():
    wl = synth.make_workload("qwen30b_128k_fp8", L=3000, Hq=16, Hkv=2, n_planted=6)
    _check_full(wl)


@pytest.mark.parametrize("Hq,Hkv,B,fp8,splits", [
    (6, 2, 128, False, 0),    # G = 3: 384 packed rows, the second 256-row sub-tile half empty
    (10, 2, 128, False, 0),   # G = 5 (40 / 8 heads): 640 rows, third sub-tile half empty
    (14, 2, 64, False, 0),    # G = 7 (28 / 4 heads), 64-key blocks: 448 rows
    (10, 2, 128, True, 0),    # G = 5 with FP8 products
    (6, 2, 128, False, 3),    # G = 3, split-KV
    (12, 4, 64, True, 3),     # G = 3, 64-key blocks: 192 rows (two waves idle), FP8, split-KV
])
def test_gqa_ratios_that_leave_waves_without_rows(Hq, Hkv, B, fp8, splits):
    """GQA ratios whose G B packed rows do not fill whole 256-row sub-tiles:
    the last sub-tile of every row has waves without rows (which still issue
    their share of each block's DMA and take part in every barrier), and
    pooling sums an odd number of query heads per group. Ragged requests,
    paged K / V with 16-token pages for the bf16 cases."""
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[1500, 700], Hq=Hq, Hkv=Hkv, min_sparse_len=0,
                             n_planted=3, B=B, fp8=fp8, page_size=0 if fp8 else 16)
    assert wl.num_q_heads // wl.num_kv_heads * B % 256 != 0
    _check_full(wl, num_splits=splits)


@pytest.mark.parametrize("Hq,Hkv,B,fp8", [
    (32, 2, 128, False),   # G = 16: 2048 packed rows, 8 sub-tiles per row
    (32, 1, 128, False),   # one KV head (multi-query), G = 32: 16 sub-tiles, 32 heads pooled per group
    (32, 1, 64, True),     # multi-query with 64-key blocks and FP8
    (32, 32, 128, False),  # multi-head, 32 KV heads (the KV head of a work slot rotates every 32 query blocks)
    (48, 16, 128, True),   # 16 KV heads, G = 3, FP8
])
def test_head_counts(Hq, Hkv, B, fp8):
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[1000, 380], Hq=Hq, Hkv=Hkv, min_sparse_len=0,
                             n_planted=2, B=B, fp8=fp8, page_size=0 if fp8 else 64)
    _check_full(wl)


@pytest.mark.parametrize("page_size", [0, 64, 6])
def test_fp8_block64_varlen(page_size):
    # FP8 products with 64-key blocks (one FP8 K DMA instruction per wave) on
    # ragged requests, unsplit and split; paged K / V (page sizes with and
    # without whole 8-row groups per page) must equal the contiguous layout
    # bit for bit.
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[700, 1333], Hq=8, Hkv=2, min_sparse_len=0,
                             n_planted=3, B=64, fp8=True, page_size=page_size)
    assert wl.dtype == "fp8" and wl.paged == (page_size > 0)
    _check_full(wl, num_splits=1)
    _check_full(wl, num_splits=3)
    if page_size:
        a = run_gpu(wl, paged=True, num_splits=1)
        b = run_gpu(wl, paged=False, num_splits=1)
        for key in ("row_ptr", "col_idx", "out", "lse"):
            assert np.array_equal(a[key], b[key]), key


def test_varlen_paged_min_sparse_len():
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[300, 1000, 2100, 129], Hq=8, Hkv=2,
                             min_sparse_len=1000, page_size=64)
    _check_full(wl)


def test_varlen_paged_odd_page_size():
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[700, 1333], Hq=4, Hkv=1, min_sparse_len=0,
                             page_size=48, n_planted=3)
    _check_full(wl)


def test_paged_equals_contiguous_bitwise():
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[900, 1700], Hq=8, Hkv=2, min_sparse_len=0,
                             page_size=64, n_planted=4)
    a = run_gpu(wl, paged=True)
    b = run_gpu(wl, paged=False)
    for key in ("q_bar", "k_bar", "v_bar", "row_ptr", "col_idx", "out", "lse"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("page_size", [17, 6])
def test_paged_page_size_not_multiple_of_4(page_size):
    # Page sizes that are not a multiple of 4 take the per-row page lookup
    # (the four rows one DMA instruction of a wave fills may straddle pages);
    # the result must equal the contiguous layout's bit for bit.
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[700, 1333], Hq=4, Hkv=1, min_sparse_len=0,
                             page_size=page_size, n_planted=3)
    _check_full(wl)
    a = run_gpu(wl, paged=True)
    b = run_gpu(wl, paged=False)
    for key in ("row_ptr", "col_idx", "out", "lse"):
        assert np.array_equal(a[key], b[key]), key


def test_alpha_zero_sparse_equals_dense_kernel_and_oracle():
    # unsplit, so both calls process each row's key blocks in one sequence
    wl = synth.make_workload("llama_32k", L=1800, Hq=8, Hkv=2, n_planted=4)
    sp = run_gpu(wl, alpha=0.0, num_splits=1)
    dn = run_gpu(wl, dense=True, num_splits=1)
    nb = -(-1800 // 128)
    assert sp["row_ptr"][-1] == 2 * nb * (nb + 1) // 2
    assert np.array_equal(sp["out"], dn["out"]) and np.array_equal(sp["lse"], dn["lse"])
    orc = run_oracle(wl, alpha=0.0)
    compare_outputs(dn["out"], dn["lse"], orc.O, orc.LSE, O_TOL["bf16"])


def test_dense_kernel_fp8_and_varlen():
    wl = synth.make_workload("qwen30b_128k_fp8", L=1300, Hq=8, Hkv=1, n_planted=3)
    dn = run_gpu(wl, dense=True)
    orc = run_oracle(wl, alpha=0.0)
    compare_outputs(dn["out"], dn["lse"], orc.O, orc.LSE, O_TOL["fp8"])
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[200, 640, 1000], Hq=4, Hkv=2, page_size=64,
                             min_sparse_len=0)
    dn = run_gpu(wl, dense=True)
    orc = run_oracle(wl, alpha=0.0)
    compare_outputs(dn["out"], dn["lse"], orc.O, orc.LSE, O_TOL["bf16"])


def test_alpha_above_one_keeps_only_diagonal():
    wl = synth.make_workload("llama_32k", L=1200, Hq=4, Hkv=1, n_planted=3)
    gpu = _check_full(wl, alpha=1.5)
    nb = -(-1200 // 128)
    assert gpu["row_ptr"][-1] == nb
    assert np.array_equal(gpu["col_idx"], np.arange(nb))


@pytest.mark.parametrize("fp8", [False, True])
def test_single_token_and_one_block_requests(fp8):
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[1, 2, 127, 128, 129], Hq=4, Hkv=2, page_size=16,
                             min_sparse_len=0, n_planted=0, fp8=fp8)
    _check_full(wl)
    _check_full(wl, paged=False, num_splits=1)


@pytest.mark.parametrize("num_splits", [1, 3])
def test_lse_buffer_is_optional(num_splits):
    """lse = NULL skips the log-sum-exp: the sparse and dense calls, unsplit
    and split (whose merge kernel writes the LSE), give bitwise the same
    output with and without it. Ragged GQA-4 batch, FP8."""
    import block_sparse_long_fp_amd as fp
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[1300, 500], Hq=8, Hkv=2, min_sparse_len=0,
                             n_planted=3, fp8=True, page_size=0)
    prob, q, k, v = upload(wl)
    att = fp.attn_args(0.0, True, num_splits)
    bufs = fp.Buffers(prob, "cuda:0", attn=att)
    fp.run_prefill(prob, bufs, q, k, v, wl.alpha, wl.sel_scale, 0, 0.0, True, num_splits=num_splits)
    for dense in (False, True):
        outs = []
        for with_lse in (True, False):
            out = torch.full_like(bufs.out, 7.0)
            lse = torch.full_like(bufs.lse, 7.0) if with_lse else None
            if dense:
                fp.dense_prefill(prob, att, q, k, v, out, lse)
            else:
                fp.sparse_prefill(prob, att, q, k, v, bufs.k_bar, bufs.v_bar, bufs.row_ptr, bufs.col_idx, out, lse)
            torch.cuda.synchronize()
            outs.append(out.cpu())
            if with_lse:
                assert torch.isfinite(lse).all() and not (lse == 7.0).any()
        assert torch.equal(outs[0], outs[1]), f"dense={dense}"


@pytest.mark.parametrize("num_splits", [1, 3])
def test_batch_of_the_most_requests(num_splits):
    """FP_MAX_SEQS = 128 requests of seeded lengths 1 .. 399 (one- and
    two-token requests, block-boundary lengths, ragged tails), 64-key blocks,
    paged K / V: the attention kernel's multi-request decode holds request q
    in lane q and, past 64 requests, in lane q + 64 as well; pooling,
    selection tiles and the CSR offsets walk the whole request table."""
    rng = np.random.default_rng(128)
    lengths = [int(x) for x in rng.integers(1, 400, 128)]
    lengths[:6] = [1, 2, 63, 64, 65, 128]
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=lengths, Hq=4, Hkv=1, B=64, min_sparse_len=0,
                             n_planted=0, page_size=16)
    assert len(wl.seqlens) == 128
    _check_full(wl, num_splits=num_splits)


@pytest.mark.parametrize("num_splits", [1, 3])
def test_chunk_of_the_most_requests(num_splits):
    """A chunked-prefill call over 128 requests: each request's queries are
    its positions 128 .. 383 (fewer where it ends sooner) against every key
    before them, so every request's first query block is key block 2 and the
    chunks end raggedly. Paged K / V, 64-key blocks."""
    rng = np.random.default_rng(129)
    lengths = [int(x) for x in rng.integers(150, 900, 128)]
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=lengths, Hq=4, Hkv=1, B=64, min_sparse_len=0,
                             n_planted=0, page_size=16)
    batch = synth.chunk_of(wl, 128, 256)
    assert len(batch.seqlens) == 128 and batch.cu_seqlens_k is not None
    _check_full(batch, num_splits=num_splits)


@pytest.mark.parametrize("forced", [dict(sink=2, window=4, last_n=8), dict(sink=1, window=0, last_n=0),
                                    dict(sink=0, window=2, last_n=3)])
def test_forced_keeps_sink_window_last_n(forced):
    """The article's serving flags (attention sink 2, window 4, last-n 8
    blocks) and single rules, on a ragged GQA-4 batch."""
    wl = synth.make_workload("llama_32k", lengths=[3000, 5000], Hq=8, Hkv=2, n_planted=4, kind="varlen",
                             seeds_base=7, page_size=0, min_sparse_len=0)
    gpu = _check_full(wl, forced=forced)
    # every forced block is in the GPU's CSR
    nb = [-(-L // wl.block_size) for L in wl.seqlens]
    off = np.concatenate([[0], np.cumsum(nb)])
    for h in range(wl.num_kv_heads):
        for r, NB in enumerate(nb):
            for I in range(NB):
                row = h * off[-1] + off[r] + I
                cols = set(gpu["col_idx"][gpu["row_ptr"][row]:gpu["row_ptr"][row + 1]].tolist())
                want = set(np.nonzero(oracle.forced_keep(I, NB, **forced))[0].tolist())
                assert want <= cols, (h, r, I)


def test_runs_are_bitwise_deterministic():
    wl = synth.make_workload("llama_32k", L=2600, Hq=8, Hkv=2, n_planted=6)
    a = run_gpu(wl)
    b = run_gpu(wl)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


# ---------------------------------------------------------------- chunked prefill

def _with_whole_request(chunk, whole):
    """Append a whole-prompt request (keys = queries) to a chunked batch."""
    import dataclasses
    Tq, Tk = chunk.cu_seqlens[-1], chunk.cu_seqlens_k[-1]
    L = whole.cu_seqlens[-1]
    return dataclasses.replace(chunk, q=torch.cat([chunk.q, whole.q]), k=torch.cat([chunk.k, whole.k]),
                               v=torch.cat([chunk.v, whole.v]), cu_seqlens=chunk.cu_seqlens + [Tq + L],
                               cu_seqlens_k=chunk.cu_seqlens_k + [Tk + L])


def test_chunked_prefill_ragged():
    """Chunked prefill ([digest] Table 6): a 1000-query chunk after 2048
    earlier positions of one request, the short last chunk (552 queries) of
    another, and a ragged whole prompt, in one batch; then the dense kernel
    on the same batch against the oracle with every block kept."""
    wl = synth.make_workload("llama_32k", lengths=[3048, 2600], Hq=8, Hkv=2, n_planted=4, kind="varlen",
                             seeds_base=20, page_size=0, min_sparse_len=0)
    whole = synth.make_workload("llama_32k", L=777, Hq=8, Hkv=2, n_planted=2)
    batch = _with_whole_request(synth.chunk_of(wl, 2048, 1000), whole)
    assert batch.seqlens == [1000, 552, 777] and batch.key_seqlens == [3048, 2600, 777]
    _check_full(batch)
    dn = run_gpu(batch, dense=True)
    orc = run_oracle(batch, alpha=0.0)
    compare_outputs(dn["out"], dn["lse"], orc.O, orc.LSE, O_TOL["bf16"])


def test_chunked_prefill_paged_fp8_and_forced():
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[2900, 1500], Hq=8, Hkv=2, min_sparse_len=0,
                             page_size=48, n_planted=3)
    _check_full(synth.chunk_of(wl, 1024, 1024), forced=dict(sink=1, window=2, last_n=2))
    wl8 = synth.make_workload("qwen30b_128k_fp8", L=3500, Hq=16, Hkv=2, n_planted=6)
    _check_full(synth.chunk_of(wl8, 2560, 2048))


def test_chunked_rows_equal_whole_prefill_bitwise():
    """A chunk's rows see the same pooled statistics, the same selection and
    the same items in the same order as in one prefill of the whole prompt,
    so the GPU path gives bitwise the same outputs for them."""
    wl = synth.make_workload("llama_32k", L=3000, Hq=8, Hkv=2, n_planted=6)
    whole = run_gpu(wl, num_splits=1)
    B, start = wl.block_size, 1536
    ch = run_gpu(synth.chunk_of(wl, start, 4096), num_splits=1)
    assert np.array_equal(ch["out"], whole["out"][start:])
    assert np.array_equal(ch["lse"], whole["lse"][:, start:])
    assert np.array_equal(ch["k_bar"], whole["k_bar"]) and np.array_equal(ch["v_bar"], whole["v_bar"])
    nb, qb0 = -(-3000 // B), start // B
    for h in range(wl.num_kv_heads):
        assert np.array_equal(ch["q_bar"][h], whole["q_bar"][h, qb0:])
        for i in range(nb - qb0):
            a = ch["col_idx"][ch["row_ptr"][h * (nb - qb0) + i]:ch["row_ptr"][h * (nb - qb0) + i + 1]]
            gr = h * nb + qb0 + i
            assert np.array_equal(a, whole["col_idx"][whole["row_ptr"][gr]:whole["row_ptr"][gr + 1]])


def test_chunk_pooling_reuses_earlier_blocks():
    """fp_pool_chunk_blocks pools only the key blocks a chunk adds: on buffers
    sized for the whole prompt (pooled_pitch), rows of earlier blocks are left
    as they were, and a sequence of chunks, each pooled that way, then
    selected and attended, gives bitwise the whole prefill's outputs."""
    import block_sparse_long_fp_amd as fp
    wl = synth.make_workload("llama_32k", L=3000, Hq=8, Hkv=2, n_planted=6)
    whole = run_gpu(wl, num_splits=1)
    B, C, L = wl.block_size, 1024, 3000
    NB = -(-L // B)
    dev = "cuda:0"
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    kbar = torch.full((2, NB, 128), 7.0, device=dev)
    vbar = torch.full((2, NB, 128), 7.0, device=dev)
    for s0 in range(0, L, C):
        c = min(C, L - s0)
        print(f"[parity] chunk at {s0}, {c} queries", flush=True)
        prob = fp.Problem([0, c], 8, 2, B, cu_seqlens_k=[0, s0 + c], pooled_pitch=NB)
        bufs = fp.Buffers(prob, dev)
        # a fresh buffer: rows before the chunk keep a sentinel
        sk = torch.full((2, NB, 128), 3.0, device=dev)
        sv = torch.full((2, NB, 128), 3.0, device=dev)
        fp.pool_chunk_blocks(prob, q[s0:s0 + c], k, v, bufs.q_bar, sk, sv)
        fp.pool_chunk_blocks(prob, q[s0:s0 + c], k, v, bufs.q_bar, kbar, vbar)
        fp.select_blocks(prob, fp.select_args(wl.alpha), bufs.q_bar, kbar, bufs.row_ptr, bufs.col_idx,
                         bufs.workspace)
        fp.sparse_prefill(prob, fp.attn_args(num_splits=1), q[s0:s0 + c], k, v, kbar, vbar, bufs.row_ptr,
                          bufs.col_idx, bufs.out, bufs.lse, bufs.attn_workspace)
        torch.cuda.synchronize()
        qb0, nbk = s0 // B, -(-(s0 + c) // B)
        assert (sk[:, :qb0] == 3.0).all() and (sv[:, :qb0] == 3.0).all()
        assert (sk[:, nbk:] == 3.0).all()
        assert np.array_equal(sk[:, qb0:nbk].cpu().numpy(), whole["k_bar"][:, qb0:nbk])
        assert np.array_equal(sv[:, qb0:nbk].cpu().numpy(), whole["v_bar"][:, qb0:nbk])
        assert np.array_equal(bufs.out.float().cpu().numpy(), whole["out"][s0:s0 + c])
        assert np.array_equal(bufs.lse.cpu().numpy(), whole["lse"][:, s0:s0 + c])
    assert np.array_equal(kbar.cpu().numpy(), whole["k_bar"])


def test_chunk_pooling_two_requests_keeps_rows_in_place():
    """A batch of two ragged paged requests prefilled in 1024-query chunks,
    each chunk pooling only the key blocks it adds (fp_pool_chunk_blocks).
    pooled_row_off gives each request a fixed region of the pooled buffers
    (rows 0..22 and 23..46 of a pitch-47 buffer, the whole prefill's layout),
    so a request's earlier rows stay where the earlier chunks wrote them even
    though the other request's key-block count grows from chunk to chunk.
    Every chunk's outputs must equal the same rows of one whole prefill of
    the batch bit for bit, and so must the pooled buffers at the end."""
    import block_sparse_long_fp_amd as fp
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[2900, 3000], Hq=8, Hkv=2, min_sparse_len=0,
                             page_size=64, n_planted=4)
    whole = run_gpu(wl, num_splits=1)
    B, C = wl.block_size, 1024
    nbs = [-(-L // B) for L in wl.seqlens]
    base, pitch = [0, nbs[0]], sum(nbs)
    dev = "cuda:0"
    q = wl.q.to(dev)
    kp, vp, table = wl.k_pages.to(dev), wl.v_pages.to(dev), wl.page_table.to(dev)
    kbar = torch.full((2, pitch, 128), 7.0, device=dev)
    vbar = torch.full((2, pitch, 128), 7.0, device=dev)
    for s0 in range(0, max(wl.seqlens), C):
        lens = [min(C, L - s0) for L in wl.seqlens]
        assert min(lens) > 0
        print(f"[parity] two-request chunk at {s0}: {lens} queries", flush=True)
        cu = [0, lens[0], lens[0] + lens[1]]
        cuk = [0, s0 + lens[0], 2 * s0 + lens[0] + lens[1]]
        qc = torch.cat([q[wl.cu_seqlens[r] + s0:wl.cu_seqlens[r] + s0 + lens[r]] for r in range(2)]).contiguous()
        prob = fp.Problem(cu, 8, 2, B, page_table=table, page_size=64, num_pages=kp.shape[0], cu_seqlens_k=cuk,
                          pooled_pitch=pitch, pooled_row_off=base)
        bufs = fp.Buffers(prob, dev)
        fp.pool_chunk_blocks(prob, qc, kp, vp, bufs.q_bar, kbar, vbar)
        fp.select_blocks(prob, fp.select_args(wl.alpha), bufs.q_bar, kbar, bufs.row_ptr, bufs.col_idx,
                         bufs.workspace)
        fp.sparse_prefill(prob, fp.attn_args(num_splits=1), qc, kp, vp, kbar, vbar, bufs.row_ptr, bufs.col_idx,
                          bufs.out, bufs.lse, bufs.attn_workspace)
        torch.cuda.synchronize()
        out, lse = bufs.out.float().cpu().numpy(), bufs.lse.cpu().numpy()
        for r in range(2):
            a, e = wl.cu_seqlens[r] + s0, wl.cu_seqlens[r] + s0 + lens[r]
            assert np.array_equal(out[cu[r]:cu[r + 1]], whole["out"][a:e]), (s0, r)
            assert np.array_equal(lse[:, cu[r]:cu[r + 1]], whole["lse"][:, a:e]), (s0, r)
    assert np.array_equal(kbar.cpu().numpy(), whole["k_bar"])
    assert np.array_equal(vbar.cpu().numpy(), whole["v_bar"])


# ---------------------------------------------------------------- split-KV

@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_split_kv_parts(splits):
    """[digest] Table 7, count-balanced CSR splits: each row's items cut into
    parts of equal cost, merged by log-sum-exp; any part count gives the
    oracle's result (parts with no key leave their weight at zero)."""
    wl = synth.make_workload("llama_32k", L=2700, Hq=8, Hkv=2, n_planted=6)
    _check_full(wl, num_splits=splits)


def test_split_kv_close_to_unsplit_and_dense():
    wl = synth.make_workload("llama_32k", L=2000, Hq=4, Hkv=1, n_planted=4)
    a = run_gpu(wl, num_splits=1)
    b = run_gpu(wl, num_splits=5)
    assert np.array_equal(a["col_idx"], b["col_idx"])
    assert np.abs(a["out"] - b["out"]).max() <= 1e-2
    assert np.abs(a["lse"] - b["lse"]).max() <= 1e-4 * max(1.0, np.abs(a["lse"]).max())
    dn = run_gpu(wl, dense=True, num_splits=4)
    orc = run_oracle(wl, alpha=0.0)
    compare_outputs(dn["out"], dn["lse"], orc.O, orc.LSE, O_TOL["bf16"])


def test_split_kv_chunk_paged_fp8():
    wl = synth.make_workload("qwen4b_varlen_paged", lengths=[2900, 1500], Hq=8, Hkv=2, min_sparse_len=0,
                             page_size=48, n_planted=3)
    _check_full(synth.chunk_of(wl, 1024, 1024), num_splits=4)
    wl8 = synth.make_workload("qwen30b_128k_fp8", L=3500, Hq=16, Hkv=2, n_planted=6)
    _check_full(synth.chunk_of(wl8, 2560, 2048), num_splits=3)


# ---------------------------------------------------------------- temperature

@pytest.mark.parametrize("tau,alpha", [(1.0 / 128 ** 0.5, 0.9), (2.0, 0.3)])
def test_selection_temperature(tau, alpha):
    """sel_scale, the temperature tau of exp(tau (z - m)) >= alpha ([digest]
    abstract: max-based dynamic thresholding), other than 1, on a ragged GQA-4
    batch: the GPU's CSR must equal the oracle's at the same tau, and the
    temperature must change the selection (it is not ignored)."""
    import dataclasses
    wl = synth.make_workload("llama_32k", lengths=[3000, 5000], Hq=8, Hkv=2, n_planted=4, kind="varlen",
                             seeds_base=30, page_size=0, min_sparse_len=0, sel_scale=tau)
    assert wl.sel_scale == tau
    gpu = _check_full(wl, alpha=alpha)
    plain = run_oracle(dataclasses.replace(wl, sel_scale=1.0), alpha, do_attend=False)
    assert not np.array_equal(gpu["row_ptr"], plain.row_ptr)


# ---------------------------------------------------------------- rows longer than the column cache

_LONG = {}


def _long_rows():
    """70000 tokens of one KV head (4 query heads) in 64-token blocks: 1094
    key blocks, more than the 1024 CSR columns the attention kernel caches in
    LDS (later columns are read from global memory) and more than one
    selection tile of key blocks."""
    if not _LONG:
        wl = synth.make_workload("llama_32k", L=70000, Hq=4, Hkv=1, B=64, n_planted=30)
        _LONG["wl"] = wl
        _LONG["qkv"] = host_values(wl)
    return _LONG["wl"], _LONG["qkv"]


@pytest.mark.parametrize("num_splits,last_n", [(1, 0), (3, 0), (1, 4)])
def test_rows_beyond_the_column_cache(num_splits, last_n):
    """alpha = 0.04 keeps about 97 % of each late row's causal blocks, so the
    last rows hold up to 1082 kept blocks plus correction columns for the
    pruned ones; last_n = 4 makes the last four rows dense (1091 .. 1094
    blocks, no correction). Unsplit and split launches."""
    import math
    wl, (Q, K, V) = _long_rows()
    alpha = 0.04
    forced = dict(sink=0, window=0, last_n=last_n)
    print(f"[parity] long rows L=70000 B=64 splits={num_splits} last_n={last_n}", flush=True)
    gpu = run_gpu(wl, alpha, num_splits=num_splits, forced=forced)
    orc = run_oracle(wl, alpha, do_attend=False, Qkv=(Q, K, V), forced=forced)
    compare_pooled(gpu, orc)
    compare_csr(gpu, orc)
    counts = np.diff(gpu["row_ptr"])
    NB = len(counts)
    assert NB == 1094 and (counts > 1025).sum() >= 20
    rows = sorted({NB - 1, NB - 2, NB - 5, int(np.argmax(counts)), int(np.nonzero(counts > 1025)[0][0])})
    sets = sets_from_csr(gpu["row_ptr"], gpu["col_idx"], orc.blk_off, 1)[0][0]
    O = np.full_like(Q, np.nan)
    LSE = np.full((4, Q.shape[0]), np.nan)
    for I in rows:
        o, l = oracle.attend_row(Q, K, V, orc.kbar, orc.vbar, np.asarray(sets[I]), 0, I, 64, 4,
                                 1.0 / math.sqrt(128), True)
        O[I * 64:I * 64 + o.shape[0]] = o
        LSE[:, I * 64:I * 64 + o.shape[0]] = l.T
    o_err, l_rel, l_abs = compare_outputs(gpu["out"], gpu["lse"], O, LSE, O_TOL["bf16"])
    print(f"[parity] ok: rows {rows} cols {[int(counts[I]) for I in rows]} O_err={o_err:.2e} "
          f"LSE_rel={l_rel:.2e}", flush=True)


def test_rows_with_more_pruned_blocks_than_the_list():
    """140000 tokens of one KV head (4 query heads) in 64-token blocks: 2188
    key blocks. At alpha = 0.5 the late rows prune more than the 2048 blocks
    whose list the attention kernel keeps in LDS, so their correction chunks
    span consecutive key blocks (selected ones masked) instead of the listed
    pruned blocks; rows just below that count use the list."""
    import math
    wl = synth.make_workload("llama_32k", L=140000, Hq=4, Hkv=1, B=64, n_planted=30)
    Q, K, V = host_values(wl)
    alpha = 0.5
    print(f"[parity] pruned-list overflow L=140000 B=64 alpha={alpha}", flush=True)
    gpu = run_gpu(wl, alpha)
    orc = run_oracle(wl, alpha, do_attend=False, Qkv=(Q, K, V))
    compare_pooled(gpu, orc)
    compare_csr(gpu, orc)
    counts = np.diff(gpu["row_ptr"])
    NB = len(counts)
    pruned = np.arange(NB) - (counts - 1)
    assert NB == 2188 and (pruned > 2048).sum() >= 20 and (pruned <= 2048).sum() >= 20
    over = np.nonzero(pruned > 2048)[0]
    under = np.nonzero(pruned <= 2048)[0]
    rows = sorted({NB - 1, int(over[0]), int(under[-1]), int(np.argmax(pruned))})
    sets = sets_from_csr(gpu["row_ptr"], gpu["col_idx"], orc.blk_off, 1)[0][0]
    O = np.full_like(Q, np.nan)
    LSE = np.full((4, Q.shape[0]), np.nan)
    for I in rows:
        o, l = oracle.attend_row(Q, K, V, orc.kbar, orc.vbar, np.asarray(sets[I]), 0, I, 64, 4,
                                 1.0 / math.sqrt(128), True)
        O[I * 64:I * 64 + o.shape[0]] = o
        LSE[:, I * 64:I * 64 + o.shape[0]] = l.T
    o_err, l_rel, l_abs = compare_outputs(gpu["out"], gpu["lse"], O, LSE, O_TOL["bf16"])
    print(f"[parity] ok: rows {rows} pruned {[int(pruned[I]) for I in rows]} O_err={o_err:.2e} "
          f"LSE_rel={l_rel:.2e}", flush=True)


@pytest.mark.parametrize("page_size,L,alpha", [(16, 70000, 0.04), (6, 140000, 0.5)])
def test_paged_long_rows_equal_contiguous_bitwise(page_size, L, alpha):
    """The long-row branches (CSR columns past the LDS cache at 70000 tokens
    and alpha = 0.04; correction chunks over consecutive key blocks at 140000
    tokens and alpha = 0.5) through the paged kernels, with page sizes that
    are (16) and are not (6) multiples of 4: every output equals the
    contiguous layout's bit for bit, and the CSR the oracle's."""
    wl = synth.make_workload("llama_32k", L=L, Hq=4, Hkv=1, B=64, n_planted=30, page_size=page_size)
    print(f"[parity] paged long rows L={L} page_size={page_size} alpha={alpha}", flush=True)
    a = run_gpu(wl, alpha, paged=True)
    b = run_gpu(wl, alpha, paged=False)
    for key in ("q_bar", "k_bar", "v_bar", "row_ptr", "col_idx", "out", "lse"):
        assert np.array_equal(a[key], b[key]), key
    orc = run_oracle(wl, alpha, do_attend=False, paged=False)
    compare_pooled(a, orc)
    compare_csr(a, orc)
    counts = np.diff(a["row_ptr"])
    pruned = np.arange(len(counts)) - (counts - 1)
    if L == 70000:
        assert (counts > 1025).sum() >= 20
    else:
        assert (pruned > 2048).sum() >= 20
    print(f"[parity] ok: max kept {int(counts.max())} max pruned {int(pruned.max())}", flush=True)


_FP8_LONG = {}


@pytest.mark.parametrize("L,alpha,num_splits", [(70000, 0.04, 1), (140000, 0.5, 1), (140000, 0.5, 3)])
def test_fp8_rows_beyond_the_column_cache_and_the_pruned_list(L, alpha, num_splits):
    """The two long-row branches of the attention kernel with FP8 inputs:
    70000 tokens at alpha = 0.04 give rows of more than 1025 kept blocks (CSR
    columns past the LDS cache read from global memory); 140000 tokens at
    alpha = 0.5 give rows of more than 2048 pruned blocks (correction chunks
    over consecutive key blocks, the selected ones masked), unsplit and split.
    One KV head, 4 query heads, 64-token blocks."""
    import math
    if L not in _FP8_LONG:  # FP8 encoding of 140000 tokens takes about 17 s on the host
        w = synth.make_workload("llama_32k", L=L, Hq=4, Hkv=1, B=64, n_planted=30, fp8=True)
        _FP8_LONG.clear()
        _FP8_LONG[L] = (w, host_values(w))
    wl, (Q, K, V) = _FP8_LONG[L]
    assert wl.dtype == "fp8"
    print(f"[parity] fp8 long rows L={L} B=64 alpha={alpha} splits={num_splits}", flush=True)
    gpu = run_gpu(wl, alpha, num_splits=num_splits)
    orc = run_oracle(wl, alpha, do_attend=False, Qkv=(Q, K, V))
    compare_pooled(gpu, orc)
    compare_csr(gpu, orc)
    counts = np.diff(gpu["row_ptr"])
    NB = len(counts)
    pruned = np.arange(NB) - (counts - 1)
    if L == 70000:
        assert NB == 1094 and (counts > 1025).sum() >= 20
        rows = {NB - 1, int(np.argmax(counts)), int(np.nonzero(counts > 1025)[0][0])}
    else:
        assert NB == 2188 and (pruned > 2048).sum() >= 20 and (pruned <= 2048).sum() >= 20
        rows = {NB - 1, int(np.nonzero(pruned > 2048)[0][0]), int(np.nonzero(pruned <= 2048)[0][-1]),
                int(np.argmax(pruned))}
    rows = sorted(rows)
    sets = sets_from_csr(gpu["row_ptr"], gpu["col_idx"], orc.blk_off, 1)[0][0]
    O = np.full_like(Q, np.nan)
    LSE = np.full((4, Q.shape[0]), np.nan)
    for I in rows:
        o, l = oracle.attend_row(Q, K, V, orc.kbar, orc.vbar, np.asarray(sets[I]), 0, I, 64, 4,
                                 1.0 / math.sqrt(128), True)
        O[I * 64:I * 64 + o.shape[0]] = o
        LSE[:, I * 64:I * 64 + o.shape[0]] = l.T
    o_err, l_rel, l_abs = compare_outputs(gpu["out"], gpu["lse"], O, LSE, O_TOL["fp8"])
    print(f"[parity] ok: rows {rows} kept {[int(counts[I]) for I in rows]} pruned "
          f"{[int(pruned[I]) for I in rows]} O_err={o_err:.2e} LSE_rel={l_rel:.2e}", flush=True)


# ---------------------------------------------------------------- fused Stage 1

def test_stage1_equals_separate_calls_and_reuses_its_workspace():
    """fp_stage1 (pooling whose kernel also resets the selection workspace,
    then the selection kernel) gives bitwise the results of fp_pool_blocks
    followed by fp_select_blocks (reset kernel, then selection); and one
    selection workspace serves several calls in a row, each starting from
    what the previous call left (the look-back states are reset every call).
    Ragged chunked batch, forced keeps."""
    import block_sparse_long_fp_amd as fp
    wl = synth.make_workload("llama_32k", lengths=[3048, 2600], Hq=8, Hkv=2, n_planted=4, kind="varlen",
                             seeds_base=20, page_size=0, min_sparse_len=0)
    batch = synth.chunk_of(wl, 2048, 1000)
    forced = dict(sink=1, window=1, last_n=1)
    a = run_gpu(batch, forced=forced, fused_stage1=True)
    b = run_gpu(batch, forced=forced, fused_stage1=False)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    _check_full(batch, forced=forced)
    prob, q, k, v = upload(batch)
    bufs = fp.Buffers(prob, "cuda:0")
    sel = fp.select_args(batch.alpha, 1.0, 0, **{"sink": 1, "window": 1, "last_n": 1})
    for it in range(3):
        bufs.row_ptr.fill_(-7)
        bufs.col_idx.fill_(-7)
        if it % 2 == 0:
            fp.stage1(prob, sel, q, k, v, bufs.q_bar, bufs.k_bar, bufs.v_bar, bufs.row_ptr, bufs.col_idx,
                      bufs.workspace)
        else:
            fp.select_blocks(prob, sel, bufs.q_bar, bufs.k_bar, bufs.row_ptr, bufs.col_idx, bufs.workspace)
        torch.cuda.synchronize()
        rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
        assert np.array_equal(rp, a["row_ptr"]), it
        assert np.array_equal(bufs.col_idx[:rp[-1]].cpu().numpy().astype(np.int64), a["col_idx"]), it


def test_selection_splits_long_rows_among_workgroups():
    """4 KV heads x 1094 query blocks (70000 tokens, block 64): too few 16-row
    blocks for one selection tile per CU, so each tile's key blocks (more
    than 1024 per row) are split among two workgroups that spill their scores
    and row maxima to the workspace, the last to arrive finishing the tile.
    Pooled statistics and the CSR against the oracle; fp_stage1 against the
    separate calls."""
    wl = synth.make_workload("llama_32k", L=70000, Hq=4, Hkv=4, B=64, n_planted=30, alpha=0.3)
    a = run_gpu(wl, fused_stage1=True)
    b = run_gpu(wl, fused_stage1=False)
    for key in ("row_ptr", "col_idx", "q_bar", "k_bar"):
        assert np.array_equal(a[key], b[key]), key
    orc = run_oracle(wl, do_attend=False)
    compare_pooled(a, orc)
    n_near = compare_csr(a, orc)
    print(f"[parity] ok: nnz={a['row_ptr'][-1]} rows={len(a['row_ptr']) - 1} near_rows={n_near}", flush=True)


def test_pooling_does_not_depend_on_the_launch_shape():
    """A whole 32896-token prompt with 8 KV heads is 2056 pooling workgroups
    (256 threads each); its last 1024-query chunk pooled alone is 64 (1024
    threads each). The per-token summation order is fixed, so the chunk's
    pooled queries and its key blocks' pooled keys and values equal the whole
    prompt's bit for bit."""
    import block_sparse_long_fp_amd as fp
    wl = synth.make_workload("llama_32k", L=32896, Hq=8, Hkv=8, n_planted=8)
    whole = run_gpu(wl, num_splits=1)
    B, start, L = 128, 31872, 32896
    NB, qb0 = L // B, start // B
    dev = "cuda:0"
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    prob = fp.Problem([0, L - start], 8, 8, B, cu_seqlens_k=[0, L], pooled_pitch=NB)
    bufs = fp.Buffers(prob, dev)
    kbar = torch.zeros(8, NB, 128, device=dev)
    vbar = torch.zeros(8, NB, 128, device=dev)
    fp.pool_chunk_blocks(prob, q[start:].contiguous(), k, v, bufs.q_bar, kbar, vbar)
    torch.cuda.synchronize()
    assert np.array_equal(kbar[:, qb0:].cpu().numpy(), whole["k_bar"][:, qb0:])
    assert np.array_equal(vbar[:, qb0:].cpu().numpy(), whole["v_bar"][:, qb0:])
    assert np.array_equal(bufs.q_bar.cpu().numpy(), whole["q_bar"][:, qb0:])
