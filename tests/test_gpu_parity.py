"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Sizes are small enough for the oracle to finish in seconds, yet span several
key blocks, several workgroups per (KV head, query block) and ragged tails.
Bar: bit-exact CSR outside the near-threshold band; O max-abs <= 2e-2 (bf16)
or 6e-2 (fp8); LSE |error| <= 1e-3 * max(1, |LSE|).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_common import (O_TOL, compare_csr, compare_outputs, compare_pooled, run_gpu, run_oracle,
                        sets_from_csr, host_values)
import oracle

pytestmark = pytest.mark.gpu


def _check_full(wl, alpha=None, mean_correction=True, paged=None, min_sparse_len=None, forced=None, num_splits=0):
    print(f"[parity] {wl.name} L={wl.seqlens} Lk={wl.key_seqlens} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} B={wl.block_size} "
          f"dtype={wl.dtype} alpha={alpha if alpha is not None else wl.alpha} mc={mean_correction} "
          f"paged={paged if paged is not None else wl.paged} forced={forced}", flush=True)
    gpu = run_gpu(wl, alpha, mean_correction, paged, min_sparse_len=min_sparse_len, forced=forced,
                  num_splits=num_splits)
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
                             wl.block_size, G, 1.0 / math.sqrt(wl.head_dim), mean_correction,
                             q_off=(ke - ks) - (e - s))
        O[s:e], LSE[:, s:e] = o, l
    o_err, l_err = compare_outputs(gpu["out"], gpu["lse"], O, LSE, O_TOL[wl.dtype])
    print(f"[parity] ok: nnz={gpu['row_ptr'][-1]} near_rows={n_near} O_err={o_err:.2e} LSE_err={l_err:.2e}",
          flush=True)
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


def test_fp8_gqa8():
    wl = synth.make_workload("qwen30b_128k_fp8", L=3000, Hq=16, Hkv=2, n_planted=6)
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
