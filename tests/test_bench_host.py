"""Host logic of bench.py: the work accounting behind `roofline.achieved`, and
the one-GPU guard. No GPU is used."""
import importlib.util
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _wl(seqlens, key_seqlens, Hq=4, Hkv=2, B=16, d=8, min_sparse_len=0):
    return SimpleNamespace(seqlens=seqlens, key_seqlens=key_seqlens, num_q_heads=Hq, num_kv_heads=Hkv,
                           block_size=B, head_dim=d, min_sparse_len=min_sparse_len)


def _random_csr(wl, rng, keep=0.4):
    """Row (h, r, i) keeps the diagonal and each earlier key block with
    probability `keep`; rows are ordered head-major as the library's are."""
    B = wl.block_size
    nbq = [-(-L // B) for L in wl.seqlens]
    blk_off = np.concatenate([[0], np.cumsum(nbq)]).astype(np.int64)
    rows = []
    for h in range(wl.num_kv_heads):
        for r, (Lq, Lk) in enumerate(zip(wl.seqlens, wl.key_seqlens)):
            qb0 = (Lk - Lq) // B
            for i in range(nbq[r]):
                I = qb0 + i
                rows.append(sorted([J for J in range(I) if rng.random() < keep] + [I]))
    row_ptr = np.concatenate([[0], np.cumsum([len(x) for x in rows])]).astype(np.int64)
    col_idx = np.concatenate([np.asarray(x, dtype=np.int64) for x in rows])
    return row_ptr, col_idx, blk_off, rows


def _brute_force(wl, rows, mean_correction):
    """Multiply-adds of QK^T and PV counted pair by pair: every packed query
    row of block I against every key of each selected block (the whole tile on
    the diagonal for `computed`, the causal half for `strict`), plus one pooled
    column per pruned block when the correction is on and the request is sparse."""
    B, d, G = wl.block_size, wl.head_dim, wl.num_q_heads // wl.num_kv_heads
    computed = strict = 0
    k = 0
    for h in range(wl.num_kv_heads):
        for Lq, Lk in zip(wl.seqlens, wl.key_seqlens):
            qb0 = (Lk - Lq) // B
            for i in range(-(-Lq // B)):
                I = qb0 + i
                sel = set(rows[k])
                k += 1
                for t in range(I * B, min((I + 1) * B, Lk)):   # query positions of block I
                    for J in range(I + 1):
                        if J in sel:
                            keys = range(J * B, min((J + 1) * B, Lk))
                            computed += G * (len(keys) if J < I else min((I + 1) * B, Lk) - I * B)
                            strict += G * sum(1 for s in keys if s <= t)
                        elif mean_correction and Lq >= wl.min_sparse_len:
                            computed += G
                            strict += G
    return 4 * d * computed, 4 * d * strict


def test_csr_work_matches_a_pair_by_pair_count():
    bench = _bench()
    rng = np.random.default_rng(7)
    # a whole prompt, a chunk whose queries start at key block 3 (ragged end),
    # and a short request that runs dense (below min_sparse_len)
    wl = _wl([70, 40, 20], [70, 88, 20], min_sparse_len=30)
    row_ptr, col_idx, blk_off, rows = _random_csr(wl, rng)
    for mc in (True, False):
        flops, strict, kept, exact = bench.csr_work(row_ptr, col_idx, wl, blk_off, mc)
        bf_computed, bf_strict = _brute_force(wl, rows, mc)
        assert flops == bf_computed
        assert strict == bf_strict
        # causal (query block, key block) pairs: key blocks 0 .. I for each row
        pairs = wl.num_kv_heads * sum((Lk - Lq) // 16 + i + 1
                                      for Lq, Lk in zip(wl.seqlens, wl.key_seqlens) for i in range(-(-Lq // 16)))
        assert kept == row_ptr[-1] / pairs
    _, _, _, exact_only = bench.csr_work(row_ptr, col_idx, wl, blk_off, False)
    assert exact == exact_only


def test_csr_work_all_kept_is_dense_causal():
    """Every causal block kept and no correction: the strict count is the
    dense causal attention's 4 d Hq sum_t (positions visible to t), in closed
    form L (L + 1) / 2 per whole prompt and Lq (Lk - Lq) + Lq (Lq + 1) / 2 per
    chunk."""
    bench = _bench()
    wl = _wl([100, 37, 64], [100, 37 + 48, 64])
    row_ptr, col_idx, blk_off, _ = _random_csr(wl, np.random.default_rng(0), keep=1.0)
    _, strict, kept, _ = bench.csr_work(row_ptr, col_idx, wl, blk_off, False)
    dense = 4 * wl.head_dim * wl.num_q_heads * sum(Lq * (Lk - Lq) + Lq * (Lq + 1) // 2
                                                   for Lq, Lk in zip(wl.seqlens, wl.key_seqlens))
    assert strict == dense
    assert kept == 1.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
