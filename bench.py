#!/usr/bin/env python3
"""Benchmark of one mean-corrected block-sparse causal prefill layer on MI355X.

One step = the whole hot path over one batch: Stage 1 (fp_stage1: block
pooling, then scoring + threshold + CSR) and block-sparse attention with the
fused mean correction (fp_sparse_prefill). Inputs are synthetic, seeded, and
resident in HBM before timing starts; L2 and MALL are evicted (a 512 MiB
read) before every timed step.

Default workload: the Llama-3.1-8B-shaped layer at 128K tokens (32 query / 8
KV heads, head dim 128, block 128, bf16, alpha 0.3). Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--alpha A]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "ms/layer & dense-equiv TFLOP/s at 128K causal prefill; % MFMA peak on computed FLOPs"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA peaks


def mixed_peak(flops, exact_flops, dtype):
    """Matrix-core peak of the FP8 kernel's actual mix: the kept blocks' QK^T
    (half of their FLOPs) at the FP8 rate, their PV and the correction columns
    at the bf16 rate. For bf16 inputs, the bf16 peak."""
    if dtype != "fp8" or flops <= 0:
        return PEAK_TFLOPS[dtype]
    f8 = exact_flops / 2
    return flops / (f8 / PEAK_TFLOPS["fp8"] + (flops - f8) / PEAK_TFLOPS["bf16"])
HBM_PEAK_GBS = 8000.0


# rocprofv3 HBM counters of the attention kernel are recorded in these files
# together with a hash of the kernel's sources; the benchmark reports them as
# roofline.traffic only while the sources still hash the same.
TRAFFIC_RECORDS = [os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f)
                   for f in ("attn_kernel_llama128k_bf16.md", "attn_kernel_qwen30b128k_fp8.md")]
ATTN_SOURCES = ["attn.hip", "common.h"]


def attn_source_hash():
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_sparse_long_fp_amd", "csrc")
    for name in ATTN_SOURCES:
        with open(os.path.join(d, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload, alpha):
    """HBM bytes per attention launch from the recorded FETCH_SIZE / WRITE_SIZE
    counters (KiB per dispatch, scaled by the copy-calibration factors), or None
    when no record matches this workload and the current kernel sources."""
    lines = []
    for path in TRAFFIC_RECORDS:
        try:
            with open(path) as f:
                lines += [ln.strip() for ln in f if ln.strip().startswith("traffic-record:")]
        except OSError:
            continue
    src = attn_source_hash()
    for ln in lines:
        kv = dict(tok.split("=", 1) for tok in ln.split()[1:] if "=" in tok)
        try:
            if (kv.get("source_sha256") == src and kv.get("workload") == workload
                    and abs(float(kv.get("alpha", "nan")) - alpha) < 1e-9):
                return (float(kv["fetch_kib"]) * float(kv["fetch_scale"])
                        + float(kv["write_kib"]) * float(kv["write_scale"])) * 1024.0
        except (KeyError, ValueError):
            continue
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama_128k")
    ap.add_argument("--seq-len", type=int, default=None,
                    help="override the sequence length of a single-request workload (same recipe and seed)")
    ap.add_argument("--alpha", type=float, default=None)
    ap.add_argument("--block-size", type=int, default=None, help="override the workload's block size (64 or 128)")
    ap.add_argument("--page-size", type=int, default=None,
                    help="override the KV page size in tokens (0: contiguous K / V)")
    ap.add_argument("--kv-heads", type=int, default=None,
                    help="one GPU's share under head sharding: this many KV heads (same GQA ratio)")
    ap.add_argument("--sink", type=int, default=0, help="forced keep: first key blocks of each request")
    ap.add_argument("--window", type=int, default=0, help="forced keep: key blocks left of the diagonal")
    ap.add_argument("--last-n", type=int, default=0, help="forced keep: dense last query blocks")
    ap.add_argument("--no-mean-correction", action="store_true", help="drop pruned blocks (the ablation)")
    ap.add_argument("--chunk", type=int, default=0,
                    help="chunked prefill: run the prompt as consecutive chunks of this many queries")
    ap.add_argument("--splits", type=int, default=0,
                    help="split-KV parts per attention row (0: the library's automatic choice)")
    ap.add_argument("--chunk-repool", action="store_true",
                    help="with --chunk: pool every key block so far in each chunk (no reuse)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--dense-reps", type=int, default=3, help="timed repetitions of the dense comparator")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps for this long before the dense comparator and the warm-up, so the "
                         "engine clock has settled")
    ap.add_argument("--cpu-rows", type=int, default=96,
                    help="attention rows the CPU baseline computes (96: about 10 s of oracle work at 128K)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    return ap.parse_args()


def copy_probe():
    """A plain device-to-device copy of exactly 1 GiB, three times: the reference
    dispatch for scaling FETCH_SIZE / WRITE_SIZE counter readings."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "dispatches": 3}), flush=True)


def csr_work(row_ptr, col_idx, wl, blk_off, mean_correction=True):
    """Algorithmic work of one attention launch from the CSR.

    Per selected (h, I, J): 4 * d * (G * n_I) * n_J FLOPs (QK^T and PV over the
    packed rows; full tile on the diagonal). Per pruned causal (h, I, J < I):
    4 * d * (G * n_I) FLOPs (one pooled column). Also returns the strict
    causal count (diagonal tile halved), the kept fraction over causal pairs
    and the FLOPs of the selected blocks alone.
    Query block i of a request sits at key block I = qb0 + i (qb0 > 0 for a
    chunk of a chunked prefill).
    """
    d, B = wl.head_dim, wl.block_size
    G = wl.num_q_heads // wl.num_kv_heads
    NBt = blk_off[-1]
    counts = np.diff(row_ptr)
    flops = 0.0
    strict = 0.0
    exact_flops = 0.0
    pairs = 0
    for r, (Lq, Lk) in enumerate(zip(wl.seqlens, wl.key_seqlens)):
        nb = blk_off[r + 1] - blk_off[r]
        I = (Lk - Lq) // B + np.arange(nb)
        nI = np.minimum(B, Lk - I * B).astype(np.float64)
        dense_req = Lq < wl.min_sparse_len
        for h in range(wl.num_kv_heads):
            rows = h * NBt + blk_off[r] + np.arange(nb)
            c = counts[rows].astype(np.float64)
            # every selected J < I is a full block; the diagonal is n_I x n_I
            exact = (c - 1) * nI * B + nI * nI
            flops += 4 * d * G * float(exact.sum())
            exact_flops += 4 * d * G * float(exact.sum())
            strict += 4 * d * G * float(((c - 1) * nI * B + nI * (nI + 1) / 2).sum())
            if mean_correction and not dense_req:
                pruned = I - (c - 1)
                flops += 4 * d * G * float((pruned * nI).sum())
                strict += 4 * d * G * float((pruned * nI).sum())
            pairs += int((I + 1).sum())
    kept = float(row_ptr[-1]) / float(pairs)
    return flops, strict, kept, exact_flops


def stage1_bytes(wl):
    """Algorithmic HBM bytes of pooling: read the queries and every key and value
    position once; write the pooled tensors."""
    e = 1 if wl.dtype == "fp8" else 2
    d, B = wl.head_dim, wl.block_size
    nbq = sum(-(-L // B) for L in wl.seqlens)
    nbk = sum(-(-L // B) for L in wl.key_seqlens)
    return (sum(wl.seqlens) * wl.num_q_heads + 2 * sum(wl.key_seqlens) * wl.num_kv_heads) * d * e + \
        (nbq + 2 * nbk) * wl.num_kv_heads * d * 4


def host_description():
    """Cores this process may run on, the CPU model and the BLAS numpy calls
    (vendor and thread count), for the CPU baseline record."""
    info = {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": None, "blas": None, "blas_threads": None}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    info["cpu_model"] = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = int(blas[0].get("num_threads", 0)) or None
    except Exception:  # pragma: no cover
        pass
    return info


def timing_stats(ms):
    """mean / median / min of a list of HIP-event times in ms."""
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)), "min": float(a.min())}


def cpu_baseline(wl, row_ptr, n_rows, seed=0, mean_correction=True, forced=None):
    """Time the fp64 oracle on the host (pool + select for the whole layer,
    attention for a few sampled rows, extrapolated by computed key count)."""
    import torch
    import oracle
    host = host_description()
    threads = host["blas_threads"] or host["affinity_cores"]
    t0 = time.perf_counter()
    def deq(t, s):
        x = t.to(torch.float32) if t.dtype == torch.float8_e4m3fn else t
        x = x.to(torch.float64).numpy()
        return x * s if s is not None else x
    Q, K, V = deq(wl.q, wl.descale_q), deq(wl.k, wl.descale_k), deq(wl.v, wl.descale_v)
    t_conv = time.perf_counter() - t0
    t0 = time.perf_counter()
    forced = forced or {}
    res = oracle.prefill(Q, K, V, wl.cu_seqlens, wl.num_kv_heads, wl.block_size, wl.alpha, wl.sel_scale,
                         wl.min_sparse_len, 1.0 / math.sqrt(wl.head_dim), mean_correction, do_attend=False, **forced)
    t_sel = time.perf_counter() - t0
    rng = np.random.default_rng(seed)
    nrows = len(res.row_ptr) - 1
    sample = sorted(set(int(x) for x in rng.integers(0, nrows, size=n_rows)))
    # cost of a row ~ n_I * (|S| * B + pruned): keys visited per query
    blk_off = res.blk_off
    NBt = blk_off[-1]
    def row_cost(gr):
        h, b = divmod(gr, NBt)
        r = int(np.searchsorted(blk_off, b, side="right") - 1)
        I = b - blk_off[r]
        c = res.row_ptr[gr + 1] - res.row_ptr[gr]
        dense_req = wl.seqlens[r] < wl.min_sparse_len
        return c * wl.block_size + (0 if dense_req or not mean_correction else I - (c - 1))
    total_cost = float(sum(row_cost(g) for g in range(nrows)))
    sample_cost = float(sum(row_cost(g) for g in sample))
    t0 = time.perf_counter()
    oracle.prefill(Q, K, V, wl.cu_seqlens, wl.num_kv_heads, wl.block_size, wl.alpha, wl.sel_scale,
                   wl.min_sparse_len, 1.0 / math.sqrt(wl.head_dim), mean_correction, do_attend=True, rows=sample,
                   **forced)
    t_att_sample = time.perf_counter() - t0 - t_sel   # prefill re-runs pool+select first
    t_att = max(t_att_sample, 0.0) * total_cost / max(sample_cost, 1.0)
    sec = t_sel + t_att
    return dict(value=wl.dense_equiv_flops() / sec / 1e12, unit="TFLOP/s (dense-equivalent)", cores=threads,
                kind="oracle", seconds_per_layer=sec, affinity_cores=host["affinity_cores"],
                cpu_model=host["cpu_model"], blas=host["blas"],
                sample=(f"fp64 numpy oracle: pool+select over all {nrows} rows ({t_sel:.1f} s), attention over "
                        f"{len(sample)} random rows ({t_att_sample:.1f} s) extrapolated by visited-key count to "
                        f"{t_att:.0f} s; input conversion {t_conv:.1f} s not counted"))


def run_chunked(args, wl, fp, torch, q, k, v, descales):
    """The whole prompt as consecutive chunks of ``args.chunk`` queries, each
    against every key position so far (chunked prefill: pool, select and
    attend once per chunk). A step is one pass over all chunks; the record
    has the same fields as a whole-prefill run, summed over the chunks."""
    import synth
    if len(wl.seqlens) != 1 or wl.paged:
        sys.exit("--chunk needs a single-request contiguous workload")
    L, C = wl.seqlens[0], args.chunk
    if C % wl.block_size:
        sys.exit("--chunk must be a multiple of the block size")
    starts = list(range(0, L, C))
    dt = fp.FP_FP8_E4M3 if wl.dtype == "fp8" else fp.FP_BF16
    sel = fp.select_args(wl.alpha, wl.sel_scale, wl.min_sparse_len, args.sink, args.window, args.last_n)
    att = fp.attn_args(0.0, not args.no_mean_correction, args.splits)
    NB = -(-L // wl.block_size)
    jobs = []
    for s0 in starts:
        c = min(C, L - s0)
        prob = fp.Problem([0, c], wl.num_q_heads, wl.num_kv_heads, wl.block_size, wl.head_dim, dt, descales,
                          cu_seqlens_k=[0, s0 + c], pooled_pitch=NB)
        jobs.append((s0, c, prob, fp.Buffers(prob, q.device, attn=att)))
    # one k_bar / v_bar for the whole prompt: each chunk pools only its own key
    # blocks into it (unless --chunk-repool, which pools every block so far)
    k_bar, v_bar = jobs[0][3].k_bar, jobs[0][3].v_bar
    torch.cuda.synchronize()

    def step(evs=None):
        for n, (s0, c, prob, b) in enumerate(jobs):
            ev = None if evs is None else evs[n]
            qc = q[s0:s0 + c]
            if ev is not None:
                ev[0].record()
            fp.stage1(prob, sel, qc, k, v, b.q_bar, k_bar, v_bar, b.row_ptr, b.col_idx, b.workspace,
                      chunk_only=not args.chunk_repool)
            if ev is not None:
                ev[1].record()
            fp.sparse_prefill(prob, att, qc, k, v, k_bar, v_bar, b.row_ptr, b.col_idx, b.out, b.lse,
                              b.attn_workspace)
            if ev is not None:
                ev[2].record()

    # Untimed passes for --settle-ms first, so the engine clock has settled.
    t_end = time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in jobs] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    def stage(a, b):
        return float(np.mean([sum(e[a].elapsed_time(e[b]) for e in se) for se in evs]))
    s1_ms, att_ms = stage(0, 1), stage(1, 2)
    ms = float(np.mean([se[0][0].elapsed_time(se[-1][2]) for se in evs]))
    flops = strict = 0.0
    nnz = pairs = 0
    for s0, c, prob, b in jobs:
        cw = synth.chunk_of(wl, s0, c)
        rp = b.row_ptr.cpu().numpy().astype(np.int64)
        nbq = -(-c // wl.block_size)
        f, st, _, _ = csr_work(rp, None, cw, np.array([0, nbq]), not args.no_mean_correction)
        flops, strict = flops + f, strict + st
        nnz += int(rp[-1])
        qb0 = s0 // wl.block_size
        pairs += wl.num_kv_heads * sum(qb0 + i + 1 for i in range(nbq))
    dense_eq = wl.dense_equiv_flops()
    peak = PEAK_TFLOPS[wl.dtype]
    achieved = flops / (att_ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": dense_eq / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "seq_lens": wl.seqlens, "chunk_tokens": C, "chunks": len(jobs),
                   "chunk_pooling": "repool" if args.chunk_repool else "reuse",
                   "num_splits": [fp.attn_num_splits(j[2], att) for j in jobs],
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads, "block_size": wl.block_size,
                   "alpha": wl.alpha, "mean_correction": not args.no_mean_correction,
                   "kept_fraction": nnz / max(pairs, 1), "nnz": nnz},
        "ms_per_layer": ms,
        "stages_ms": {"stage1": s1_ms, "attention": att_ms},
        "attn_mfma_frac_computed": achieved / peak,
        "attn_flops_computed": flops,
        "attn_flops_causal_strict": strict,
        "dense_equiv_flops": dense_eq,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": None, "kernel": "attn_kernel (fp_sparse_prefill)"},
        "wall_s_timed": wall,
    }
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the kernels shard by KV head "
              f"with no exchange, so a multi-GPU figure would be N independent copies of this one.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_long_fp_amd as fp
    import synth

    t0 = time.perf_counter()
    over = {} if args.alpha is None else {"alpha": args.alpha}
    if args.block_size is not None:
        over["B"] = args.block_size
    if args.kv_heads is not None:
        base = synth.CONFIGS[args.workload]
        over["Hkv"] = args.kv_heads
        over["Hq"] = args.kv_heads * (base["Hq"] // base["Hkv"])
    if args.page_size is not None:
        over["page_size"] = args.page_size
    if args.seq_len is not None:
        over["L"] = args.seq_len
        over["n_planted"] = max(1, args.seq_len // 2048)  # the recipe's one planted block per 2048 tokens
    wl = synth.make_workload(args.workload, **over)
    t_gen = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    q = wl.q.to(dev)
    if wl.paged:
        k, v, table = wl.k_pages.to(dev), wl.v_pages.to(dev), wl.page_table.to(dev)
    else:
        k, v, table = wl.k.to(dev), wl.v.to(dev), None
    descales = None
    if wl.dtype == "fp8":
        descales = [torch.tensor([s], dtype=torch.float32, device=dev) for s in
                    (wl.descale_q, wl.descale_k, wl.descale_v)]
    if args.chunk:
        run_chunked(args, wl, fp, torch, q, k, v, descales)
        return
    prob = fp.Problem(wl.cu_seqlens, wl.num_q_heads, wl.num_kv_heads, wl.block_size, wl.head_dim,
                      fp.FP_FP8_E4M3 if wl.dtype == "fp8" else fp.FP_BF16, descales, table,
                      wl.page_size, k.shape[0] if wl.paged else 0)
    att = fp.attn_args(0.0, not args.no_mean_correction, args.splits)
    bufs = fp.Buffers(prob, dev, attn=att)
    sel = fp.select_args(wl.alpha, wl.sel_scale, wl.min_sparse_len, args.sink, args.window, args.last_n)
    torch.cuda.synchronize()

    # Between timed steps a read of a 512 MiB buffer evicts L2 and the 256
    # MiB MALL, so no step starts with the previous step's data in cache; it
    # runs outside the events. A read leaves clean lines behind: the step does
    # not pay for writing back someone else's dirty lines (a 512 MiB write
    # before the step made the first kernel, pooling, 20 % slower). The buffer
    # is fp32 so that the sum reads it in place (an int32 sum first widens
    # the whole buffer to int64, a 1 GiB write).
    flush_buf = torch.ones(128 << 20, dtype=torch.float32, device=dev)

    def evict():
        flush_buf.sum()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fp.stage1(prob, sel, q, k, v, bufs.q_bar, bufs.k_bar, bufs.v_bar, bufs.row_ptr, bufs.col_idx,
                  bufs.workspace)
        if ev is not None:
            ev[1].record()
        fp.sparse_prefill(prob, att, q, k, v, bufs.k_bar, bufs.v_bar, bufs.row_ptr, bufs.col_idx, bufs.out,
                          bufs.lse, bufs.attn_workspace)
        if ev is not None:
            ev[2].record()

    # Untimed steps for --settle-ms first, so the engine clock has settled (a
    # sparse step that starts from an idle GPU measured 10.9 ms against 9.3
    # once the clock had settled, over the first four steps); warm-up steps
    # then run exactly as the timed ones. The dense comparator runs after the
    # timed steps.
    t_end = time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_end:
        evict()
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        evict()
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        evict()
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    s1_ms = [e[0].elapsed_time(e[1]) for e in evs]
    att_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    ms = float(np.mean(step_ms))

    # Stage 1 split into its pooling and selection calls (separate launches,
    # timed apart from the steps above).
    split_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(3)]
    for i in range(len(split_ev)):
        evict()
        split_ev[i][0].record()
        fp.pool_blocks(prob, q, k, v, bufs.q_bar, bufs.k_bar, bufs.v_bar)
        split_ev[i][1].record()
        fp.select_blocks(prob, sel, bufs.q_bar, bufs.k_bar, bufs.row_ptr, bufs.col_idx, bufs.workspace)
        split_ev[i][2].record()
    torch.cuda.synchronize()
    pool_ms = [e[0].elapsed_time(e[1]) for e in split_ev]
    sel_ms = [e[1].elapsed_time(e[2]) for e in split_ev]

    row_ptr = bufs.row_ptr.cpu().numpy().astype(np.int64)
    col_idx = bufs.col_idx[: int(row_ptr[-1])].cpu().numpy()
    nbs = [-(-L // wl.block_size) for L in wl.seqlens]
    blk_off = np.concatenate([[0], np.cumsum(nbs)]).astype(np.int64)
    flops, strict, kept, exact_flops = csr_work(row_ptr, col_idx, wl, blk_off, not args.no_mean_correction)
    att_avg = float(np.mean(att_ms))
    dense_eq = wl.dense_equiv_flops()
    peak = PEAK_TFLOPS[wl.dtype]
    achieved = flops / (att_avg * 1e-3) / 1e12

    dense = None
    if not args.no_dense:
        dws = fp.attn_workspace_bytes(prob, False, att)
        dws = torch.empty(dws, dtype=torch.uint8, device="cuda:0") if dws else None
        fp.dense_prefill(prob, att, q, k, v, bufs.out, bufs.lse, dws)   # warm-up
        dense_ms = []
        for i in range(args.dense_reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            evict()
            e0.record()
            fp.dense_prefill(prob, att, q, k, v, bufs.out, bufs.lse, dws)
            e1.record()
            torch.cuda.synchronize()
            dense_ms.append(e0.elapsed_time(e1))
        dense = timing_stats(dense_ms)
        dense["reps"] = len(dense_ms)

    rec = {
        "metric": METRIC,
        "value": dense_eq / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "seq_lens": wl.seqlens,
            "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim,
            "block_size": wl.block_size,
            "alpha": wl.alpha,
            "forced_keep_blocks": {"sink": args.sink, "window": args.window, "last_n": args.last_n},
            "mean_correction": not args.no_mean_correction,
            "num_splits": fp.attn_num_splits(prob, att),
            "sel_scale": wl.sel_scale,
            "min_sparse_len": wl.min_sparse_len,
            "paged": wl.paged,
            "page_size": wl.page_size,
            "kept_fraction": kept,
            "nnz": int(row_ptr[-1]),
            "csr_bytes": int(row_ptr[-1]) * 4 + len(row_ptr) * 4,
        },
        "ms_per_layer": ms,
        "ms_per_step_stats": timing_stats(step_ms),
        "stages_ms": {"stage1": float(np.mean(s1_ms)), "attention": att_avg},
        "stages_ms_stats": {"stage1": timing_stats(s1_ms), "attention": timing_stats(att_ms)},
        "steps_ms": {"step": [round(x, 4) for x in step_ms], "attention": [round(x, 4) for x in att_ms]},
        "stage1_split_ms": {"pool": timing_stats(pool_ms), "select": timing_stats(sel_ms)},
        "timing": "HIP events on the library's stream; L2 and MALL evicted (512 MiB read) before every timed "
                  "step and dense repetition, outside the events",
        "attn_mfma_frac_computed": achieved / peak,
        # FP8: against the peak of its FP8 / bf16 product mix (= frac for bf16)
        "attn_mfma_frac_mixed_peak": achieved / mixed_peak(flops, exact_flops, wl.dtype),
        "attn_flops_computed": flops,
        "attn_flops_causal_strict": strict,
        "dense_kernel_ms": None if dense is None else dense["mean"],
        "dense_kernel_ms_stats": dense,
        "dense_equiv_flops": dense_eq,
        "pool_hbm_gbs": stage1_bytes(wl) / (float(np.median(pool_ms)) * 1e-3) / 1e9,
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": recorded_traffic(args.workload, wl.alpha),
            "kernel": "attn_kernel (fp_sparse_prefill)",
        },
        "wall_s_timed": wall,
        "input_gen_s": t_gen,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] GPU timing done ({ms:.2f} ms/layer); timing the CPU oracle baseline", file=sys.stderr,
              flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, row_ptr, args.cpu_rows, mean_correction=not args.no_mean_correction,
                                           forced=dict(sink=args.sink, window=args.window, last_n=args.last_n))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
