"""Plain fp64 oracle of mean-corrected block-sparse causal prefill attention.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline may use it; the product path never does.

Sources (the pages this method is described on):
  [digest]  "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context
            LLM Serving", paper digest on metallab.ai (abstract, "What they
            did", Figures 3-4, Tables 7-9).
  [article] "128K context now demands Hopper hardware", nestfrontier.com
            (section "A serving setup you can actually test": the SGLang flags).
  [podcast] ResearchPod episode on FlashPrefill V2, researchpod.app (the
            block pre-scan with a simple average).

What is computed, per request of Lk key positions whose queries are the last
Lq <= Lk positions (Lq = Lk for a whole prefill; Lq < Lk is one chunk of a
chunked prefill, [digest] Table 6 and [podcast]: selection runs per chunk):

1. Blocking: NB = ceil(Lk / B) blocks; block J holds positions
   [J*B, min((J+1)*B, Lk)), n_J of them. The chunk starts at a block
   boundary, off = Lk - Lq = qb0 * B, so query block i of the chunk is block
   I = qb0 + i.
2. Pooling ([digest] Fig. 3 "pools block-mean statistics", Fig. 4 (k_J, v_J)
   means): kbar[h,J], vbar[h,J] = mean of K, V over block J; the grouped
   query heads of KV head h are packed ([digest] Fig. 3 PackGQA) and pooled
   into qbar[h,I] = mean over the G heads and the n_I tokens of block I.
3. Selection ([digest] abstract: max-based dynamic thresholding; [article]
   threshold flag: a higher threshold keeps fewer blocks):
   z_J = tau * qbar[h,I] . kbar[h,J] for J <= I, m = max_J z_J, keep J iff
   exp(z_J - m) >= alpha; the diagonal block I is always kept. alpha <= 0,
   or a request with fewer queries than the minimum sparse length, keeps
   every causal block. tau (``sel_scale``) defaults to 1.
4. Exact stream ([digest] Fig. 3 "exact path"): s_ij = sm * q_i . k_j for every
   position j <= pos(i) of a selected block.
5. Mean correction ([digest] Fig. 4): every pruned causal block J < I adds one
   surrogate logit sigma_iJ = sm * q_i . kbar_J + ln n_J with value vbar_J,
   i.e. |B_J| exp(sm q_i . kbar_J) on (vbar_J, 1) in numerator and denominator.
6. Softmax over the union of both streams ([digest] Fig. 3: the two streams
   merge in one softmax): o_i = sum(w v) / sum(w), LSE_i = max + ln sum.

Readings where the pages are silent (each is listed with its reason in the
design notes): the query of the surrogate is the per-token q_i; pooled
queries are the plain mean over the G*n_I packed rows; sm = 1/sqrt(d); the
LSE is natural-log over the full denominator including surrogates; query
block = key block = B.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np


def block_bounds(L: int, B: int) -> List[Tuple[int, int]]:
    """Step 1: (start, n_J) of every block of an L-token request."""
    return [(s, min(B, L - s)) for s in range(0, L, B)]


def pool_keys(K: np.ndarray, B: int) -> np.ndarray:
    """Step 2 for keys or values: K [L, Hkv, d] -> block means [Hkv, NB, d].

    [digest] Fig. 4: each pruned block is represented by its mean key and mean
    value.
    """
    L, Hkv, d = K.shape
    out = np.empty((Hkv, -(-L // B), d))
    for J, (s, n) in enumerate(block_bounds(L, B)):
        out[:, J, :] = K[s:s + n].mean(axis=0)
    return out


def pool_queries(Q: np.ndarray, B: int, G: int) -> np.ndarray:
    """Step 2 for queries: Q [L, Hq, d] -> [Hkv, NB, d].

    [digest] Fig. 3: queries are packed per KV head (PackGQA) before pooling;
    the pooled query of (h, I) is the mean over all G*n_I packed rows.
    """
    L, Hq, d = Q.shape
    Hkv = Hq // G
    out = np.empty((Hkv, -(-L // B), d))
    for J, (s, n) in enumerate(block_bounds(L, B)):
        blk = Q[s:s + n]                                  # [n, Hq, d]
        for h in range(Hkv):
            out[h, J, :] = blk[:, h * G:(h + 1) * G, :].mean(axis=(0, 1))
    return out


def forced_keep(I: int, NB: int, sink: int = 0, window: int = 0, last_n: int = 0) -> np.ndarray:
    """Blocks J <= I a row keeps whatever their score: the diagonal, the first
    ``sink`` blocks (attention sink), the ``window`` blocks left of the
    diagonal (local window), and every causal block when I is one of the
    request's last ``last_n`` query blocks ([article] SGLang flags
    --flashprefill-attention-sink, --flashprefill-window and
    --flashprefill-last-n-blocks; counts are in blocks)."""
    J = np.arange(I + 1)
    keep = (J == I) | (J < sink) | (J >= I - window)
    if I >= NB - last_n:
        keep[:] = True
    return keep


def select_blocks(qbar: np.ndarray, kbar: np.ndarray, alpha: float, sel_scale: float = 1.0,
                  dense: bool = False, band_rel: float = 1e-4, sink: int = 0, window: int = 0,
                  last_n: int = 0, q_block0: int = 0):
    """Step 3: per (h, i) the ascending list of kept key blocks of query block
    i, which sits at key block I = q_block0 + i (q_block0 > 0 for a chunk).

    [digest] abstract and Table 9 (alpha, "max-based dynamic thresholding");
    the diagonal is always kept, and so are the forced blocks of
    ``forced_keep`` (all off by default; NB there is the key block count).
    Returns (sets, near): sets[h][i] is an int64 array of key block ids;
    ``near`` lists (h, i, J) whose exp(z - m) lies within band_rel * alpha of
    alpha and that no rule forces, the pairs a float32 implementation may
    decide either way.
    """
    Hkv, NBq, d = qbar.shape
    NB = kbar.shape[1]
    sets: List[List[np.ndarray]] = []
    near: List[Tuple[int, int, int]] = []
    for h in range(Hkv):
        rows = []
        for i in range(NBq):
            I = q_block0 + i
            if dense or alpha <= 0.0:
                rows.append(np.arange(I + 1, dtype=np.int64))
                continue
            z = sel_scale * (kbar[h, :I + 1, :] @ qbar[h, i, :])   # [I+1]
            m = z.max()
            ratio = np.exp(z - m)
            forced = forced_keep(I, NB, sink, window, last_n)
            keep = (ratio >= alpha) | forced
            rows.append(np.nonzero(keep)[0].astype(np.int64))
            close = (np.abs(ratio - alpha) <= band_rel * alpha) & ~forced
            near.extend((h, i, int(J)) for J in np.nonzero(close)[0])
        sets.append(rows)
    return sets, near


def attend_row(Q: np.ndarray, K: np.ndarray, V: np.ndarray, kbar: np.ndarray, vbar: np.ndarray,
               sel: np.ndarray, h: int, I: int, B: int, G: int, sm_scale: float, mean_correction: bool,
               q_off: int = 0):
    """Steps 4-6 for one packed row tile (KV head h, the queries at block I).

    Q holds the queries at positions q_off .. q_off + len(Q) - 1; K, V hold
    positions 0 .. Lk - 1. Returns (o [n_I, G, d], lse [n_I, G]) for query
    heads h*G .. h*G+G-1.
    """
    L = K.shape[0]
    nI = min(B, L - I * B)
    qs = I * B - q_off                                                # row in Q
    q = Q[qs:qs + nI, h * G:(h + 1) * G, :]                          # [nI, G, d]
    # Exact stream over the positions of the selected blocks (Fig. 3 exact path).
    pos = np.concatenate([np.arange(J * B, min((J + 1) * B, L)) for J in sel])
    k_sel, v_sel = K[pos, h, :], V[pos, h, :]                         # [m, d]
    s = sm_scale * np.einsum("tgd,jd->tgj", q, k_sel)                 # [nI, G, m]
    qpos = np.arange(I * B, I * B + nI)
    s = np.where(pos[None, None, :] <= qpos[:, None, None], s, -np.inf)
    logits, values = [s], [v_sel]
    # Correction stream: one surrogate per pruned causal block (Fig. 4).
    if mean_correction:
        pruned = np.setdiff1d(np.arange(I), sel)
        if pruned.size:
            nJ = np.array([min(B, L - J * B) for J in pruned], dtype=np.float64)
            sig = sm_scale * np.einsum("tgd,jd->tgj", q, kbar[h, pruned, :]) + np.log(nJ)[None, None, :]
            logits.append(sig)
            values.append(vbar[h, pruned, :])
    z = np.concatenate(logits, axis=-1)
    vals = np.concatenate(values, axis=0)
    M = z.max(axis=-1, keepdims=True)
    w = np.exp(z - M)
    l = w.sum(axis=-1)
    o = np.einsum("tgj,jd->tgd", w, vals) / l[..., None]
    return o, M[..., 0] + np.log(l)


def attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, kbar: np.ndarray, vbar: np.ndarray,
           sets, B: int, G: int, sm_scale: float, mean_correction: bool = True,
           rows: Optional[Sequence[Tuple[int, int]]] = None, q_off: int = 0):
    """Steps 4-6 for one request: O [Lq, Hq, d], LSE [Hq, Lq].

    Queries sit at positions q_off .. (q_off a multiple of B); sets[h][i]
    belongs to query block i, key block q_off / B + i. ``rows`` restricts the
    work to some (h, i) tiles; other outputs stay NaN.
    """
    Lq, Hq, d = Q.shape
    Hkv = Hq // G
    NBq = -(-Lq // B)
    qb0 = q_off // B
    O = np.full((Lq, Hq, d), np.nan)
    LSE = np.full((Hq, Lq), np.nan)
    todo = rows if rows is not None else [(h, i) for h in range(Hkv) for i in range(NBq)]
    for h, i in todo:
        o, lse = attend_row(Q, K, V, kbar, vbar, np.asarray(sets[h][i]), h, qb0 + i, B, G, sm_scale,
                            mean_correction, q_off)
        qs = i * B
        O[qs:qs + o.shape[0], h * G:(h + 1) * G, :] = o
        LSE[h * G:(h + 1) * G, qs:qs + o.shape[0]] = lse.T
    return O, LSE


def attend_loop(Q, K, V, kbar, vbar, sets, B: int, G: int, sm_scale: float, mean_correction: bool = True,
                q_off: int = 0):
    """Second, independent coding of steps 4-6: one query token at a time.

    Walks keys one by one in plain Python (tiny shapes only) with a streaming
    max/sum, so it shares neither the vectorised layout nor the single-pass
    softmax of ``attend``. Query t sits at position q_off + t.
    """
    Lq, Hq, d = Q.shape
    L = K.shape[0]
    O = np.zeros((Lq, Hq, d))
    LSE = np.zeros((Hq, Lq))
    for g in range(Hq):
        h = g // G
        for t in range(Lq):
            i = q_off + t                     # position of the query
            I = i // B
            chosen = set(int(J) for J in sets[h][I - q_off // B])
            terms = []  # (logit, value vector)
            for J in sorted(chosen):
                for j in range(J * B, min((J + 1) * B, L)):
                    if j <= i:
                        terms.append((sm_scale * float(np.dot(Q[t, g], K[j, h])), V[j, h]))
            if mean_correction:
                for J in range(I):
                    if J not in chosen:
                        nJ = min(B, L - J * B)
                        terms.append((sm_scale * float(np.dot(Q[t, g], kbar[h, J])) + math.log(nJ), vbar[h, J]))
            m = -math.inf
            ssum = 0.0
            acc = np.zeros(d)
            for logit, val in terms:          # online max/sum, key by key
                if logit > m:
                    r = math.exp(m - logit) if m > -math.inf else 0.0
                    ssum *= r
                    acc *= r
                    m = logit
                e = math.exp(logit - m)
                ssum += e
                acc += e * val
            O[t, g] = acc / ssum
            LSE[g, t] = m + math.log(ssum)
    return O, LSE


def gather_paged(pages: np.ndarray, table_row: np.ndarray, L: int, page_size: int) -> np.ndarray:
    """Read one request's K or V [L, Hkv, d] through its page table row.

    [digest] "What they did", Fix 3, and Table 7 (paged KV with arbitrary page
    size): token t of the request lives in page table_row[t // page_size] at
    slot t % page_size.
    """
    t = np.arange(L)
    return pages[table_row[t // page_size], t % page_size]


def csr_from_sets(all_sets: List[List[List[np.ndarray]]], Hkv: int):
    """Row-major CSR over rows ordered (h, request, I), request-local columns.

    [digest] Table 7: the index is a CSR of selected blocks per KV head,
    int32 block ids.
    """
    row_ptr = [0]
    cols: List[int] = []
    for h in range(Hkv):
        for sets_r in all_sets:
            for sel in sets_r[h]:
                cols.extend(int(j) for j in sel)
                row_ptr.append(len(cols))
    return np.asarray(row_ptr, dtype=np.int64), np.asarray(cols, dtype=np.int64)


@dataclasses.dataclass
class OracleResult:
    qbar: np.ndarray            # [Hkv, NBq_tot, d]
    kbar: np.ndarray            # [Hkv, NBk_tot, d]
    vbar: np.ndarray
    row_ptr: np.ndarray         # [Hkv*NBq_tot + 1]
    col_idx: np.ndarray
    near: List[Tuple[int, int]]  # (global row, J) pairs inside the threshold band
    O: Optional[np.ndarray]     # [Tq, Hq, d]
    LSE: Optional[np.ndarray]   # [Hq, Tq]
    sets: list                  # sets[r][h][i]
    blk_off: List[int]          # query-block offsets (CSR rows, q_bar rows)
    kblk_off: List[int] = None  # key-block offsets (k_bar, v_bar rows)


def prefill(Q: np.ndarray, K: np.ndarray, V: np.ndarray, cu_seqlens: Sequence[int], num_kv_heads: int,
            B: int, alpha: float, sel_scale: float = 1.0, min_sparse_len: int = 0,
            sm_scale: Optional[float] = None, mean_correction: bool = True, do_attend: bool = True,
            rows: Optional[Sequence[int]] = None, K_pages=None, V_pages=None, page_table=None,
            page_size: int = 0, sink: int = 0, window: int = 0, last_n: int = 0,
            cu_seqlens_k: Optional[Sequence[int]] = None) -> OracleResult:
    """The whole path over a ragged batch ([digest] Fix 3: continuous batching).

    Q [Tq, Hq, d] and (contiguous) K, V [Tk, Hkv, d] hold the dequantised fp64
    values; ``cu_seqlens`` are the query offsets, ``cu_seqlens_k`` the key
    offsets (None: the same, a whole prefill); request r's queries are its last
    positions (a chunk, [digest] Table 6). With ``page_table`` given, K and V
    are instead read per request through the page table from
    ``K_pages``/``V_pages``. Requests with fewer queries than
    ``min_sparse_len`` run dense ([article] minimum sparse query length flag).
    ``rows`` limits attention to some global CSR rows (h*NBq_tot + blk_off[r] + i).
    ``sink``, ``window``, ``last_n``: forced keeps per request (``forced_keep``).
    """
    T, Hq, d = Q.shape
    Hkv = num_kv_heads
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    cuk = list(cu_seqlens) if cu_seqlens_k is None else list(cu_seqlens_k)
    R = len(cu_seqlens) - 1
    Lqs = [cu_seqlens[r + 1] - cu_seqlens[r] for r in range(R)]
    Lks = [cuk[r + 1] - cuk[r] for r in range(R)]
    for r in range(R):
        if Lks[r] < Lqs[r] or (Lks[r] - Lqs[r]) % B:
            raise ValueError(f"request {r}: the chunk must end the sequence and start on a block boundary")
    blk_off, kblk_off = [0], [0]
    for r in range(R):
        blk_off.append(blk_off[-1] + -(-Lqs[r] // B))
        kblk_off.append(kblk_off[-1] + -(-Lks[r] // B))
    NBt, NBk = blk_off[-1], kblk_off[-1]
    qbar = np.zeros((Hkv, NBt, d)); kbar = np.zeros((Hkv, NBk, d)); vbar = np.zeros((Hkv, NBk, d))
    all_sets, near = [], []
    O = np.full((T, Hq, d), np.nan) if do_attend else None
    LSE = np.full((Hq, T), np.nan) if do_attend else None
    want = None
    if rows is not None:
        want = {}
        for gr in rows:
            h, rem = divmod(int(gr), NBt)
            r = int(np.searchsorted(blk_off, rem, side="right") - 1)
            want.setdefault(r, []).append((h, rem - blk_off[r]))
    for r in range(R):
        s, e = cu_seqlens[r], cu_seqlens[r + 1]
        Lk = Lks[r]
        q_off = Lk - Lqs[r]
        q = Q[s:e]
        if page_table is not None:
            k = gather_paged(K_pages, page_table[r], Lk, page_size)
            v = gather_paged(V_pages, page_table[r], Lk, page_size)
        else:
            k, v = K[cuk[r]:cuk[r + 1]], V[cuk[r]:cuk[r + 1]]
        qb, kb, vb = pool_queries(q, B, G), pool_keys(k, B), pool_keys(v, B)
        a, b = blk_off[r], blk_off[r + 1]
        qbar[:, a:b] = qb
        kbar[:, kblk_off[r]:kblk_off[r + 1]], vbar[:, kblk_off[r]:kblk_off[r + 1]] = kb, vb
        dense = Lqs[r] < min_sparse_len
        sets, nr = select_blocks(qb, kb, alpha, sel_scale, dense=dense, sink=sink, window=window, last_n=last_n,
                                 q_block0=q_off // B)
        all_sets.append(sets)
        near.extend((h * NBt + a + i, J) for (h, i, J) in nr)
        if do_attend:
            rr = None if want is None else want.get(r, [])
            if rr is None or rr:
                o, lse = attend(q, k, v, kb, vb, sets, B, G, sm_scale, mean_correction, rows=rr, q_off=q_off)
                O[s:e] = o
                LSE[:, s:e] = lse
    row_ptr, col_idx = csr_from_sets(all_sets, Hkv)
    return OracleResult(qbar, kbar, vbar, row_ptr, col_idx, near, O, LSE, all_sets, blk_off, kblk_off)
