"""Seeded synthetic long-context attention inputs ("needle" workloads).

The pages measure the operator on needle-in-a-haystack prompts fed through
real models (FlashPrefill V2 paper digest on metallab.ai, Table 1 caption and
Table 3). Neither the models nor the prompts are available here, so these
generators stand in for them: Q, K and V are Gaussian, and a few key blocks per
KV head are planted with a shared direction that the queries also carry, so a
block selector has real structure to find. Nothing here is taken from a
benchmark suite.

Recipes (the shapes follow the pages' Llama-3.1-8B and Qwen3 attention layers,
head dim 128):

* ``tiny``   one head, N=4096, block 64. Q, K, V ~ N(0,1) drawn in that
  order, K scaled by 0.5; u = unit(N(0, I)); 8 blocks chosen without
  replacement get +1.5 u on every key; every query gets +1.0 u.
* ``planted_prefill`` (multi-head): Q [L, Hq, d], K and V [L, Hkv, d] ~ N(0,1)
  drawn in that order. Then, per KV head h in order: u_h = unit(N(0, I));
  one band direction per block w_{h,J} = unit(x - (x.u_h) u_h), x ~ N(0, I);
  planted set P_h = {0} (the sink) plus ``n_planted`` distinct blocks from
  1..NB-1. Every key of block J gets +1.5 w_{h,J}, plus +1.5 u_h when J is in
  P_h. Every query of block I in the heads of group h gets +1.0 u_h and
  +1.0 w_{h,I-t} for t = 1..4 with I-t >= 0, so the 4 blocks left of the
  diagonal form a local band.

Draws are float32 from numpy's PCG64; the tensors are then rounded to bf16 by
round-to-nearest-even (torch's float32 -> bfloat16 cast). The FP8 workload
quantizes the bf16 tensors per tensor to OCP E4M3 (scale = amax / 448, codes
rounded to nearest even and saturated).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# Rounding helpers (input creation, not attention arithmetic)
# --------------------------------------------------------------------------

def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32/float64 numpy -> bf16 torch CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3 (FN variant) byte codes -> float64.

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits. Exponent 0
    is subnormal (m/8 * 2^-6). The only NaN pattern is S.1111.111; there is no
    infinity, so the largest finite value is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def _e4m3_table() -> np.ndarray:
    return fp8_e4m3_decode(np.arange(256, dtype=np.uint8))


def fp8_e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float -> OCP E4M3 codes, round to nearest (ties to even code), saturating.

    Works by searching the sorted table of the 126 finite non-negative values:
    the encoder picks the nearest representable magnitude, and on an exact tie
    the one whose code is even (even mantissa), which is round-half-even.
    Magnitudes above 448 saturate to 448.
    """
    x = np.asarray(x, dtype=np.float64)
    table = _e4m3_table()
    pos_codes = np.arange(0, 0x7F, dtype=np.int64)  # 0x00..0x7E, finite, >= 0
    pos_vals = table[pos_codes]                       # increasing
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(pos_vals, a, side="left")
    hi = np.clip(hi, 0, len(pos_vals) - 1)
    lo = np.clip(hi - 1, 0, len(pos_vals) - 1)
    d_lo = a - pos_vals[lo]
    d_hi = pos_vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (pos_codes[hi] % 2 == 0))
    code = np.where(pick_hi, pos_codes[hi], pos_codes[lo])
    code = np.where(a >= pos_vals[hi], pos_codes[hi], code)  # exact hits
    neg = (np.signbit(x)) & (code != 0)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_fp8_per_tensor(x_bf16: torch.Tensor):
    """bf16 tensor -> (float8_e4m3fn tensor, scale) with x ~= code * scale."""
    x = x_bf16.to(torch.float64).numpy()
    amax = float(np.max(np.abs(x)))
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    scale = float(np.float32(scale))  # the scale travels as a float32 scalar
    codes = fp8_e4m3_encode(x / scale)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn)
    return t, scale


# --------------------------------------------------------------------------
# Workload container
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    q: torch.Tensor                 # [T, Hq, d] bf16 or float8_e4m3fn (CPU)
    k: torch.Tensor                 # [T, Hkv, d] contiguous K
    v: torch.Tensor                 # [T, Hkv, d] contiguous V
    cu_seqlens: List[int]           # [R+1] token offsets
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    alpha: float
    sel_scale: float = 1.0
    min_sparse_len: int = 0
    descale_q: Optional[float] = None
    descale_k: Optional[float] = None
    descale_v: Optional[float] = None
    # paged KV (optional): pools [num_pages, page_size, Hkv, d], table [R, maxp]
    k_pages: Optional[torch.Tensor] = None
    v_pages: Optional[torch.Tensor] = None
    page_table: Optional[torch.Tensor] = None
    page_size: int = 0
    planted: Optional[list] = None  # per request, per KV head: planted block ids
    # chunked prefill (optional): key offsets [R+1]; q then holds only each
    # request's last queries (a chunk), k / v every key position so far
    cu_seqlens_k: Optional[List[int]] = None

    @property
    def dtype(self) -> str:
        return "fp8" if self.q.dtype == torch.float8_e4m3fn else "bf16"

    @property
    def seqlens(self) -> List[int]:
        c = self.cu_seqlens
        return [c[i + 1] - c[i] for i in range(len(c) - 1)]

    @property
    def total_tokens(self) -> int:
        return self.cu_seqlens[-1]

    @property
    def paged(self) -> bool:
        return self.page_table is not None

    @property
    def key_seqlens(self) -> List[int]:
        c = self.cu_seqlens_k or self.cu_seqlens
        return [c[i + 1] - c[i] for i in range(len(c) - 1)]

    def dense_equiv_flops(self) -> float:
        """4 * d * Hq * sum(Lq * off + Lq^2 / 2): causal dense attention FLOPs
        (QK^T and PV) of queries at the end of Lk = off + Lq keys; L^2 / 2 per
        request for a whole prefill."""
        return 4.0 * self.head_dim * self.num_q_heads * sum(
            Lq * (Lk - Lq) + Lq * Lq / 2.0 for Lq, Lk in zip(self.seqlens, self.key_seqlens))


# --------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------

def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def needle_tiny(seed: int = 0, L: int = 4096, d: int = 128, B: int = 64, n_planted: int = 8):
    """Single-head needle recipe (``tiny`` in the module docstring)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((L, 1, d), dtype=np.float32)
    k = rng.standard_normal((L, 1, d), dtype=np.float32)
    v = rng.standard_normal((L, 1, d), dtype=np.float32)
    k *= np.float32(0.5)
    u = _unit(rng.standard_normal(d)).astype(np.float32)
    NB = -(-L // B)
    planted = np.sort(rng.choice(NB, size=min(n_planted, NB), replace=False))
    for J in planted:
        k[J * B:min((J + 1) * B, L), 0, :] += np.float32(1.5) * u
    q += np.float32(1.0) * u
    return q, k, v, [[int(j) for j in planted]]


def planted_prefill(seed: int, L: int, Hq: int, Hkv: int, d: int, B: int, n_planted: int,
                    band: int = 4, key_amp: float = 1.5, q_amp: float = 1.0):
    """Multi-head planted recipe (``planted_prefill`` in the module docstring)."""
    assert Hq % Hkv == 0
    G = Hq // Hkv
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((L, Hq, d), dtype=np.float32)
    k = rng.standard_normal((L, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((L, Hkv, d), dtype=np.float32)
    NB = -(-L // B)
    blk_of_tok = np.arange(L) // B
    planted_all = []
    for h in range(Hkv):
        u = _unit(rng.standard_normal(d))
        x = rng.standard_normal((NB, d))
        w = _unit(x - (x @ u)[:, None] * u[None, :])
        n_pl = min(n_planted, NB - 1)
        extra = rng.choice(np.arange(1, NB), size=n_pl, replace=False) if n_pl > 0 else np.zeros(0, int)
        planted = np.sort(np.concatenate([[0], extra]).astype(np.int64))
        planted_all.append([int(j) for j in planted])
        is_pl = np.zeros(NB, dtype=bool)
        is_pl[planted] = True
        kadd = key_amp * w + key_amp * u[None, :] * is_pl[:, None]          # [NB, d]
        k[:, h, :] += kadd[blk_of_tok].astype(np.float32)
        qadd = np.repeat(q_amp * u[None, :], NB, axis=0)                       # [NB, d]
        for t in range(1, band + 1):
            qadd[t:] += q_amp * w[:-t] if t < NB else 0.0
        q[:, h * G:(h + 1) * G, :] += qadd[blk_of_tok][:, None, :].astype(np.float32)
    return q, k, v, planted_all


def paginate(kv: torch.Tensor, cu_seqlens: List[int], page_size: int, perm: np.ndarray):
    """Scatter a contiguous [T, Hkv, d] tensor into pages.

    Request r's local page p holds tokens [p*page_size, (p+1)*page_size) of the
    request; its physical page id is ``perm[n]`` where n counts pages in request
    order. Unused tail slots of the last page are zero. Returns
    (pages [num_pages, page_size, Hkv, d], page_table int32 [R, max_pages]
    padded with -1).
    """
    R = len(cu_seqlens) - 1
    npages = [-(-(cu_seqlens[r + 1] - cu_seqlens[r]) // page_size) for r in range(R)]
    total = sum(npages)
    assert len(perm) == total
    maxp = max(npages)
    pages = torch.zeros((total, page_size) + tuple(kv.shape[1:]), dtype=kv.dtype)
    table = torch.full((R, maxp), -1, dtype=torch.int32)
    n = 0
    for r in range(R):
        s, e = cu_seqlens[r], cu_seqlens[r + 1]
        for p in range(npages[r]):
            phys = int(perm[n])
            n += 1
            a = s + p * page_size
            b = min(a + page_size, e)
            pages[phys, : b - a] = kv[a:b]
            table[r, p] = phys
    return pages, table


def chunk_of(wl: Workload, start: int, length: int) -> Workload:
    """One chunk of a chunked prefill of a whole-prefill workload: per request,
    the queries at positions [start, min(start + length, L_r)) against keys
    [0, min(start + length, L_r)). Requests with L_r <= start drop out.
    ``start`` must be a multiple of the block size (chunks start on block
    boundaries). Contiguous K / V keep each request's key prefix; paged K / V
    keep the pools and the surviving requests' page-table rows."""
    if wl.cu_seqlens_k is not None:
        raise ValueError("already chunked")
    if start % wl.block_size:
        raise ValueError("chunks start on block boundaries")
    cu = wl.cu_seqlens
    keep = [r for r in range(len(cu) - 1) if cu[r + 1] - cu[r] > start]
    qs, ks, vs, cq, ck = [], [], [], [0], [0]
    for r in keep:
        L = cu[r + 1] - cu[r]
        end = min(start + length, L)
        qs.append(wl.q[cu[r] + start:cu[r] + end])
        ks.append(wl.k[cu[r]:cu[r] + end])
        vs.append(wl.v[cu[r]:cu[r] + end])
        cq.append(cq[-1] + end - start)
        ck.append(ck[-1] + end)
    out = dataclasses.replace(wl, q=torch.cat(qs), k=torch.cat(ks), v=torch.cat(vs), cu_seqlens=cq,
                              cu_seqlens_k=ck, planted=None)
    if wl.page_table is not None:
        out.page_table = wl.page_table[keep].contiguous()
    return out


# Named workloads. ``L`` etc. can be overridden to make smaller parity cases of
# the same recipe (same seed and structure, fewer tokens).
CONFIGS = {
    # Tiny single-head needle case (block 64, alpha 0.5).
    "tiny_4k": dict(kind="tiny", seed=0, L=4096, Hq=1, Hkv=1, d=128, B=64, n_planted=8, alpha=0.5),
    # Llama-3.1-8B-shaped layer at 32K (GQA 4, block 128, alpha 0.3).
    "llama_32k": dict(kind="planted", seed=1, L=32768, Hq=32, Hkv=8, d=128, B=128, n_planted=16, alpha=0.3),
    # Same layer at 128K, 64 planted blocks per head (alpha swept 0.1/0.3/0.5).
    "llama_128k": dict(kind="planted", seed=2, L=131072, Hq=32, Hkv=8, d=128, B=128, n_planted=64, alpha=0.3),
    # Qwen3-30B-A3B-shaped layer at 128K (GQA 8), FP8 E4M3 per-tensor.
    "qwen30b_128k_fp8": dict(kind="planted", seed=3, L=131072, Hq=32, Hkv=4, d=128, B=128, n_planted=64,
                             alpha=0.3, fp8=True),
    # Qwen3-4B-shaped continuous batch: 6 ragged requests, 64-token pages,
    # sparsity only for requests of at least 8192 tokens.
    "qwen4b_varlen_paged": dict(kind="varlen", seeds_base=100,
                                lengths=[4096, 9000, 16384, 33000, 65536, 120000],
                                Hq=32, Hkv=8, d=128, B=128, alpha=0.3, page_size=64,
                                perm_seed=5, min_sparse_len=8192),
}


def make_workload(name: str, **over) -> Workload:
    """Build a named workload; keyword overrides shrink or reshape it."""
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    kind = cfg["kind"]
    if kind == "tiny":
        q, k, v, planted = needle_tiny(cfg["seed"], cfg["L"], cfg["d"], cfg["B"], cfg["n_planted"])
        wl = Workload(name, to_bf16(q), to_bf16(k), to_bf16(v), [0, cfg["L"]], 1, 1, cfg["d"], cfg["B"],
                      cfg["alpha"], planted=[planted])
    elif kind == "planted":
        q, k, v, planted = planted_prefill(cfg["seed"], cfg["L"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["B"],
                                           cfg["n_planted"])
        wl = Workload(name, to_bf16(q), to_bf16(k), to_bf16(v), [0, cfg["L"]], cfg["Hq"], cfg["Hkv"],
                      cfg["d"], cfg["B"], cfg["alpha"], planted=[planted])
        del q, k, v
    elif kind == "varlen":
        lens = list(cfg["lengths"])
        qs, ks, vs, planted = [], [], [], []
        for r, L in enumerate(lens):
            n_pl = cfg.get("n_planted", None)
            n_pl = int(round(L / 2048)) if n_pl is None else n_pl
            q, k, v, pl = planted_prefill(cfg["seeds_base"] + r, L, cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["B"], n_pl)
            qs.append(to_bf16(q)); ks.append(to_bf16(k)); vs.append(to_bf16(v)); planted.append(pl)
        cu = [0]
        for L in lens:
            cu.append(cu[-1] + L)
        wl = Workload(name, torch.cat(qs), torch.cat(ks), torch.cat(vs), cu, cfg["Hq"], cfg["Hkv"], cfg["d"],
                      cfg["B"], cfg["alpha"], min_sparse_len=cfg.get("min_sparse_len", 0), planted=planted)
        del qs, ks, vs
    else:
        raise ValueError(kind)
    wl.min_sparse_len = cfg.get("min_sparse_len", wl.min_sparse_len)
    if "sel_scale" in cfg:
        wl.sel_scale = cfg["sel_scale"]
    if cfg.get("fp8"):
        wl.q, wl.descale_q = quantize_fp8_per_tensor(wl.q)
        wl.k, wl.descale_k = quantize_fp8_per_tensor(wl.k)
        wl.v, wl.descale_v = quantize_fp8_per_tensor(wl.v)
    ps = cfg.get("page_size", 0)
    if ps:
        R = len(wl.cu_seqlens) - 1
        total = sum(-(-(wl.cu_seqlens[r + 1] - wl.cu_seqlens[r]) // ps) for r in range(R))
        perm = np.random.default_rng(cfg.get("perm_seed", 5)).permutation(total)
        wl.k_pages, wl.page_table = paginate(wl.k, wl.cu_seqlens, ps, perm)
        wl.v_pages, _ = paginate(wl.v, wl.cu_seqlens, ps, perm)
        wl.page_size = ps
    return wl
