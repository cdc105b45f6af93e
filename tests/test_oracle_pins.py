"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test pins one part of the oracle to mathematics or to an independent
library routine (torch's scaled_dot_product_attention in float64 on the CPU),
chosen so that a plausible slip (a dropped term, a wrong sign, a wrong index,
a missing causal mask, a wrong surrogate bias) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import fp8_e4m3_decode, fp8_e4m3_encode, make_workload

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def sdpa_with_lse(q, k, v, bias, sm):
    """Library attention plus its log-sum-exp.

    q [H, Lq, d], k/v [H, Lk, d], bias [H or 1, Lq, Lk] additive float mask.
    The LSE is recovered with one extra key of logit 0 whose value is a new
    unit coordinate: its weight is w = 1 / (1 + exp(LSE)), so
    LSE = log(1/w - 1). Only the library routine does the softmax.
    """
    H, Lq, d = q.shape
    Lk = k.shape[1]
    qt = torch.from_numpy(q)[None]
    kx = np.concatenate([k, np.zeros((H, 1, d))], axis=1)
    vx = np.concatenate([np.concatenate([v, np.zeros((H, Lk, 1))], axis=2),
                         np.concatenate([np.zeros((H, 1, d)), np.ones((H, 1, 1))], axis=2)], axis=1)
    bx = np.concatenate([np.broadcast_to(bias, (H, Lq, Lk)), np.zeros((H, Lq, 1))], axis=2)
    out = F.scaled_dot_product_attention(qt, torch.from_numpy(kx)[None], torch.from_numpy(vx)[None],
                                         attn_mask=torch.from_numpy(np.ascontiguousarray(bx))[None],
                                         scale=sm)[0].numpy()
    w = out[..., d]
    # out[..., :d] = (sum_j e^{s_j} v_j) / (e^LSE + 1); undo the extra key's share.
    o = out[..., :d] / (1.0 - w)[..., None]
    return o, np.log(1.0 / w - 1.0)


def dense_reference(Q, K, V, G, sm):
    """Causal dense attention by the library routine: O [L, Hq, d], LSE [Hq, L]."""
    L, Hq, d = Q.shape
    Kx = np.repeat(K, G, axis=1)
    Vx = np.repeat(V, G, axis=1)
    causal = np.where(np.arange(L)[None, :] <= np.arange(L)[:, None], 0.0, -np.inf)[None]
    o, lse = sdpa_with_lse(Q.transpose(1, 0, 2).copy(), Kx.transpose(1, 0, 2).copy(),
                           Vx.transpose(1, 0, 2).copy(), causal, sm)
    return o.transpose(1, 0, 2), lse


def run_oracle(Q, K, V, Hkv, B, alpha, mc=True, sel_scale=1.0):
    sm = 1.0 / math.sqrt(Q.shape[2])
    return oracle.prefill(Q, K, V, [0, Q.shape[0]], Hkv, B, alpha, sel_scale=sel_scale, sm_scale=sm,
                          mean_correction=mc)


# ---------------------------------------------------------------- pooling

def test_pool_closed_forms():
    L, Hkv, d, B = 203, 2, 4, 16
    t = np.arange(L, dtype=np.float64)
    K = np.broadcast_to(t[:, None, None], (L, Hkv, d)).copy() + np.arange(Hkv)[None, :, None] * 1000.0
    kb = oracle.pool_keys(K, B)
    NB = -(-L // B)
    assert kb.shape == (Hkv, NB, d)
    for J in range(NB):
        s, n = J * B, min(B, L - J * B)
        mid = s + (n - 1) / 2.0                       # mean of a ramp = its midpoint
        for h in range(Hkv):
            assert np.allclose(kb[h, J], mid + 1000.0 * h, rtol=0, atol=1e-12)
    # sum_J n_J * mean_J equals the total (checks the ragged last block's n_J)
    X = _rand((L, Hkv, d), 1)
    xb = oracle.pool_keys(X, B)
    nJ = np.array([n for _, n in oracle.block_bounds(L, B)], dtype=np.float64)
    assert np.allclose((xb * nJ[None, :, None]).sum(axis=1), X.sum(axis=0), atol=1e-10)
    assert oracle.block_bounds(L, B)[-1] == (192, 11)


def test_pool_queries_packs_group_heads():
    L, Hq, G, d, B = 70, 6, 3, 5, 32
    Q = np.zeros((L, Hq, d))
    for g in range(Hq):
        Q[:, g, :] = g + 1.0                         # head g holds the constant g+1
    qb = oracle.pool_queries(Q, B, G)
    for h in range(Hq // G):
        expect = np.mean([g + 1.0 for g in range(h * G, (h + 1) * G)])
        assert np.allclose(qb[h], expect)


# ---------------------------------------------------------------- P1 dense identity

@pytest.mark.parametrize("L,Hq,Hkv,d,B", [(50, 2, 1, 8, 8), (97, 4, 2, 16, 16), (64, 1, 1, 8, 64)])
def test_alpha_zero_equals_dense(L, Hq, Hkv, d, B):
    Q, K, V = _rand((L, Hq, d), 2), _rand((L, Hkv, d), 3), _rand((L, Hkv, d), 4)
    res = run_oracle(Q, K, V, Hkv, B, alpha=0.0)
    o_ref, lse_ref = dense_reference(Q, K, V, Hq // Hkv, 1.0 / math.sqrt(d))
    assert np.allclose(res.O, o_ref, atol=1e-10)
    assert np.allclose(res.LSE, lse_ref, atol=1e-10)
    # every causal block kept
    NB = -(-L // B)
    assert res.row_ptr[-1] == Hkv * NB * (NB + 1) // 2


# ---------------------------------------------------------------- P2 / P3 exact surrogates

@pytest.mark.parametrize("alpha", [0.3, 0.9, 2.0])
def test_block_size_one_is_dense_for_any_selection(alpha):
    L, Hq, Hkv, d = 40, 2, 1, 8
    Q, K, V = _rand((L, Hq, d), 5), _rand((L, Hkv, d), 6), _rand((L, Hkv, d), 7)
    res = run_oracle(Q, K, V, Hkv, 1, alpha)
    assert res.row_ptr[-1] < Hkv * L * (L + 1) // 2        # blocks really were pruned
    o_ref, lse_ref = dense_reference(Q, K, V, Hq // Hkv, 1.0 / math.sqrt(d))
    assert np.allclose(res.O, o_ref, atol=1e-10)
    assert np.allclose(res.LSE, lse_ref, atol=1e-10)
    # and without the correction it is NOT dense (the correction carries the mass)
    res_nc = run_oracle(Q, K, V, Hkv, 1, alpha, mc=False)
    assert not np.allclose(res_nc.LSE, lse_ref, atol=1e-3)


def test_constant_keys_per_block_make_correction_exact():
    L, Hq, Hkv, d, B = 90, 4, 2, 8, 8
    rng = np.random.default_rng(8)
    NB = -(-L // B)
    Kb = rng.standard_normal((NB, Hkv, d))
    K = np.repeat(Kb, B, axis=0)[:L]
    Q, V = _rand((L, Hq, d), 9), _rand((L, Hkv, d), 10)
    res = run_oracle(Q, K, V, Hkv, B, alpha=0.6)
    assert res.row_ptr[-1] < Hkv * NB * (NB + 1) // 2
    o_ref, lse_ref = dense_reference(Q, K, V, Hq // Hkv, 1.0 / math.sqrt(d))
    assert np.allclose(res.O, o_ref, atol=1e-10)
    assert np.allclose(res.LSE, lse_ref, atol=1e-10)


# ---------------------------------------------------------------- P4 augmented keys

def test_augmented_key_identity():
    L, Hq, Hkv, d, B = 77, 4, 2, 8, 8
    G = Hq // Hkv
    sm = 1.0 / math.sqrt(d)
    Q, K, V = _rand((L, Hq, d), 11), _rand((L, Hkv, d), 12), _rand((L, Hkv, d), 13)
    res = run_oracle(Q, K, V, Hkv, B, alpha=0.5)
    sets = res.sets[0]
    NB = -(-L // B)
    for h in range(Hkv):
        for I in range(NB):
            sel = [int(j) for j in sets[h][I]]
            pruned = [J for J in range(I) if J not in sel]
            qs, nI = I * B, min(B, L - I * B)
            pos = [j for J in sel for j in range(J * B, min(J * B + B, L))]
            keys = np.concatenate([K[pos, h], res.kbar[h, pruned]]) if pruned else K[pos, h]
            vals = np.concatenate([V[pos, h], res.vbar[h, pruned]]) if pruned else V[pos, h]
            bias = np.zeros((nI, len(keys)))
            for a in range(nI):
                for b, j in enumerate(pos):
                    if j > qs + a:
                        bias[a, b] = -np.inf
            for c, J in enumerate(pruned):
                bias[:, len(pos) + c] = math.log(min(B, L - J * B))
            q = Q[qs:qs + nI, h * G:(h + 1) * G].transpose(1, 0, 2).copy()
            o, lse = sdpa_with_lse(q, np.repeat(keys[None], G, 0), np.repeat(vals[None], G, 0), bias[None], sm)
            assert np.allclose(res.O[qs:qs + nI, h * G:(h + 1) * G], o.transpose(1, 0, 2), atol=1e-10)
            assert np.allclose(res.LSE[h * G:(h + 1) * G, qs:qs + nI], lse, atol=1e-10)


# ---------------------------------------------------------------- P5 Jensen ordering

def test_jensen_ordering_of_lse():
    L, Hq, Hkv, d, B = 128, 2, 1, 16, 16
    Q, K, V = _rand((L, Hq, d), 14), _rand((L, Hkv, d), 15), _rand((L, Hkv, d), 16)
    res = run_oracle(Q, K, V, Hkv, B, alpha=0.7)
    nc = run_oracle(Q, K, V, Hkv, B, alpha=0.7, mc=False)
    dn = run_oracle(Q, K, V, Hkv, B, alpha=0.0)
    eps = 1e-12
    assert np.all(nc.LSE <= res.LSE + eps)
    assert np.all(res.LSE <= dn.LSE + eps)
    assert np.any(nc.LSE < res.LSE - 1e-3) and np.any(res.LSE < dn.LSE - 1e-3)


# ---------------------------------------------------------------- P6 invariances

def test_key_shift_and_value_affinity():
    L, Hq, Hkv, d, B = 96, 4, 2, 8, 16
    G = Hq // Hkv
    sm = 1.0 / math.sqrt(d)
    Q, K, V = _rand((L, Hq, d), 17), _rand((L, Hkv, d), 18), _rand((L, Hkv, d), 19)
    c = _rand((Hkv, d), 20)
    base = run_oracle(Q, K, V, Hkv, B, alpha=0.5)
    shifted = run_oracle(Q, K + c[None], V, Hkv, B, alpha=0.5)
    assert np.array_equal(base.row_ptr, shifted.row_ptr) and np.array_equal(base.col_idx, shifted.col_idx)
    assert np.allclose(base.O, shifted.O, atol=1e-10)
    qc = np.einsum("lgd,gd->gl", Q, np.repeat(c, G, axis=0))
    assert np.allclose(shifted.LSE - sm * qc, base.LSE, atol=1e-10)
    a, b = 2.5, _rand((d,), 21)
    aff = run_oracle(Q, K, a * V + b, Hkv, B, alpha=0.5)
    assert np.allclose(aff.O, a * base.O + b, atol=1e-10)


# ---------------------------------------------------------------- P7 threshold rule

def test_threshold_nesting_and_limits():
    L, Hq, Hkv, d, B = 300, 2, 2, 8, 10
    Q, K, V = _rand((L, Hq, d), 22), _rand((L, Hkv, d), 23), _rand((L, Hkv, d), 24)
    G = Hq // Hkv
    qb, kb = oracle.pool_queries(Q, B, G), oracle.pool_keys(K, B)
    NB = qb.shape[1]
    prev = None
    for alpha in [0.0, 0.05, 0.2, 0.5, 0.9, 1.0, 1.5]:
        sets, _ = oracle.select_blocks(qb, kb, alpha, sel_scale=3.0)
        for h in range(Hkv):
            for I in range(NB):
                s = set(sets[h][I].tolist())
                assert I in s and max(s) == I and min(s) >= 0
                if alpha <= 0:
                    assert s == set(range(I + 1))
                if alpha > 1:
                    assert s == {I}
                if prev is not None:
                    assert s <= prev[h][I]
        prev = [[set(sets[h][I].tolist()) for I in range(NB)] for h in range(Hkv)]
    # alpha = 1 keeps exactly the argmax and the diagonal
    sets, _ = oracle.select_blocks(qb, kb, 1.0, sel_scale=3.0)
    for h in range(Hkv):
        for I in range(NB):
            z = kb[h, :I + 1] @ qb[h, I]
            assert set(sets[h][I].tolist()) == {int(np.argmax(z)), I}


# ---------------------------------------------------------------- P7b temperature and band

def _spread_pooled(seed, tau=1.0, Hkv=2, NB=40, d=16):
    """Pooled rows whose tempered scores tau * z spread over about 20 nats
    below the row max whatever tau, so that alphas and temperatures move many
    blocks across the threshold."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((Hkv, NB, d)), rng.standard_normal((Hkv, NB, d)) * (1.2 / tau)


def _as_sets(sets):
    return [[set(r.tolist()) for r in per_h] for per_h in sets]


@pytest.mark.parametrize("tau", [1.0 / math.sqrt(128), 0.5, 2.0, 3.0])
def test_temperature_is_a_power_of_alpha(tau):
    """For tau > 0, exp(tau (z - m)) >= alpha  <=>  exp(z - m) >= alpha^(1/tau):
    selection at temperature tau equals selection at tau = 1 with alpha
    raised to 1/tau. A tau that is dropped, applied twice, applied to the
    threshold instead of the scores, or multiplied into alpha fails this (the
    test also checks that those readings select differently on these
    inputs)."""
    qbar, kbar = _spread_pooled(40, tau)
    for alpha in (0.05, 0.3, 0.7):
        got = _as_sets(oracle.select_blocks(qbar, kbar, alpha, sel_scale=tau)[0])
        want = _as_sets(oracle.select_blocks(qbar, kbar, alpha ** (1.0 / tau), sel_scale=1.0)[0])
        assert got == want
        # the plausible slips select a different set here
        for wrong in (alpha, alpha ** (1.0 / tau ** 2), alpha * tau, alpha ** tau):
            assert _as_sets(oracle.select_blocks(qbar, kbar, wrong, sel_scale=1.0)[0]) != want


def test_temperature_scales_the_pooled_dot_product():
    """z = tau * qbar . kbar: scaling qbar by c and tau by 1/c leaves every
    decision unchanged, while scaling qbar alone changes them."""
    qbar, kbar = _spread_pooled(41)
    base = _as_sets(oracle.select_blocks(qbar, kbar, 0.3, sel_scale=1.5)[0])
    assert _as_sets(oracle.select_blocks(qbar * 4.0, kbar, 0.3, sel_scale=1.5 / 4.0)[0]) == base
    assert _as_sets(oracle.select_blocks(qbar * 4.0, kbar, 0.3, sel_scale=1.5)[0]) != base


@pytest.mark.parametrize("tau", [1.0, 0.25, 3.0])
@pytest.mark.parametrize("alpha", [0.3, 0.01])
def test_near_threshold_band_width(tau, alpha):
    """The exclusion band: a pair is listed near iff |exp(tau (z - m)) - alpha|
    <= 1e-4 alpha, and forced pairs are never listed. One row with scores
    built so that the probability ratios are exactly alpha (1 +- 5e-5)
    (inside the band: listed, kept above and pruned below) and alpha
    (1 +- 5e-4) (outside: not listed); the diagonal is forced."""
    d, I = 4, 5
    ratios = {1: alpha * (1 + 5e-5), 2: alpha * (1 - 5e-5), 3: alpha * (1 + 5e-4), 4: alpha * (1 - 5e-4),
              5: alpha * 1e-3}
    kbar = np.zeros((1, I + 1, d))
    for J, r in ratios.items():
        kbar[0, J, 0] = math.log(r) / tau     # tau * qbar . kbar - m = ln r, with m = 0 at J = 0
    qbar = np.zeros((1, I + 1, d))
    qbar[0, I, 0] = 1.0
    sets, near = oracle.select_blocks(qbar, kbar, alpha, sel_scale=tau)
    assert set(sets[0][I].tolist()) == {0, 1, 3, 5}
    assert sorted(J for (h, i, J) in near if i == I) == [1, 2]
    # the diagonal stays unlisted when its ratio sits inside the band too
    kbar[0, I, 0] = math.log(alpha * (1 - 2e-5)) / tau
    sets, near = oracle.select_blocks(qbar, kbar, alpha, sel_scale=tau)
    assert I in sets[0][I] and sorted(J for (h, i, J) in near if i == I) == [1, 2]


# ---------------------------------------------------------------- P8 planted recovery

def test_planted_recovery_tiny_workload():
    """Sanity check of the scoring reading on the single-head needle input.

    After the first planted block, every planted block left of the diagonal
    is kept (with a margin over the threshold), and non-planted blocks are
    pruned in all but a couple of rows where pooled query noise brings one
    close to the row max.
    """
    wl = make_workload("tiny_4k")
    Q, K = wl.q.double().numpy(), wl.k.double().numpy()
    B = wl.block_size
    qb, kb = oracle.pool_queries(Q, B, 1), oracle.pool_keys(K, B)
    sets, near = oracle.select_blocks(qb, kb, wl.alpha)
    planted = wl.planted[0][0]
    first = min(planted)
    la = math.log(wl.alpha)
    extra_rows = 0
    for I in range(first + 1, qb.shape[1]):
        expect = {J for J in planted if J < I} | {I}
        got = set(sets[0][I].tolist())
        assert expect <= got
        extra_rows += got != expect
        z = kb[0, :I + 1] @ qb[0, I]
        gap = z - z.max()
        on = [J for J in range(I) if J in planted]
        assert min(gap[on]) > la + 0.05
    assert extra_rows <= 2
    assert not near


# ---------------------------------------------------------------- P9 decompositions

def test_gqa_packing_equals_per_head_with_shared_selection():
    L, Hq, Hkv, d, B = 80, 4, 2, 8, 16
    G = Hq // Hkv
    sm = 1.0 / math.sqrt(d)
    Q, K, V = _rand((L, Hq, d), 25), _rand((L, Hkv, d), 26), _rand((L, Hkv, d), 27)
    res = run_oracle(Q, K, V, Hkv, B, alpha=0.4)
    sets = res.sets[0]
    for g in range(Hq):
        h = g // G
        o, lse = oracle.attend(Q[:, g:g + 1], K[:, h:h + 1], V[:, h:h + 1], res.kbar[h:h + 1],
                               res.vbar[h:h + 1], [sets[h]], B, 1, sm)
        assert np.allclose(res.O[:, g:g + 1], o, atol=1e-12)
        assert np.allclose(res.LSE[g:g + 1], lse, atol=1e-12)


def test_varlen_equals_per_request_and_paged_equals_contiguous():
    lens = [37, 64, 100]
    Hq, Hkv, d, B, ps = 4, 2, 8, 16, 8
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    T = cu[-1]
    Q, K, V = _rand((T, Hq, d), 28), _rand((T, Hkv, d), 29), _rand((T, Hkv, d), 30)
    full = oracle.prefill(Q, K, V, cu, Hkv, B, 0.5, min_sparse_len=50)
    NBt = full.blk_off[-1]
    for r, n in enumerate(lens):
        s, e = cu[r], cu[r + 1]
        one = oracle.prefill(Q[s:e], K[s:e], V[s:e], [0, n], Hkv, B, 0.5 if n >= 50 else 0.0)
        assert np.allclose(full.O[s:e], one.O, atol=1e-12)
        assert np.allclose(full.LSE[:, s:e], one.LSE, atol=1e-12)
        nb = -(-n // B)
        for h in range(Hkv):
            for I in range(nb):
                gr = h * NBt + full.blk_off[r] + I
                a, b = full.row_ptr[gr], full.row_ptr[gr + 1]
                lr = h * nb + I
                assert np.array_equal(full.col_idx[a:b], one.col_idx[one.row_ptr[lr]:one.row_ptr[lr + 1]])
    # the 37-token request is below min_sparse_len: dense rows
    for I in range(3):
        gr = 0 * NBt + 0 + I
        assert np.array_equal(full.col_idx[full.row_ptr[gr]:full.row_ptr[gr + 1]], np.arange(I + 1))
    # paged: scatter K/V into shuffled pages and read them back through the table
    import synth
    perm = np.random.default_rng(31).permutation(sum(-(-n // ps) for n in lens))
    kp, table = synth.paginate(torch.from_numpy(K), cu, ps, perm)
    vp, _ = synth.paginate(torch.from_numpy(V), cu, ps, perm)
    paged = oracle.prefill(Q, None, None, cu, Hkv, B, 0.5, min_sparse_len=50, K_pages=kp.numpy(),
                           V_pages=vp.numpy(), page_table=table.numpy(), page_size=ps)
    assert np.array_equal(paged.O, full.O) and np.array_equal(paged.col_idx, full.col_idx)


# ---------------------------------------------------------------- P10 fp8 codec

def test_fp8_codec_roundtrip_and_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8_e4m3_decode(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254 and np.nanmax(vals) == 448.0 and vals[1] == 2.0 ** -9
    back = fp8_e4m3_encode(vals[finite])
    ok = (back == codes[finite]) | ((codes[finite] == 0x80) & (back == 0))
    assert ok.all()
    x = np.random.default_rng(32).standard_normal(200000) * np.exp2(np.random.default_rng(33).uniform(-12, 8, 200000))
    x = np.clip(x, -448, 448)
    mine = fp8_e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    same = (mine == ref) | ((fp8_e4m3_decode(mine) == 0) & (fp8_e4m3_decode(ref) == 0))
    assert same.all()
    assert fp8_e4m3_encode(np.array([1e9, -1e9])).tolist() == [0x7E, 0xFE]  # saturating


# ---------------------------------------------------------------- P11 two codings

@pytest.mark.parametrize("alpha,mc", [(0.5, True), (0.5, False), (0.0, True), (0.9, True)])
def test_vectorised_and_loop_codings_agree(alpha, mc):
    L, Hq, Hkv, d, B = 45, 4, 2, 8, 8
    Q, K, V = _rand((L, Hq, d), 34), _rand((L, Hkv, d), 35), _rand((L, Hkv, d), 36)
    res = run_oracle(Q, K, V, Hkv, B, alpha, mc=mc)
    o, lse = oracle.attend_loop(Q, K, V, res.kbar, res.vbar, res.sets[0], B, Hq // Hkv, 1.0 / math.sqrt(d), mc)
    assert np.allclose(res.O, o, atol=1e-12, rtol=0)
    assert np.allclose(res.LSE, lse, atol=1e-12, rtol=0)


def test_sampled_rows_match_full_run():
    L, Hq, Hkv, d, B = 150, 4, 2, 8, 16
    Q, K, V = _rand((L, Hq, d), 37), _rand((L, Hkv, d), 38), _rand((L, Hkv, d), 39)
    full = run_oracle(Q, K, V, Hkv, B, 0.5)
    NB = -(-L // B)
    rows = [0, 3, NB - 1, NB + 4, 2 * NB - 1]
    part = oracle.prefill(Q, K, V, [0, L], Hkv, B, 0.5, rows=rows)
    for gr in rows:
        h, I = divmod(gr, NB)
        s, e = I * B, min(I * B + B, L)
        hs = slice(h * 2, h * 2 + 2)
        assert np.array_equal(part.O[s:e, hs], full.O[s:e, hs])
        assert np.array_equal(part.LSE[hs, s:e], full.LSE[hs, s:e])


@pytest.mark.parametrize("sink,window,last_n", [(2, 4, 8), (1, 0, 0), (0, 3, 0), (0, 0, 2), (40, 40, 40)])
def test_forced_keeps_rules(sink, window, last_n):
    """[article] serving flags: attention sink, local window and dense last-n
    query blocks, all counted in blocks. With alpha > 1 only forced blocks
    survive, so each row must be exactly the rule's set (built here from
    Python sets); with a real alpha the row is the unforced selection united
    with the forced set, and no forced pair is listed as near-threshold."""
    rng = np.random.default_rng(11)
    Hkv, NB, d = 2, 13, 16
    qbar = rng.standard_normal((Hkv, NB, d))
    kbar = rng.standard_normal((Hkv, NB, d))
    only, _ = oracle.select_blocks(qbar, kbar, 2.0, sink=sink, window=window, last_n=last_n)
    for h in range(Hkv):
        for I in range(NB):
            want = {I} | {J for J in range(min(sink, I + 1))} | {J for J in range(max(0, I - window), I + 1)}
            if I >= NB - last_n:
                want = set(range(I + 1))
            assert set(only[h][I].tolist()) == want, (h, I)
    plain, _ = oracle.select_blocks(qbar, kbar, 0.3)
    forced, near = oracle.select_blocks(qbar, kbar, 0.3, sink=sink, window=window, last_n=last_n)
    for h in range(Hkv):
        for I in range(NB):
            assert set(forced[h][I].tolist()) == set(plain[h][I].tolist()) | set(only[h][I].tolist())
    for h, I, J in near:
        assert J not in set(only[h][I].tolist())


# ---------------------------------------------------------------- chunked prefill

def test_chunked_alpha_zero_equals_dense_over_the_prefix():
    """A chunk's queries sit at the end of the key sequence (bottom-right causal
    alignment): with every block kept, query t of a chunk of Lq after off
    earlier positions attends to keys 0 .. off + t, which the library routine
    computes here from an explicit mask."""
    Lk, Lq, Hq, Hkv, d, B = 100, 36, 4, 2, 8, 16        # off = 64 = 4 blocks
    Q, K, V = _rand((Lq, Hq, d), 60), _rand((Lk, Hkv, d), 61), _rand((Lk, Hkv, d), 62)
    sm = 1.0 / math.sqrt(d)
    res = oracle.prefill(Q, K, V, [0, Lq], Hkv, B, 0.0, sm_scale=sm, cu_seqlens_k=[0, Lk])
    G = Hq // Hkv
    off = Lk - Lq
    mask = np.where(np.arange(Lk)[None, :] <= off + np.arange(Lq)[:, None], 0.0, -np.inf)[None]
    o, lse = sdpa_with_lse(Q.transpose(1, 0, 2).copy(), np.repeat(K, G, axis=1).transpose(1, 0, 2).copy(),
                           np.repeat(V, G, axis=1).transpose(1, 0, 2).copy(), mask, sm)
    assert np.allclose(res.O, o.transpose(1, 0, 2), atol=1e-10)
    assert np.allclose(res.LSE, lse, atol=1e-10)
    # rows of query block i hold key blocks 0 .. 4 + i
    NBq = -(-Lq // B)
    assert res.row_ptr[-1] == Hkv * sum(off // B + i + 1 for i in range(NBq))
    assert res.qbar.shape[1] == NBq and res.kbar.shape[1] == -(-Lk // B)


@pytest.mark.parametrize("alpha,mc,last_n", [(0.5, True, 0), (0.3, False, 0), (0.5, True, 2)])
def test_chunked_rows_equal_the_whole_prefill(alpha, mc, last_n):
    """Every quantity of a row depends only on its own queries and on keys at
    or before them, so the last Lq positions run as a chunk give the same
    pooled query, the same selected blocks and the same outputs as in one
    prefill of the whole sequence (the forced last-n rule counts from the end
    of the keys in both). Checked for two requests of a ragged batch."""
    Hq, Hkv, d, B = 4, 2, 8, 16
    Lks, Lqs = [150, 90], [54, 90]                      # request 0 chunked at 96, request 1 whole
    T = sum(Lks)
    Q, K, V = _rand((T, Hq, d), 63), _rand((T, Hkv, d), 64), _rand((T, Hkv, d), 65)
    sm = 1.0 / math.sqrt(d)
    cuk = [0, Lks[0], T]
    full = oracle.prefill(Q, K, V, cuk, Hkv, B, alpha, sm_scale=sm, mean_correction=mc, last_n=last_n)
    qsel = np.concatenate([np.arange(Lks[0] - Lqs[0], Lks[0]), np.arange(Lks[0], T)])
    cuq = [0, Lqs[0], Lqs[0] + Lqs[1]]
    ch = oracle.prefill(Q[qsel], K, V, cuq, Hkv, B, alpha, sm_scale=sm, mean_correction=mc, last_n=last_n,
                        cu_seqlens_k=cuk)
    assert np.array_equal(ch.O, full.O[qsel]) and np.array_equal(ch.LSE, full.LSE[:, qsel])
    assert np.array_equal(ch.kbar, full.kbar) and np.array_equal(ch.vbar, full.vbar)
    NBf, NBc = full.blk_off[-1], ch.blk_off[-1]
    qb0 = [(Lks[r] - Lqs[r]) // B for r in range(2)]
    for h in range(Hkv):
        for r in range(2):
            for i in range(ch.blk_off[r + 1] - ch.blk_off[r]):
                gc = h * NBc + ch.blk_off[r] + i
                gf = h * NBf + full.blk_off[r] + qb0[r] + i
                assert np.array_equal(ch.qbar[h, ch.blk_off[r] + i], full.qbar[h, full.blk_off[r] + qb0[r] + i])
                assert np.array_equal(ch.col_idx[ch.row_ptr[gc]:ch.row_ptr[gc + 1]],
                                      full.col_idx[full.row_ptr[gf]:full.row_ptr[gf + 1]])
    assert ch.row_ptr[-1] < full.row_ptr[-1]


def test_chunked_loop_coding_agrees():
    Lk, Lq, Hq, Hkv, d, B = 77, 29, 4, 2, 8, 8          # off = 48 = 6 blocks
    Q, K, V = _rand((Lq, Hq, d), 66), _rand((Lk, Hkv, d), 67), _rand((Lk, Hkv, d), 68)
    sm = 1.0 / math.sqrt(d)
    res = oracle.prefill(Q, K, V, [0, Lq], Hkv, B, 0.5, sm_scale=sm, cu_seqlens_k=[0, Lk])
    o, lse = oracle.attend_loop(Q, K, V, res.kbar, res.vbar, res.sets[0], B, Hq // Hkv, sm, True, q_off=Lk - Lq)
    assert np.allclose(res.O, o, atol=1e-12, rtol=0)
    assert np.allclose(res.LSE, lse, atol=1e-12, rtol=0)


def test_chunked_rejects_misaligned_chunks():
    Q, K, V = _rand((10, 2, 8), 69), _rand((30, 1, 8), 70), _rand((30, 1, 8), 71)
    with pytest.raises(ValueError):
        oracle.prefill(Q, K, V, [0, 10], 1, 8, 0.5, cu_seqlens_k=[0, 30])   # off = 20, not a multiple of 8
