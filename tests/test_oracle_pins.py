"""Pins of the CPU oracle against what the pages and mathematics fix.

Every check compares the oracle with something other than itself: a closed
form, a special case that reduces to a textbook identity, a library routine
(LAPACK SVD, scipy logsumexp, torch SDPA), or brute force on tiny inputs.
Each is chosen so that a plausible slip (a dropped term, a wrong sign or
scale, a transposed operand, a wrong index) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def _page(P, d, rank=None, offset=0.0, seed=0):
    g = np.random.default_rng(seed)
    if rank is None:
        K = g.standard_normal((P, d))
    else:
        K = g.standard_normal((P, rank)) @ g.standard_normal((rank, d))
    return K + offset * g.standard_normal(d)


# ---------------------------------------------------------------- log-sum-exp

def test_lse_closed_forms(orc):
    n = 37
    x = np.log(np.arange(1, n + 1, dtype=np.float64))
    assert orc.lse(x) == pytest.approx(math.log(n * (n + 1) / 2), rel=0, abs=1e-13)
    # overflow safety: exp(1000) overflows a double, the LSE does not
    assert orc.lse([1000.0, 1000.0]) == pytest.approx(1000.0 + math.log(2.0), abs=1e-12)
    assert orc.lse([-np.inf, -np.inf]) == -np.inf
    assert orc.lse([]) == -np.inf
    assert orc.lse([-np.inf, 0.0]) == 0.0


def test_exact_page_lse_worked_example(orc):
    """Closed form: with q = (sqrt(d), 0, ...) the logit of token i is its first
    coordinate; first coordinates log(1..P) give LSE = log(P(P+1)/2).  Pins the
    1/sqrt(d) scale of the logits."""
    with open(os.path.join(GOLDEN, "exact_lse_worked_example.json")) as f:
        g = json.load(f)
    q, keys = np.array(g["q"]), np.array(g["keys"])
    assert orc.page_exact_lse(q, keys) == pytest.approx(g["expected"], abs=1e-13)
    P = keys.shape[0]
    assert g["expected"] == pytest.approx(math.log(P * (P + 1) / 2), abs=1e-15)


# ---------------------------------------------------------------- summaries

@pytest.mark.parametrize("P,d,r", [(16, 64, 4), (16, 64, 16), (64, 128, 8), (64, 32, 8),
                                   (64, 128, 2), (8, 8, 8)])
def test_summary_singular_values_match_lapack(orc, P, d, r):
    K = _page(P, d, seed=P * 1000 + d + r)
    mu, basis, coef, sigma, sweeps = orc.page_summary(K, r)
    np.testing.assert_allclose(mu, K.mean(axis=0), rtol=0, atol=1e-14)
    Kc = K - K.mean(axis=0)
    s_ref = np.linalg.svd(Kc, compute_uv=False)
    n = min(P, d)
    # the centred block has rank <= P - 1: its last value is ~0 when P <= d
    np.testing.assert_allclose(sigma[:n], s_ref[:n], rtol=1e-12, atol=1e-12 * s_ref[0])
    assert 0 < sweeps < 100


@pytest.mark.parametrize("P,d,r", [(16, 64, 4), (64, 128, 8), (64, 32, 8), (32, 64, 1)])
def test_summary_eckart_young(orc, P, d, r):
    """Residual-optimality of the page basis (section 3, Retentiegaranties):
    ||Kc - C V||_F^2 equals the tail energy sum_{k>=r} sigma_k^2; V has
    orthonormal rows; C = Kc V^T."""
    K = _page(P, d, offset=3.0, seed=7 * P + d)
    mu, basis, coef, sigma, _ = orc.page_summary(K, r)
    Kc = K - mu
    resid = np.linalg.norm(Kc - coef @ basis) ** 2
    tail = np.sum(np.linalg.svd(Kc, compute_uv=False)[r:] ** 2)
    assert resid == pytest.approx(tail, rel=1e-10, abs=1e-10)
    np.testing.assert_allclose(basis @ basis.T, np.eye(r), atol=1e-12)
    np.testing.assert_allclose(coef, Kc @ basis.T, atol=1e-12)


def test_summary_subspace_matches_lapack_projector(orc):
    """With a clear spectral gap the top-r subspace is unique: the projector
    V^T V must equal LAPACK's (sign and rotation free)."""
    P, d, r = 64, 128, 8
    g = np.random.default_rng(3)
    Q = np.linalg.qr(g.standard_normal((d, 12)))[0]
    Z = g.standard_normal((P, 12)) * (2.0 ** -np.arange(12))
    K = Z @ Q.T + 1e-3 * g.standard_normal((P, d))
    mu, basis, coef, sigma, _ = orc.page_summary(K, r)
    _, s, vt = np.linalg.svd(K - K.mean(0))
    np.testing.assert_allclose(basis.T @ basis, vt[:r].T @ vt[:r], atol=1e-9)


def test_summary_null_direction_is_zero(orc):
    """After centring, a P-token block has rank <= P - 1: at r = P <= d the
    last direction is null and is emitted as zero."""
    K = _page(8, 32, seed=11)
    mu, basis, coef, sigma, _ = orc.page_summary(K, 8)
    assert sigma[-1] < 1e-12 * sigma[0]
    assert not basis[-1].any() and not coef[:, -1].any()


def test_summary_rank_bounds(orc):
    K = _page(16, 64)
    with pytest.raises(ValueError):
        orc.page_summary(K, 17)
    with pytest.raises(ValueError):
        orc.page_summary(K, -1)


# ---------------------------------------------------------------- the estimator

@pytest.mark.parametrize("P,d", [(16, 64), (64, 128), (64, 32)])
def test_estimate_full_rank_equals_exact_lse(orc, P, d):
    """At r = min(P, d) the reconstruction is exact, so the estimate of the
    displayed equation (section 2) equals the exact page LSE: the exact-LSE
    selection that reads every key."""
    K = _page(P, d, offset=1.0, seed=P + d)
    q = np.random.default_rng(d).standard_normal(d) / math.sqrt(d) * 4
    mu, basis, coef, _, _ = orc.page_summary(K, min(P, d))
    assert orc.page_estimate(q, mu, basis, coef) == pytest.approx(orc.page_exact_lse(q, K),
                                                                  abs=1e-12)


def test_estimate_exact_on_low_rank_page(orc):
    """Keys inside mu + span(r directions): rank r already reconstructs them."""
    P, d, r = 64, 128, 5
    K = _page(P, d, rank=r, offset=2.0, seed=5)
    q = np.random.default_rng(9).standard_normal(d)
    mu, basis, coef, _, _ = orc.page_summary(K, r)
    assert orc.page_estimate(q, mu, basis, coef) == pytest.approx(orc.page_exact_lse(q, K),
                                                                  abs=1e-11)
    # rank r - 1 is not exact on such a page
    mu, basis, coef, _, _ = orc.page_summary(K, r - 1)
    assert abs(orc.page_estimate(q, mu, basis, coef) - orc.page_exact_lse(q, K)) > 1e-6


def test_estimate_rank_zero_closed_form(orc):
    """r = 0: every reconstructed logit is q.mu/sqrt(d), so the estimate is
    q.mu/sqrt(d) + log P (pins the centroid term and the log P count)."""
    P, d = 16, 64
    K = _page(P, d, offset=2.0, seed=2)
    q = np.random.default_rng(4).standard_normal(d)
    mu, basis, coef, _, _ = orc.page_summary(K, 0)
    expect = float(q @ K.mean(0)) / math.sqrt(d) + math.log(P)
    assert orc.page_estimate(q, mu, basis, coef) == pytest.approx(expect, abs=1e-12)


def test_estimate_sign_invariance(orc):
    """Flipping the sign of (v_k, c_k) leaves the estimate unchanged."""
    P, d, r = 64, 128, 8
    K = _page(P, d, seed=21)
    q = np.random.default_rng(5).standard_normal(d)
    mu, basis, coef, _, _ = orc.page_summary(K, r)
    a = orc.page_estimate(q, mu, basis, coef)
    flip = np.where(np.arange(r) % 3 == 0, -1.0, 1.0)
    b = orc.page_estimate(q, mu, basis * flip[:, None], coef * flip[None, :])
    assert a == pytest.approx(b, abs=1e-13)


def test_estimate_sees_centroid_shift(orc):
    """Shifting every key by s shifts every logit by q.s/sqrt(d)."""
    P, d, r = 16, 64, 4
    K = _page(P, d, seed=8)
    s = np.random.default_rng(1).standard_normal(d)
    q = np.random.default_rng(2).standard_normal(d)
    e1 = orc.page_estimate(q, *orc.page_summary(K, r)[:3])
    e2 = orc.page_estimate(q, *orc.page_summary(K + s, r)[:3])
    assert e2 - e1 == pytest.approx(float(q @ s) / math.sqrt(d), abs=1e-12)


# ---------------------------------------------------------------- paged drivers

def _small_layout(wl, orc, **kw):
    spec = wl.config(0).with_(**kw)
    layer = wl.make(spec)
    lay = orc.Layout(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                     layer.block_table, layer.seq_lens)
    return spec, layer, lay


def _tokens(layer, spec, b, g, pool):
    """All valid tokens of (b, g) in logical order (test-side gather)."""
    P = spec.page_size
    n = int(layer.seq_lens[b])
    rows = []
    for j in range(-(-n // P)):
        blk = layer.block_table[b, j]
        valid = min(P, n - j * P)
        rows.append(pool[blk, g, :valid])
    return np.concatenate(rows).astype(np.float64)


def test_exact_pages_compose_to_row_lse(wl, orc):
    """LSE over pages of the exact page LSEs = LSE over all tokens (scipy)."""
    spec, layer, lay = _small_layout(wl, orc, seq_lens=[1000, 333], batch=2, num_q_heads=4,
                                     num_kv_heads=2, carriers=2)
    head, page = orc.exact_pool(lay, layer.q, layer.k_f32())
    K = layer.k_f32()
    G = spec.group
    for b in range(2):
        for h in range(4):
            toks = _tokens(layer, spec, b, h // G, K)
            row = logsumexp(toks @ layer.q[b, h].astype(np.float64) / math.sqrt(spec.head_dim))
            np.testing.assert_allclose(logsumexp(head[b, h][np.isfinite(head[b, h])]), row,
                                       atol=1e-12)
        for g in range(2):
            np.testing.assert_allclose(page[b, g], logsumexp(head[b, g * G:(g + 1) * G], axis=0),
                                       atol=1e-12)


def test_scan_group_aggregation(wl, orc):
    """Group mass = LSE over the group's heads (heads h with h // G == g);
    identical heads give estimate + log G; G = 1 is the identity."""
    spec, layer, lay = _small_layout(wl, orc, num_q_heads=6, num_kv_heads=2, rank=3)
    mu, basis, coef = orc.build_pool(lay, spec.rank, layer.k_f32(), spec.num_blocks)
    head, page = orc.scan_pool(lay, spec.rank, layer.q, mu, basis, coef)
    f = spec.seq_lens[0] // spec.page_size
    np.testing.assert_allclose(page[0, :, :f], logsumexp(head[0].reshape(2, 3, -1), axis=1)[:, :f],
                               atol=1e-12)
    assert np.all(page[0, :, f:] == -np.inf)
    q_same = np.repeat(layer.q[:, :1], 6, axis=1)
    head2, page2 = orc.scan_pool(lay, spec.rank, q_same, mu, basis, coef)
    np.testing.assert_allclose(page2[0, :, :f], head2[0, ::3, :f] + math.log(3), atol=1e-12)
    spec1, layer1, lay1 = _small_layout(wl, orc)
    mu, basis, coef = orc.build_pool(lay1, spec1.rank, layer1.k_f32(), spec1.num_blocks)
    h1, p1 = orc.scan_pool(lay1, spec1.rank, layer1.q, mu, basis, coef)
    np.testing.assert_array_equal(h1, p1)


def test_scan_pool_full_rank_equals_exact_pool_on_shuffled_layout(wl, orc):
    """Paged indexing of the scan.  At r = min(P, d) the displayed estimator
    (technical summary, section 2, Reconstructie en Selectie) reduces to the
    exact page LSE, so on a shuffled block table, with two sequences (one
    ragged), two KV heads, three query heads per group, a distinct query per
    head and per-page centroid offsets, scan_pool must return exact_pool's
    values per head and per group.  exact_pool is pinned above against scipy
    over tokens gathered through the block table with head h in group h // G,
    so a wrong head -> group map, a head's output written to another head's
    row, or a unit read from the wrong physical block fails here by orders
    of magnitude more than the fp32 rounding of the summaries."""
    lens = [16 * 21 + 5, 16 * 13]
    spec, layer, lay = _small_layout(wl, orc, seq_lens=lens, batch=2, num_q_heads=6,
                                     num_kv_heads=2, carriers=2, page_offset_std=1.0)
    P, d, G = spec.page_size, spec.head_dim, spec.group
    r = min(P, d)
    K = layer.k_f32()
    assert G == 3
    # the layout is really shuffled: physical block != logical position
    assert np.count_nonzero(layer.block_table[0, :lens[0] // P] != np.arange(lens[0] // P)) > 10
    mu, basis, coef = orc.build_pool(lay, r, K, spec.num_blocks)
    head, page = orc.scan_pool(lay, r, layer.q, mu, basis, coef)
    ehead, epage = orc.exact_pool(lay, layer.q, K)
    for b in range(2):
        f = lens[b] // P
        np.testing.assert_allclose(head[b, :, :f], ehead[b, :, :f], rtol=0, atol=1e-6)
        np.testing.assert_allclose(page[b, :, :f], epage[b, :, :f], rtol=0, atol=1e-6)
        assert np.all(head[b, :, f:] == -np.inf) and np.all(page[b, :, f:] == -np.inf)
    # the inputs separate every alternative map: heads, groups and pages differ
    f0 = lens[0] // P
    for h in range(1, 6):
        assert np.abs(ehead[0, 0, :f0] - ehead[0, h, :f0]).max() > 1e-2
    assert np.abs(epage[0, 0, :f0] - epage[0, 1, :f0]).max() > 1e-2
    assert np.abs(np.diff(epage[0, 0, :f0])).min() > 1e-6


def test_mean_share_reads_each_groups_own_heads(orc):
    """Head -> group map of the mean-of-share scores (technical summary,
    section 2, Group-Shared Selection), on a case with a known answer.  Each
    query head h puts all of its estimated mass, in equal parts, on its own
    set S_h of pages (the sets are disjoint), plus an arbitrary per-head
    shift that the share removes.  The share of head h is then 1/|S_h| on S_h
    and 0 elsewhere, so group g's mean share is 1 / (G |S_h|) on the pages of
    its own heads h (h // G == g) and 0 (log: -inf) on every other page.  A
    second case compares random per-head estimates with a numpy mean share
    built over the heads h with h // G == g."""
    B, Hq, Hkv, P, MP = 2, 6, 2, 16, 40
    G = Hq // Hkv
    lens = [16 * 40, 16 * 37 + 9]
    lay = _share_layout(orc, B, Hq, Hkv, P, lens, MP)
    g_rng = np.random.default_rng(21)
    hm = np.full((B, Hq, MP), -np.inf)
    expect = np.full((B, Hkv, MP), -np.inf)
    for b in range(B):
        f = lens[b] // P
        owner = g_rng.permutation(np.arange(f) % Hq)  # page -> the head that owns it
        for h in range(Hq):
            S = np.flatnonzero(owner == h)
            hm[b, h, S] = 4.0 * h - 7.0  # equal parts, then a per-head shift
            expect[b, h // G, S] = -math.log(G * S.size)
    sh = orc.share_pool(lay, hm)
    np.testing.assert_array_equal(np.isneginf(sh), np.isneginf(expect))
    fin = np.isfinite(expect)
    np.testing.assert_allclose(sh[fin], expect[fin], rtol=0, atol=1e-12)

    hm = _random_heads(B, Hq, MP, lens, P, 22) + g_rng.normal(0, 3, (B, Hq, 1))
    ref = np.full((B, Hkv, MP), -np.inf)
    for b in range(B):
        f = lens[b] // P
        for g in range(Hkv):
            heads = [h for h in range(Hq) if h // G == g]
            shares = [np.exp(hm[b, h, :f] - logsumexp(hm[b, h, :f])) for h in heads]
            ref[b, g, :f] = np.log(np.mean(shares, axis=0))
    sh = orc.share_pool(lay, hm)
    np.testing.assert_array_equal(np.isneginf(sh), np.isneginf(ref))
    fin = np.isfinite(ref)
    np.testing.assert_allclose(sh[fin], ref[fin], rtol=0, atol=1e-12)


def _share_layout(orc, B, Hq, Hkv, P, lens, MP):
    bt = np.arange(B * MP, dtype=np.int32).reshape(B, MP)
    return orc.Layout(Hq, Hkv, 8, P, bt, np.asarray(lens, np.int32))


def _random_heads(B, Hq, MP, lens, P, seed):
    g = np.random.default_rng(seed)
    hm = g.normal(3.0, 2.0, (B, Hq, MP))
    for b in range(B):
        hm[b, :, lens[b] // P:] = -np.inf
    return hm


def test_mean_share_sums_to_one_and_ignores_head_shifts(orc):
    """Mean-of-share scores (technical summary, section 2, Group-Shared
    Selection): every head's shares over the full pages sum to 1, so their
    mean does too; a per-head shift of the estimates cancels in the share
    (while the LSE aggregation would move); non-full pages are -inf."""
    B, Hq, Hkv, P, MP = 2, 8, 2, 16, 50
    lens = [16 * 50, 16 * 31 + 5]
    lay = _share_layout(orc, B, Hq, Hkv, P, lens, MP)
    hm = _random_heads(B, Hq, MP, lens, P, 7)
    sh = orc.share_pool(lay, hm)
    for b in range(B):
        f = lens[b] // P
        np.testing.assert_allclose(np.exp(sh[b, :, :f]).sum(axis=-1), 1.0, atol=1e-12)
        assert np.all(sh[b, :, f:] == -np.inf)
    shift = np.random.default_rng(8).normal(0, 5, (1, Hq, 1))
    sh2 = orc.share_pool(lay, hm + shift)
    fin = np.isfinite(sh)
    np.testing.assert_allclose(sh2[fin], sh[fin], atol=1e-12)


def test_mean_share_special_cases(orc):
    """G = 1: the share is the head's estimate minus its total (a shift), so
    the selection equals the LSE-aggregation selection.  Identical heads: the
    mean share is each head's share."""
    B, P, MP = 1, 16, 40
    lens = [16 * 40]
    lay1 = _share_layout(orc, B, 2, 2, P, lens, MP)
    hm = _random_heads(B, 2, MP, lens, P, 9)
    sh = orc.share_pool(lay1, hm)
    for h in range(2):
        np.testing.assert_allclose(sh[0, h], hm[0, h] - logsumexp(hm[0, h]), atol=1e-12)
    sel_share, _ = orc.select_pool(lay1, 16 * 8, sh.astype(np.float32), 8)
    sel_lse, _ = orc.select_pool(lay1, 16 * 8, (hm - logsumexp(hm, axis=-1, keepdims=True))
                                 .astype(np.float32), 8)
    np.testing.assert_array_equal(sel_share, sel_lse)
    lay4 = _share_layout(orc, B, 4, 1, P, lens, MP)
    one = _random_heads(B, 1, MP, lens, P, 10)
    sh4 = orc.share_pool(lay4, np.repeat(one, 4, axis=1))
    np.testing.assert_allclose(sh4[0, 0], one[0, 0] - logsumexp(one[0, 0]), atol=1e-12)


def test_scan_full_rank_equals_exact(wl, orc):
    """Pool-level P1 on the tiny workload at r = min(P, d) = 16, with the
    summaries kept in double (build_units) so only rounding remains."""
    spec, layer, lay = _small_layout(wl, orc)
    f = spec.seq_lens[0] // spec.page_size
    units = np.array([[0, 0, j] for j in range(f)], np.int32)
    mu, basis, coef, sigma = orc.build_units(lay, 16, layer.k_f32(), units)
    _, exact = orc.exact_pool(lay, layer.q, layer.k_f32())
    for u in range(f):
        est = orc.page_estimate(layer.q[0, 0], mu[u], basis[u], coef[u])
        assert est == pytest.approx(exact[0, 0, u], abs=1e-12)


def test_build_pool_matches_units(wl, orc):
    spec, layer, lay = _small_layout(wl, orc, seq_lens=[200, 70], batch=2, carriers=1)
    mu, basis, coef, sig = orc.build_pool(lay, spec.rank, layer.k_f32(), spec.num_blocks,
                                          with_sigma=True)
    units = np.array([[b, 0, j] for b in range(2) for j in range(spec.seq_lens[b] // 16)],
                     np.int32)
    mu_u, basis_u, coef_u, sig_u = orc.build_units(lay, spec.rank, layer.k_f32(), units)
    for n, (b, g, j) in enumerate(units):
        blk = layer.block_table[b, j]
        np.testing.assert_array_equal(sig[blk, g], sig_u[n])
        np.testing.assert_array_equal(mu[blk, g], mu_u[n].astype(np.float32))
        np.testing.assert_array_equal(basis[blk, g], basis_u[n].astype(np.float32))
        np.testing.assert_array_equal(coef[blk, g], coef_u[n].astype(np.float32))


# ---------------------------------------------------------------- selection

def _brute_topk(mass, k):
    order = sorted(range(len(mass)), key=lambda j: (-float(mass[j]), j))
    return sorted(order[:k])


@pytest.mark.parametrize("trial", range(40))
def test_select_matches_brute_force(orc, trial):
    g = np.random.default_rng(trial)
    n = int(g.integers(0, 70))
    # few distinct values -> many exact ties
    levels = g.standard_normal(max(1, int(g.integers(1, 6)))).astype(np.float32)
    mass = levels[g.integers(0, levels.size, n)] if trial % 2 else \
        g.standard_normal(n).astype(np.float32)
    if n and trial % 5 == 0:
        mass[g.integers(0, n)] = -np.inf
    k = int(g.integers(0, 80))
    width = max(k, 1) + int(g.integers(0, 3))
    sel, sm, kk = orc.select_topk(mass, k, width)
    ref = _brute_topk(mass, min(k, n))
    assert kk == len(ref)
    assert list(sel[:kk]) == ref
    assert np.all(sel[kk:] == -1) and np.all(sm[kk:] == -np.inf)
    np.testing.assert_array_equal(sm[:kk], mass[ref])


def test_select_matches_numpy_stable_sort(orc):
    mass = np.round(np.random.default_rng(0).standard_normal(5000), 1).astype(np.float32)
    sel, _, _ = orc.select_topk(mass, 300)
    ref = np.sort(np.argsort(-mass, kind="stable")[:300])
    np.testing.assert_array_equal(sel, ref)


def test_select_pool_budget_rules(wl, orc):
    """k = floor(budget / P) pages, at most the full pages; the partial last
    page is never a candidate; a budget below one page selects nothing."""
    spec, layer, lay = _small_layout(wl, orc, seq_lens=[100], carriers=1)
    pm = np.zeros((1, 1, spec.max_pages), np.float32)
    pm[0, 0, :] = np.arange(spec.max_pages, dtype=np.float32)  # the tail page would win
    sel, sm = orc.select_pool(lay, 10 * 16, pm, 10)
    assert list(sel[0, 0]) == [0, 1, 2, 3, 4, 5, -1, -1, -1, -1]  # 6 full pages of 7
    sel, _ = orc.select_pool(lay, 3 * 16 + 15, pm, 3)
    assert list(sel[0, 0]) == [3, 4, 5]
    sel, _ = orc.select_pool(lay, 15, pm, 1)
    assert list(sel[0, 0]) == [-1]


# ---------------------------------------------------------------- attention

def _sdpa_ref(q, K, V):
    """torch's scaled-dot-product attention (CPU, float64) for one query."""
    qt = torch.from_numpy(np.asarray(q, np.float64)).view(1, 1, 1, -1)
    kt = torch.from_numpy(np.asarray(K, np.float64)).view(1, 1, K.shape[0], -1)
    vt = torch.from_numpy(np.asarray(V, np.float64)).view(1, 1, V.shape[0], -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).view(-1).numpy()


def test_attend_tokens_matches_sdpa(orc):
    g = np.random.default_rng(7)
    for n, d in [(1, 8), (17, 64), (300, 128)]:
        q = g.standard_normal(d)
        K, V = g.standard_normal((n, d)), g.standard_normal((n, d))
        out, l = orc.attend_tokens(q, K, V)
        np.testing.assert_allclose(out, _sdpa_ref(q, K, V), atol=1e-12)
        assert l == pytest.approx(logsumexp(K @ q / math.sqrt(d)), abs=1e-12)
    out, l = orc.attend_tokens(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)))
    assert l == -np.inf and not out.any()


def test_dense_attend_pool_matches_sdpa(wl, orc):
    spec, layer, lay = _small_layout(wl, orc, seq_lens=[1000, 333], batch=2, num_q_heads=4,
                                     num_kv_heads=2, carriers=2)
    out, lse = orc.attend_pool(lay, layer.q, layer.k_f32(), layer.v_f32(), None)
    for b in range(2):
        for h in range(4):
            K = _tokens(layer, spec, b, h // 2, layer.k_f32())
            V = _tokens(layer, spec, b, h // 2, layer.v_f32())
            np.testing.assert_allclose(out[b, h], _sdpa_ref(layer.q[b, h], K, V), atol=1e-12)


def test_select_all_pages_reproduces_dense(wl, orc):
    """A budget covering every page gives exactly dense attention, including
    a partial last page (attended outside the budget)."""
    spec, layer, lay = _small_layout(wl, orc, seq_lens=[1000, 333], batch=2, num_q_heads=4,
                                     num_kv_heads=2, carriers=2)
    mu, basis, coef = orc.build_pool(lay, spec.rank, layer.k_f32(), spec.num_blocks)
    _, page = orc.scan_pool(lay, spec.rank, layer.q, mu, basis, coef)
    width = spec.max_pages
    sel, _ = orc.select_pool(lay, 10 ** 6, page.astype(np.float32), width)
    o_s, l_s = orc.attend_pool(lay, layer.q, layer.k_f32(), layer.v_f32(), sel)
    o_d, l_d = orc.attend_pool(lay, layer.q, layer.k_f32(), layer.v_f32(), None)
    np.testing.assert_allclose(o_s, o_d, atol=1e-13)
    np.testing.assert_allclose(l_s, l_d, atol=1e-13)


def test_sparse_attend_uses_only_listed_pages(wl, orc):
    """Attention over a page list equals SDPA over exactly those tokens plus
    the partial last page."""
    spec, layer, lay = _small_layout(wl, orc, seq_lens=[1000], carriers=2)
    sel = np.full((1, 1, 5), -1, np.int32)
    sel[0, 0, :3] = [2, 17, 40]
    out, _ = orc.attend_pool(lay, layer.q, layer.k_f32(), layer.v_f32(), sel)
    P = spec.page_size
    K, V = layer.k_f32(), layer.v_f32()
    pages = [2, 17, 40, 62]
    Kt = np.concatenate([K[layer.block_table[0, j], 0, :min(P, 1000 - j * P)] for j in pages])
    Vt = np.concatenate([V[layer.block_table[0, j], 0, :min(P, 1000 - j * P)] for j in pages])
    np.testing.assert_allclose(out[0, 0], _sdpa_ref(layer.q[0, 0], Kt, Vt), atol=1e-12)
    # entries that are not full pages (the partial page 62 itself, an index
    # past the sequence, -1) are ignored: the partial page is attended once
    sel2 = np.array([[[2, 17, 40, 62, 75, -1, 62]]], np.int32)
    out2, _ = orc.attend_pool(lay, layer.q, layer.k_f32(), layer.v_f32(), sel2)
    np.testing.assert_allclose(out2[0, 0], _sdpa_ref(layer.q[0, 0], Kt, Vt), atol=1e-12)


def test_unsummarised_pages_are_attended_outside_the_budget(wl, orc):
    """Pages compete for the budget once their summary exists (technical
    summary, section 2: a page's summary is made when the page is final, off
    the attention's critical path).  With a count s_b of summarised pages per
    sequence: pages j >= s_b are not scanned (-inf) and never selected, the
    selection is the brute-force top-k of the masses over j < s_b, and the
    attention covers exactly the selected pages plus every page from s_b to
    the end (plain softmax with scipy over those tokens).  A count at or above
    the full pages changes nothing; selecting every candidate is dense
    attention whatever the count."""
    from scipy.special import softmax
    lens = [16 * 30 + 7, 16 * 20, 16 * 12 + 3]
    spec, layer, lay = _small_layout(wl, orc, seq_lens=lens, batch=3, num_q_heads=4,
                                     num_kv_heads=2, carriers=1)
    P, d, G, r = spec.page_size, spec.head_dim, spec.group, spec.rank
    K, V = layer.k_f32(), layer.v_f32()
    counts = np.array([27, 25, 0], np.int32)  # 3 pending + partial; all summarised; none
    lay_s = orc.Layout(spec.num_q_heads, spec.num_kv_heads, d, P, layer.block_table,
                       layer.seq_lens, summarized=counts)
    mu, basis, coef = orc.build_pool(lay, r, K, spec.num_blocks)
    _, page_all = orc.scan_pool(lay, r, layer.q, mu, basis, coef)
    _, page = orc.scan_pool(lay_s, r, layer.q, mu, basis, coef)
    k = spec.k_pages
    sel, _ = orc.select_pool(lay_s, spec.budget_tokens, page.astype(np.float32), k)
    out, lse = orc.attend_pool(lay_s, layer.q, K, V, sel)
    for b in range(3):
        full, n_all = lens[b] // P, -(-lens[b] // P)
        s_b = min(int(counts[b]), full)
        np.testing.assert_array_equal(page[b, :, :s_b], page_all[b, :, :s_b])
        assert np.all(np.isneginf(page[b, :, s_b:]))
        for g in range(2):
            want = _brute_topk(page_all[b, g, :s_b].astype(np.float32), min(k, s_b))
            assert list(sel[b, g][sel[b, g] >= 0]) == want
            pages = want + list(range(s_b, n_all))
            toks = np.concatenate([K[layer.block_table[b, j], g, :min(P, lens[b] - j * P)]
                                   for j in pages]).astype(np.float64)
            vals = np.concatenate([V[layer.block_table[b, j], g, :min(P, lens[b] - j * P)]
                                   for j in pages]).astype(np.float64)
            for h in range(g * G, (g + 1) * G):
                sc = toks @ layer.q[b, h].astype(np.float64) / math.sqrt(d)
                assert abs(lse[b, h] - logsumexp(sc)) < 1e-12
                np.testing.assert_allclose(out[b, h], softmax(sc) @ vals, rtol=0, atol=1e-12)
    # a count at or above the full pages is no count at all
    lay_f = orc.Layout(spec.num_q_heads, spec.num_kv_heads, d, P, layer.block_table,
                       layer.seq_lens, summarized=np.array([40, 20, 13], np.int32))
    _, page_f = orc.scan_pool(lay_f, r, layer.q, mu, basis, coef)
    np.testing.assert_array_equal(page_f, page_all)
    # select every candidate: dense attention, whatever the count
    sel_all, _ = orc.select_pool(lay_s, 10 ** 6, page.astype(np.float32), spec.max_pages)
    o_s, l_s = orc.attend_pool(lay_s, layer.q, K, V, sel_all)
    o_d, l_d = orc.attend_pool(lay, layer.q, K, V, None)
    np.testing.assert_allclose(o_s, o_d, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_s, l_d, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- planted mistakes

def test_pins_catch_planted_mistakes(orc):
    """The pins above fail on plausible slips.  Each mutant is a deliberate
    mistake applied to oracle outputs on the CPU (a dropped centroid term, a
    wrong scale, a transposed basis) and must be caught by one pin."""
    P, d = 16, 64
    K = _page(P, d, offset=1.0, seed=99)
    q = np.random.default_rng(3).standard_normal(d)
    mu, basis, coef, _, _ = orc.page_summary(K, min(P, d))
    exact = orc.page_exact_lse(q, K)
    # dropped centroid term
    assert abs(orc.page_estimate(q, np.zeros(d), basis, coef) - exact) > 1e-3
    # logits scaled by 1/d instead of 1/sqrt(d)
    assert abs(orc.page_estimate(q / math.sqrt(d), mu, basis, coef) - exact) > 1e-3
    # basis used transposed within the page's subspace: coefficient columns permuted
    assert abs(orc.page_estimate(q, mu, basis, coef[:, ::-1]) - exact) > 1e-3


# ---------------------------------------------------------------- quantised summaries
# Stored precision: technical summary, section 2, "Kwantisatie" (int4 basis,
# int8 coefficients and centroid); scale granularity and rounding are the
# reading stated in oracle/locks_oracle.h.

@pytest.mark.parametrize("qmax", [127, 7])
def test_quantize_grid_values_are_lossless(orc, qmax):
    """Values on a power-of-two grid with a full-range code come back exactly."""
    g = np.random.default_rng(qmax)
    k = g.integers(-qmax, qmax + 1, 200)
    k[17] = -qmax
    s0 = np.float32(2.0 ** -5)
    x = (k * s0).astype(np.float32)
    s, code = orc.quantize_vec(x, qmax)
    assert s == s0
    assert np.array_equal(code.astype(np.int64), k)


@pytest.mark.parametrize("qmax", [127, 7])
def test_quantize_error_bound_and_range(orc, qmax):
    x = np.random.default_rng(7 + qmax).standard_normal(513).astype(np.float32) * 3.0
    s, code = orc.quantize_vec(x, qmax)
    c = code.astype(np.float64)
    assert np.abs(c).max() <= qmax
    i = int(np.argmax(np.abs(x)))
    assert c[i] == np.sign(x[i]) * qmax              # the absmax element takes the end code
    err = np.abs(x.astype(np.float64) - s * c)
    assert err.max() <= 0.5 * s * (1 + 1e-6)         # round to nearest


def test_quantize_matches_numpy_float32_rounding(orc):
    """The same arithmetic through numpy's float32 division and rint."""
    for qmax in (127, 7):
        x = np.random.default_rng(qmax).standard_normal(1000).astype(np.float32)
        s, code = orc.quantize_vec(x, qmax)
        s_np = np.float32(np.abs(x).max()) / np.float32(qmax)
        ref = np.clip(np.rint(x / s_np), -qmax, qmax).astype(np.int8)
        assert s == s_np and np.array_equal(code, ref)


def test_quantize_ties_and_zero(orc):
    s, code = orc.quantize_vec(np.array([127, 2.5, 3.5, -2.5, -0.5, 0.5], np.float32), 127)
    assert s == 1.0 and code.tolist() == [127, 2, 4, -2, 0, 0]    # half to even
    s, code = orc.quantize_vec(np.zeros(9, np.float32), 7)
    assert s == 0.0 and not code.any()


def test_quantize_pool_hand_example(orc):
    """One unit (P 2, d 4, r 1) worked by hand.
    centroid [1, -1/4, 1/8, 0]: scale 1/127, codes 127, -31.75 -> -32, 15.875 -> 16, 0;
    basis row [7, -3, 1, -6] / 16: scale (7/16)/7 = 1/16, codes 7 -3 1 -6, packed low
      nibble first: 0x7 | 0xD << 4 = 0xD7, 0x1 | 0xA << 4 = 0xA1;
    coefficient column [1/4, -1]: scale 1/127, codes 31.75 -> 32, -127."""
    mu = np.array([[[1.0, -0.25, 0.125, 0.0]]], np.float32)
    basis = (np.array([[[[7.0, -3.0, 1.0, -6.0]]]]) / 16).astype(np.float32)
    coef = np.array([[[[0.25], [-1.0]]]], np.float32)
    mu_q, basis_q, coef_q, scales = orc.quantize_pool(mu, basis, coef)
    assert mu_q.reshape(-1).tolist() == [127, -32, 16, 0]
    assert basis_q.reshape(-1).tolist() == [0xD7, 0xA1]
    assert coef_q.reshape(-1).tolist() == [32, -127]
    third = np.float32(1.0) / np.float32(127.0)
    assert scales.reshape(-1).tolist() == [third, 1.0 / 16, third]
    m2, b2, c2 = orc.dequantize_pool(mu_q, basis_q, coef_q, scales)
    assert b2.reshape(-1).tolist() == basis.reshape(-1).tolist()      # on the grid: exact
    assert np.allclose(m2, mu, atol=0.5 * third) and np.allclose(c2, coef, atol=0.5 * third)


def test_quantize_pool_granularity(orc):
    """One scale per basis row and per coefficient column: scaling one row (one
    column) by 2 doubles its scale alone and leaves every code unchanged."""
    g = np.random.default_rng(5)
    NB, H, P, d, r = 3, 2, 16, 64, 4
    mu = g.standard_normal((NB, H, d)).astype(np.float32)
    basis = g.standard_normal((NB, H, r, d)).astype(np.float32)
    coef = g.standard_normal((NB, H, P, r)).astype(np.float32)
    ref = orc.quantize_pool(mu, basis, coef)
    b2, c2 = basis.copy(), coef.copy()
    b2[1, 0, 2] *= 2
    c2[2, 1, :, 3] *= 2
    out = orc.quantize_pool(mu, b2, c2)
    for a, b in zip(ref[:3], out[:3]):
        assert np.array_equal(a, b)
    ds = out[3] / ref[3]
    expect = np.ones_like(ds)
    expect[1, 0, 1 + 2] = 2
    expect[2, 1, 1 + r + 3] = 2
    assert np.array_equal(ds, expect)


def test_dequantised_estimate_on_grid_equals_unquantised(wl, orc):
    """Summaries already on the quantiser's grid survive quantisation exactly,
    so the page masses of the dequantised summaries equal the originals."""
    spec = wl.config(0)
    layer = wl.make(spec)
    L = orc.Layout(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                   layer.block_table, layer.seq_lens)
    mu, basis, coef = orc.build_pool(L, spec.rank, layer.k_f32(), spec.num_blocks)
    # snap each vector to a power-of-two grid with a full-range code
    def snap(x, axis, qmax):
        m = np.abs(x).max(axis=axis, keepdims=True)
        s = 2.0 ** np.ceil(np.log2(np.where(m > 0, m, 1) / qmax))
        y = np.clip(np.round(x / s), -qmax, qmax)
        y = np.where(np.abs(y).max(axis=axis, keepdims=True) == qmax, y,
                     np.where(np.abs(x) == m, np.sign(x) * qmax, y))
        return (y * s).astype(np.float32)
    mu_g, basis_g, coef_g = snap(mu, -1, 127), snap(basis, -1, 7), snap(coef, -2, 127)
    deq = orc.dequantize_pool(*orc.quantize_pool(mu_g, basis_g, coef_g))
    for a, b in zip(deq, (mu_g, basis_g, coef_g)):
        assert np.array_equal(a, b)
    q = layer.q
    _, pm_a = orc.scan_pool(L, spec.rank, q, mu_g, basis_g, coef_g)
    _, pm_b = orc.scan_pool(L, spec.rank, q, *deq)
    assert np.array_equal(pm_a, pm_b)


# ---------------------------------------------------------------- shared-basis sketch (ablation)
# Baseline of the ablation: one basis per KV head, shared by every page
# (technical summary, section 3, the proposition on shared projections).

def _manual_layout(orc, K, Hq=2):
    """Pool [NB][1][P][d] as one sequence of NB full pages."""
    NB, H, P, d = K.shape
    return orc.Layout(Hq, H, d, P, np.arange(NB, dtype=np.int32)[None],
                      np.array([NB * P], np.int32))


def test_pooled_covariance_matches_numpy(wl, orc):
    spec, layer, lay = _small_layout(wl, orc, num_q_heads=2, num_kv_heads=2, seq_lens=[16 * 9 + 5])
    K = layer.k_f32()
    cov = orc.pooled_covariance(lay, K)
    for g in range(2):
        ref = np.zeros((spec.head_dim, spec.head_dim))
        for j in range(9):
            Kp = K[layer.block_table[0, j], g].astype(np.float64)
            Kc = Kp - Kp.mean(0)
            ref += Kc.T @ Kc
        np.testing.assert_allclose(cov[g], ref, rtol=1e-12, atol=1e-10)


def test_shared_basis_captures_the_top_energy(wl, orc):
    """Eckart-Young for the pooled covariance: the residual of projecting every
    page's centred keys on the shared basis is the sum of the trailing
    eigenvalues; the basis is orthonormal."""
    spec, layer, lay = _small_layout(wl, orc)
    K = layer.k_f32()
    rho = 10
    basis, eig = orc.shared_basis(lay, rho, K)
    V = basis[0]
    assert np.abs(V @ V.T - np.eye(rho)).max() < 1e-12
    resid = 0.0
    for j in range(spec.seq_lens[0] // spec.page_size):
        Kp = K[layer.block_table[0, j], 0].astype(np.float64)
        Kc = Kp - Kp.mean(0)
        resid += np.sum((Kc - Kc @ V.T @ V) ** 2)
    assert resid == pytest.approx(eig[0, rho:].sum(), rel=1e-9)


def test_sketch_is_exact_when_pages_share_one_subspace(orc):
    """Keys of every page in one common m-dimensional subspace (plus the
    page's own centroid): a shared basis of rank m spans every page, so the
    sketch's page masses equal the exact ones."""
    g = np.random.default_rng(8)
    NB, P, d, m = 12, 16, 64, 5
    W = g.standard_normal((m, d))
    K = np.stack([g.standard_normal(d) + g.standard_normal((P, m)) @ W for _ in range(NB)])
    K = K.astype(np.float32)[:, None]
    lay = _manual_layout(orc, K)
    q = (g.standard_normal((1, 2, d)) / 8).astype(np.float32)
    basis, _ = orc.shared_basis(lay, m, K)
    mu, rep, coef = orc.sketch_pool(lay, m, K, basis, NB)
    _, est = orc.scan_pool(lay, m, q, mu, rep, coef)
    _, exact = orc.exact_pool(lay, q, K)
    np.testing.assert_allclose(est[0, 0, :NB], exact[0, 0, :NB], atol=1e-4)


def test_sketch_full_basis_is_exact_on_shuffled_layout(wl, orc):
    """Paged indexing of the sketch: with a shared basis of full rank d every
    page's centred keys are kept exactly, so on a shuffled block table (two
    sequences, two KV heads) the sketch's masses equal exact_pool's (pinned
    against scipy through the block table), per head and per group."""
    lens = [16 * 11 + 7, 16 * 9]
    spec, layer, lay = _small_layout(wl, orc, seq_lens=lens, batch=2, num_q_heads=4,
                                     num_kv_heads=2, carriers=1, page_offset_std=1.0)
    K, d, P = layer.k_f32(), spec.head_dim, spec.page_size
    assert np.count_nonzero(layer.block_table[0, :lens[0] // P] != np.arange(lens[0] // P)) > 5
    sb, _ = orc.shared_basis(lay, d, K)
    head, page = orc.scan_pool(lay, d, layer.q, *orc.sketch_pool(lay, d, K, sb, spec.num_blocks))
    ehead, epage = orc.exact_pool(lay, layer.q, K)
    for b in range(2):
        f = lens[b] // P
        np.testing.assert_allclose(head[b, :, :f], ehead[b, :, :f], rtol=0, atol=1e-5)
        np.testing.assert_allclose(page[b, :, :f], epage[b, :, :f], rtol=0, atol=1e-5)
    assert np.abs(epage[0, 0, :lens[0] // P] - epage[0, 1, :lens[0] // P]).max() > 1e-2


def test_sketch_is_blind_where_page_summaries_are_exact(orc):
    """Every page in its own m-dimensional subspace: rank-m page summaries
    are exact on every page, while the shared basis at the same storage
    (rho = m (1 + d / P)) is not (the union of the subspaces is wider than
    rho) - the pages' claim, on a constructed example; at rho = d it is."""
    g = np.random.default_rng(9)
    NB, P, d, m = 24, 16, 64, 3
    K = np.stack([g.standard_normal(d) + g.standard_normal((P, m)) @ g.standard_normal((m, d))
                  for _ in range(NB)]).astype(np.float32)[:, None]
    lay = _manual_layout(orc, K)
    q = (g.standard_normal((1, 2, d)) / 8).astype(np.float32)
    _, exact = orc.exact_pool(lay, q, K)
    exact = exact[0, 0, :NB]
    mu, basis, coef = orc.build_pool(lay, m, K, NB)
    _, page = orc.scan_pool(lay, m, q, mu, basis, coef)
    assert np.abs(page[0, 0, :NB] - exact).max() < 1e-4
    rho = m * (1 + d // P)
    sb, _ = orc.shared_basis(lay, rho, K)
    _, sketch = orc.scan_pool(lay, rho, q, *orc.sketch_pool(lay, rho, K, sb, NB))
    assert np.abs(sketch[0, 0, :NB] - exact).max() > 1e-2
    sb_full, _ = orc.shared_basis(lay, d, K)
    _, full = orc.scan_pool(lay, d, q, *orc.sketch_pool(lay, d, K, sb_full, NB))
    np.testing.assert_allclose(full[0, 0, :NB], exact, atol=1e-4)


def test_degenerate_sequences_reduce_to_plain_softmax(wl, orc):
    """Sequences the selection cannot thin out: with no full page nothing is
    selected and the step attends the partial page alone; when every full
    page fits the budget all are selected in order.  Either way the step's
    attention is plain softmax attention over every token (scipy), and an
    empty sequence gives a zero output with lse -inf."""
    from scipy.special import softmax
    spec, layer, lay = _small_layout(wl, orc, seq_lens=[0, 9, 16 * 40 + 3, 16 * 2], batch=4,
                                     num_q_heads=4, carriers=0)
    K, V = layer.k_f32(), layer.v_f32()
    r, P, G = spec.rank, spec.page_size, spec.group
    mu, basis, coef = orc.build_pool(lay, r, K, spec.num_blocks)
    _, page = orc.scan_pool(lay, r, layer.q, mu, basis, coef, heads=False)
    k = spec.k_pages
    sel, mass = orc.select_pool(lay, spec.budget_tokens, page.astype(np.float32), k)
    out, lse = orc.attend_pool(lay, layer.q, K, V, sel)
    assert np.all(sel[0] == -1) and np.all(np.isneginf(mass[0]))
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(sel[1] == -1)
    assert list(sel[3, 0]) == [0, 1] + [-1] * (k - 2)
    for b in (1, 3):
        for h in range(spec.num_q_heads):
            g = h // G
            keys = _tokens(layer, spec, b, g, K)
            vals = _tokens(layer, spec, b, g, V)
            s = keys @ layer.q[b, h].astype(np.float64) / math.sqrt(spec.head_dim)
            assert abs(lse[b, h] - logsumexp(s)) < 1e-12
            assert np.allclose(out[b, h], softmax(s) @ vals, rtol=0, atol=1e-12)
