"""GPU parity of the summary scan (page masses) and the top-k selection,
against the oracle on the same seeded inputs, through the C ABI."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_cases import (DEV, Case, band_ok, bf16_small, masses_close, say, shifted_log2_sums, tiny,
                       to_np)
from workload.device import summaries_to_device

pytestmark = pytest.mark.gpu

RUN = 16  # pages per run maximum (LOCKS_RUN_PAGES)


def host_run_max(pm, lens, P):
    """Run maxima of fp32 masses [B][H][MP] over runs of RUN pages, counting
    only full pages (j < lens[b] // P); -inf for runs without one."""
    B, H, MP = pm.shape
    nr = -(-MP // RUN)
    out = np.full((B, H, nr), -np.inf, np.float32)
    for b in range(B):
        n = min(int(lens[b]) // P, MP)
        for r in range(-(-n // RUN)):
            out[b, :, r] = pm[b, :, r * RUN:min(n, (r + 1) * RUN)].max(axis=-1)
    return out

SCAN_CASES = [
    ("tiny-r4", lambda: tiny()),
    ("tiny-r16", lambda: tiny(rank=16)),
    ("tiny-G4-r3-ragged", lambda: tiny(num_q_heads=4, num_kv_heads=1, rank=3, seq_lens=[1000])),
    ("bf16-G16-r8", lambda: bf16_small()),
    ("bf16-G16-r2", lambda: bf16_small(rank=2)),
    ("bf16-G4-r16-offset", lambda: bf16_small(num_kv_heads=8, rank=16, page_offset_std=1.0)),
    ("bf16-G1-r5", lambda: bf16_small(num_q_heads=2, rank=5)),
    # the other two (page size, head dim) instantiations
    ("bf16-G16-r8-d64", lambda: bf16_small(head_dim=64)),
    ("tiny-P16-d128-r8", lambda: tiny(head_dim=128, rank=8, seq_lens=[16 * 70 + 9])),
]


@pytest.mark.parametrize("name,mk", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_scan_matches_oracle(name, mk):
    """Scan alone, fed the oracle's (fp32) summaries: per-head and group
    log-masses within 1e-4, -inf exactly where a page is not full."""
    case = Case(mk())
    s = case.spec
    mu, basis, coef = case.oracle_summaries()
    head_o, page_o = oracle.scan_pool(case.lay, s.rank, case.layer.q, mu, basis, coef)
    summ = summaries_to_device(mu, basis, coef)
    import kv_cache_page_rank_amd as lk
    pm = torch.full((s.batch, s.num_kv_heads, s.max_pages), 7.0, device=DEV)
    hm = torch.full((s.batch, s.num_q_heads, s.max_pages), 7.0, device=DEV)
    rm = torch.full((s.batch, s.num_kv_heads, -(-s.max_pages // RUN)), 7.0, device=DEV)
    say("scan", name, s)
    lk.locks_scan(case.q, summ, case.pages, pm, hm, run_max=rm)
    torch.cuda.synchronize()
    assert masses_close(to_np(pm), page_o) <= 1e-4
    assert masses_close(to_np(hm), head_o) <= 1e-4
    # the run maxima are exactly the maxima of the written masses
    np.testing.assert_array_equal(to_np(rm), host_run_max(to_np(pm), s.seq_lens, s.page_size))


@pytest.mark.parametrize("name,mk", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_scan_bf16_summaries_match_oracle(name, mk):
    """Scan of bf16 summaries: the oracle reads the same rounded values
    (widened exactly), so the bar is the fp32 one: log-masses within 1e-4."""
    case = Case(mk())
    s = case.spec
    mu, basis, coef = (torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
                       for x in case.oracle_summaries())
    wide = [x.float().numpy() for x in (mu, basis, coef)]
    head_o, page_o = oracle.scan_pool(case.lay, s.rank, case.layer.q, *wide)
    import kv_cache_page_rank_amd as lk
    summ = lk.Summaries(mu.to(DEV), basis.to(DEV), coef.to(DEV))
    pm = torch.full((s.batch, s.num_kv_heads, s.max_pages), 7.0, device=DEV)
    hm = torch.full((s.batch, s.num_q_heads, s.max_pages), 7.0, device=DEV)
    rm = torch.full((s.batch, s.num_kv_heads, -(-s.max_pages // RUN)), 7.0, device=DEV)
    say("scan bf16 summaries", name, s)
    lk.locks_scan(case.q, summ, case.pages, pm, hm, run_max=rm)
    pm2 = torch.full_like(pm, 7.0)
    lk.locks_scan(case.q, summ, case.pages, pm2)  # the path without per-head output
    torch.cuda.synchronize()
    assert masses_close(to_np(pm), page_o) <= 1e-4
    assert masses_close(to_np(pm2), page_o) <= 1e-4
    assert masses_close(to_np(hm), head_o) <= 1e-4
    np.testing.assert_array_equal(to_np(rm), host_run_max(to_np(pm), s.seq_lens, s.page_size))


def test_select_bf16_summaries_band():
    """locks_select over bf16 summaries (the oracle's, rounded to nearest
    even) against the oracle's selection from the same rounded values."""
    case = Case(bf16_small())
    s = case.spec
    import kv_cache_page_rank_amd as lk
    mu, basis, coef = (torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
                       for x in case.oracle_summaries())
    summ = lk.Summaries(mu.to(DEV), basis.to(DEV), coef.to(DEV))
    say("select bf16 summaries")
    wide = [x.float().numpy() for x in (mu, basis, coef)]
    _, page_o = oracle.scan_pool(case.lay, s.rank, case.layer.q, *wide, heads=False)
    k = s.k_pages
    sel_o, _ = oracle.select_pool(case.lay, s.budget_tokens, page_o.astype(np.float32), k)
    sel = torch.empty((s.batch, s.num_kv_heads, k), dtype=torch.int32, device=DEV)
    mass = torch.empty((s.batch, s.num_kv_heads, k), device=DEV)
    ws = lk.workspace(lk.workspace_bytes(lk.OP_SELECT, s.batch, s.max_pages, s.num_q_heads,
                                         s.num_kv_heads, s.page_size, s.head_dim, s.rank, k))
    lk.locks_select(case.q, summ, case.pages, s.budget_tokens, sel, mass, ws=ws)
    torch.cuda.synchronize()
    sel_g = sel.cpu().numpy()
    for b in range(s.batch):
        f = s.seq_lens[b] // s.page_size
        for g in range(s.num_kv_heads):
            assert band_ok(sel_g[b, g], sel_o[b, g], page_o[b, g, :f], min(k, f)), (b, g)


def test_scan_full_rank_is_exact_lse():
    """r = min(P, d): the GPU estimate from oracle summaries equals the exact
    page LSE (the selection that reads every key)."""
    case = Case(tiny(rank=16))
    mu, basis, coef = case.oracle_summaries()
    _, exact = oracle.exact_pool(case.lay, case.layer.q, case.k_f32)
    import kv_cache_page_rank_amd as lk
    s = case.spec
    pm = torch.empty((1, 1, s.max_pages), device=DEV)
    say("scan full rank", s)
    lk.locks_scan(case.q, summaries_to_device(mu, basis, coef), case.pages, pm)
    torch.cuda.synchronize()
    assert masses_close(to_np(pm), exact) <= 1e-4


# ------------------------------------------------------------------ top-k

def _topk_case(rng, B, H, MP, P, lens, levels=None, neg_inf=0.0):
    if levels:
        vals = rng.standard_normal(levels).astype(np.float32)
        pm = vals[rng.integers(0, levels, (B, H, MP))]
    else:
        pm = rng.standard_normal((B, H, MP)).astype(np.float32)
    if neg_inf:
        pm[rng.random(pm.shape) < neg_inf] = -np.inf
    bt = np.zeros((B, MP), np.int32)
    return pm, bt, np.asarray(lens, np.int32)


TOPK_CASES = [
    # name, B, H, max_pages, P, seq_lens, budget, width, levels, -inf fraction
    ("one-page", 1, 1, 1, 64, [64], 2048, 32, None, 0.0),
    ("fewer-pages-than-k", 2, 2, 10, 64, [640, 64 * 7 + 5], 2048, 32, None, 0.0),
    ("budget-below-page", 1, 2, 50, 64, [3200], 63, 1, None, 0.0),
    ("ties", 2, 3, 3000, 64, [64 * 3000, 64 * 1777 + 1], 2048, 32, 3, 0.0),
    ("ties-many-k", 1, 2, 5000, 16, [16 * 5000], 16 * 700, 700, 5, 0.0),
    ("neg-inf", 1, 2, 2100, 64, [64 * 2100], 2048, 32, None, 0.5),
    ("all-equal", 1, 1, 4096, 64, [64 * 4096], 2048, 32, 1, 0.0),
    ("max-pages", 1, 2, 32768, 64, [64 * 32768], 4096, 64, 50, 0.0),
    # more than 1024 runs of 16 pages with k <= 32 (both of a thread's runs in
    # the bound), partial last runs
    ("max-pages-k32", 1, 2, 32768, 64, [64 * 32760 - 5], 2048, 32, None, 0.0),
    ("runs-1188-k20", 2, 1, 19000, 64, [64 * 19000 - 1, 64 * 18999 + 40], 64 * 20, 20, None, 0.1),
    ("empty-seq", 2, 1, 8, 64, [0, 63], 2048, 32, None, 0.0),
    ("wide-rows", 1, 1, 1500, 64, [64 * 1500], 2048, 40, None, 0.0),
    ("batch-varied", 4, 2, 4000, 64, [64 * 500, 64 * 3999 + 7, 64 * 40, 64 * 1100], 2048, 32,
     None, 0.0),
    ("k64-few-runs", 2, 1, 600, 64, [64 * 600, 64 * 70], 64 * 64, 64, None, 0.0),
]


@pytest.mark.parametrize("runs", [False, True], ids=["all-masses", "run-maxima"])
@pytest.mark.parametrize("case", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_topk_bit_exact(case, runs):
    """Integer work: identical fp32 inputs give identical page lists and
    masses (ties to the lowest page index, ascending order, -1/-inf pads),
    with and without the run maxima index."""
    name, B, H, MP, P, lens, budget, width, levels, ninf = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    pm, bt, sl = _topk_case(rng, B, H, MP, P, lens, levels, ninf)
    lay = oracle.Layout(H, H, 64, P, bt, sl)
    sel_o, mass_o = oracle.select_pool(lay, budget, pm, width)
    import kv_cache_page_rank_amd as lk
    pages = lk.PageTable(torch.from_numpy(bt).to(DEV), torch.from_numpy(sl).to(DEV))
    sel = torch.full((B, H, width), -7, dtype=torch.int32, device=DEV)
    mass = torch.full((B, H, width), 7.0, device=DEV)
    rm = torch.from_numpy(host_run_max(pm, lens, P)).to(DEV) if runs else None
    say("topk", name, "runs", runs)
    lk.locks_topk(torch.from_numpy(pm).to(DEV), pages, P, budget, sel, mass, run_max=rm)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), sel_o)
    np.testing.assert_array_equal(mass.cpu().numpy(), mass_o)


def _topk_against_oracle(pm, P, lens, budget, width, offset=0, tag="", runs=False):
    """locks_topk on pm (placed `offset` floats into its device buffer) against
    the oracle's selection, bit for bit."""
    B, H, MP = pm.shape
    bt = np.zeros((B, MP), np.int32)
    sl = np.asarray(lens, np.int32)
    lay = oracle.Layout(H, H, 64, P, bt, sl)
    sel_o, mass_o = oracle.select_pool(lay, budget, pm, width)
    import kv_cache_page_rank_amd as lk
    pages = lk.PageTable(torch.from_numpy(bt).to(DEV), torch.from_numpy(sl).to(DEV))
    buf = torch.zeros(pm.size + offset, device=DEV)
    buf[offset:] = torch.from_numpy(pm.ravel()).to(DEV)
    dev_pm = buf[offset:].view(B, H, MP)
    sel = torch.full((B, H, width), -7, dtype=torch.int32, device=DEV)
    mass = torch.full((B, H, width), 7.0, device=DEV)
    rm = torch.from_numpy(host_run_max(pm, lens, P)).to(DEV) if runs else None
    say("topk", tag, "offset", offset, "runs", runs)
    lk.locks_topk(dev_pm, pages, P, budget, sel, mass, run_max=rm)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), sel_o)
    np.testing.assert_array_equal(mass.cpu().numpy(), mass_o)


@pytest.mark.parametrize("offset", [0, 1, 2])
def test_topk_unaligned_rows(offset):
    """Rows that do not start on a 16-byte boundary take the scalar-load
    layout; the result must not depend on it."""
    rng = np.random.default_rng(4242 + offset)
    pm = rng.standard_normal((2, 2, 4096)).astype(np.float32)
    _topk_against_oracle(pm, 64, [64 * 4096, 64 * 3001 + 9], 2048, 32, offset, "unaligned")


@pytest.mark.parametrize("runs", [False, True], ids=["all-masses", "run-maxima"])
@pytest.mark.parametrize("run", [64, 256, 1500])
def test_topk_planted_run(run, runs):
    """A run of consecutive pages sharing the top value: the candidates
    above the bound crowd into few threads (one wave's share overflows for
    the longer runs) and the k winners are the lowest pages of the run."""
    rng = np.random.default_rng(run)
    pm = rng.standard_normal((1, 2, 8192)).astype(np.float32)
    pm[0, 0, 100:100 + run] = 9.0
    pm[0, 1, 8192 - run:] = 9.0
    _topk_against_oracle(pm, 64, [64 * 8192], 64 * 48, 48, 0, f"run{run}", runs)


@pytest.mark.parametrize("mk", [lambda: tiny(), lambda: bf16_small(), lambda: bf16_small(rank=2)])
def test_select_end_to_end_band(mk):
    """locks_select (scan + top-k) from oracle summaries against the oracle's
    selection: identical except pages within 1e-3 of the k-th mass."""
    case = Case(mk())
    s = case.spec
    mu, basis, coef = case.oracle_summaries()
    _, page_o = oracle.scan_pool(case.lay, s.rank, case.layer.q, mu, basis, coef, heads=False)
    width = s.k_pages
    sel_o, _ = oracle.select_pool(case.lay, s.budget_tokens, page_o.astype(np.float32), width)
    import kv_cache_page_rank_amd as lk
    sel = torch.empty((s.batch, s.num_kv_heads, width), dtype=torch.int32, device=DEV)
    mass = torch.empty((s.batch, s.num_kv_heads, width), device=DEV)
    ws = lk.workspace(lk.workspace_bytes(lk.OP_SELECT, s.batch, s.max_pages, s.num_q_heads,
                                         s.num_kv_heads, s.page_size, s.head_dim, s.rank, width))
    say("select e2e", s)
    lk.locks_select(case.q, summaries_to_device(mu, basis, coef), case.pages, s.budget_tokens,
                    sel, mass, ws=ws)
    torch.cuda.synchronize()
    sel_g = sel.cpu().numpy()
    for b in range(s.batch):
        f = s.seq_lens[b] // s.page_size
        for g in range(s.num_kv_heads):
            assert band_ok(sel_g[b, g], sel_o[b, g], page_o[b, g, :f], min(width, f)), (b, g)
            assert list(sel_g[b, g]) == sorted(sel_g[b, g][sel_g[b, g] >= 0]) + \
                [-1] * int((sel_g[b, g] < 0).sum())


@pytest.mark.parametrize("mk", [lambda: tiny(), lambda: bf16_small(), lambda: bf16_small(rank=2)])
def test_select_equals_topk_of_its_masses(mk):
    """locks_select (top-k through the run maxima in its workspace) picks
    exactly what locks_topk over every mass picks from the same masses."""
    case = Case(mk())
    s = case.spec
    summ = summaries_to_device(*case.oracle_summaries())
    import kv_cache_page_rank_amd as lk
    k = s.k_pages
    ws = lk.workspace(lk.workspace_bytes(lk.OP_SELECT, s.batch, s.max_pages, s.num_q_heads,
                                         s.num_kv_heads, s.page_size, s.head_dim, s.rank, k))
    sel = torch.empty((s.batch, s.num_kv_heads, k), dtype=torch.int32, device=DEV)
    mass = torch.empty((s.batch, s.num_kv_heads, k), device=DEV)
    pm = torch.empty((s.batch, s.num_kv_heads, s.max_pages), device=DEV)
    say("select vs topk", s)
    lk.locks_select(case.q, summ, case.pages, s.budget_tokens, sel, mass, page_logmass=pm, ws=ws)
    sel2 = torch.empty_like(sel)
    mass2 = torch.empty_like(mass)
    lk.locks_topk(pm, case.pages, s.page_size, s.budget_tokens, sel2, mass2)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2)
    assert torch.equal(mass, mass2)


SHARE_CASES = [  # B, Hq, Hkv, max_pages, page_size, seq_lens
    (2, 32, 2, 2000, 64, [64 * 2000, 64 * 1234 + 17]),
    (3, 32, 8, 700, 64, [64 * 700, 64 * 3, 64 * 511 + 63]),
    (1, 6, 2, 300, 16, [16 * 299 + 4]),
    (2, 4, 4, 50, 64, [64 * 50, 0]),
]


@pytest.mark.parametrize("case", SHARE_CASES, ids=[f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}" for c in SHARE_CASES])
def test_mean_share_matches_oracle(case):
    """Mean-of-share scores from identical fp32 per-head estimates: within
    2e-5 of the oracle (fp32 exp/log against fp64), -inf exactly where a page
    is not full; the run maxima are exactly the maxima of the written scores."""
    B, Hq, Hkv, MP, P, lens = case
    rng = np.random.default_rng(Hq * 1000 + MP)
    hm = rng.normal(2.0, 3.0, (B, Hq, MP)).astype(np.float32)
    for b in range(B):
        hm[b, :, lens[b] // P:] = np.nan  # never read: past the full pages
    bt = np.zeros((B, MP), np.int32)
    lay = oracle.Layout(Hq, Hkv, 8, P, bt, np.asarray(lens, np.int32))
    ref = oracle.share_pool(lay, np.where(np.isnan(hm), -np.inf, hm).astype(np.float64))
    import kv_cache_page_rank_amd as lk
    pages = lk.PageTable(torch.from_numpy(bt).to(DEV), torch.from_numpy(np.asarray(lens, np.int32)).to(DEV))
    out = torch.full((B, Hkv, MP), 7.0, device=DEV)
    rm = torch.full((B, Hkv, -(-MP // RUN)), 7.0, device=DEV)
    ws = lk.workspace(lk.workspace_bytes(lk.OP_SELECT, B, MP, Hq, Hkv, P, 128, 8, 1))
    say("mean share", case)
    lk.locks_mean_share(torch.from_numpy(hm).to(DEV), Hkv, pages, P, out, run_max=rm, ws=ws)
    torch.cuda.synchronize()
    got = to_np(out)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.abs(got[fin] - ref[fin]).max() <= 2e-5
    np.testing.assert_array_equal(to_np(rm), host_run_max(got, lens, P))


@pytest.mark.parametrize("mk", [lambda: tiny(num_q_heads=4, num_kv_heads=1, seq_lens=[1000]),
                                lambda: bf16_small(), lambda: bf16_small(num_kv_heads=8)],
                         ids=["tiny-G4", "bf16-G16", "bf16-G4"])
def test_select_mean_share_band(mk):
    """locks_select with the mean-of-share aggregation against the oracle on
    the same summaries: scores within 1e-4, selections equal up to the 1e-3
    band around the k-th score, and equal to the top-k of its own scores."""
    case = Case(mk())
    s = case.spec
    mu, basis, coef = case.oracle_summaries()
    head_o, _ = oracle.scan_pool(case.lay, s.rank, case.layer.q, mu, basis, coef)
    share_o = oracle.share_pool(case.lay, head_o)
    k = s.k_pages
    sel_o, _ = oracle.select_pool(case.lay, s.budget_tokens, share_o.astype(np.float32), k)
    import kv_cache_page_rank_amd as lk
    sel = torch.empty((s.batch, s.num_kv_heads, k), dtype=torch.int32, device=DEV)
    mass = torch.empty((s.batch, s.num_kv_heads, k), device=DEV)
    pm = torch.empty((s.batch, s.num_kv_heads, s.max_pages), device=DEV)
    ws = lk.workspace(lk.workspace_bytes(lk.OP_SELECT, s.batch, s.max_pages, s.num_q_heads,
                                         s.num_kv_heads, s.page_size, s.head_dim, s.rank, k))
    say("select mean share", s)
    lk.locks_select(case.q, summaries_to_device(mu, basis, coef), case.pages, s.budget_tokens,
                    sel, mass, page_logmass=pm, ws=ws, agg=lk.AGG_MEAN_SHARE)
    sel2 = torch.empty_like(sel)
    mass2 = torch.empty_like(mass)
    lk.locks_topk(pm, case.pages, s.page_size, s.budget_tokens, sel2, mass2)
    torch.cuda.synchronize()
    assert masses_close(to_np(pm), share_o) <= 1e-4
    assert torch.equal(sel, sel2) and torch.equal(mass, mass2)
    sel_g = sel.cpu().numpy()
    for b in range(s.batch):
        f = s.seq_lens[b] // s.page_size
        for g in range(s.num_kv_heads):
            assert band_ok(sel_g[b, g], sel_o[b, g], share_o[b, g, :f], min(k, f)), (b, g)


def test_select_deterministic():
    case = Case(bf16_small())
    s = case.spec
    summ = summaries_to_device(*case.oracle_summaries())
    import kv_cache_page_rank_amd as lk
    outs = []
    for _ in range(2):
        sel = torch.empty((s.batch, s.num_kv_heads, s.k_pages), dtype=torch.int32, device=DEV)
        mass = torch.empty((s.batch, s.num_kv_heads, s.k_pages), device=DEV)
        pm = torch.empty((s.batch, s.num_kv_heads, s.max_pages), device=DEV)
        say("select determinism")
        lk.locks_select(case.q, summ, case.pages, s.budget_tokens, sel, mass, page_logmass=pm)
        torch.cuda.synchronize()
        outs.append((sel.cpu(), mass.cpu(), pm.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [16.0, 32.0])
def test_scan_large_logits(scale, sdt):
    """Logits of tens to hundreds (queries scaled up, page centroids offset):
    the fp32 and bf16 scans still match the oracle's masses within 1e-4 (the
    products carry an error relative to the logits' size, so this is the
    demanding case), with and without per-head output.  The group form sums
    each page's 2^logit shifted by its largest centroid term and takes the
    exact form (the page's max first) where that sum leaves [2^-60, 2^60];
    at x32 both forms are taken, which the oracle's values confirm."""
    case = Case(bf16_small(num_kv_heads=8, page_offset_std=4.0))
    s = case.spec
    vals = case.oracle_summaries()
    if sdt == "bf16":
        t = [torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) for x in vals]
        vals = [x.float().numpy() for x in t]
    q_host = (case.layer.q.astype(np.float64) * scale).astype(np.float32)
    head_o, page_o = oracle.scan_pool(case.lay, s.rank, q_host, *vals)
    shifted = shifted_log2_sums(case, q_host, vals[0], page_o)
    assert (shifted < 56).any()
    if scale >= 32:
        assert (shifted > 64).sum() >= 10
    import kv_cache_page_rank_amd as lk
    if sdt == "bf16":
        summ = lk.Summaries(*(x.to(DEV) for x in t))
    else:
        summ = summaries_to_device(*vals)
    q = torch.from_numpy(q_host).to(DEV)
    pm = torch.empty((s.batch, s.num_kv_heads, s.max_pages), device=DEV)
    pm2 = torch.empty_like(pm)
    hm = torch.empty((s.batch, s.num_q_heads, s.max_pages), device=DEV)
    say("scan large logits", scale, sdt, "shifted log2-sum range", shifted.min(), shifted.max())
    lk.locks_scan(q, summ, case.pages, pm, hm)
    lk.locks_scan(q, summ, case.pages, pm2)
    torch.cuda.synchronize()
    fin = np.isfinite(page_o)
    assert float(np.abs(page_o[fin]).max()) > 8.0  # the regime this case is for
    err = (masses_close(to_np(pm), page_o), masses_close(to_np(pm2), page_o),
           masses_close(to_np(hm), head_o))
    say("max |log-mass error|", *err)
    assert max(err) <= 1e-4
