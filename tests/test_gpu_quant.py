"""Integer-code summaries (int8 centroid and coefficients, int4 basis, fp32
scales; technical summary, section 2, Kwantisatie): the GPU quantiser is
bit-exact against the oracle's, the scan of codes matches the oracle's
estimate on the dequantised summary, the builder's quantised output equals
quantising its fp32 output, and selection over codes matches the oracle's."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import (DEV, Case, band_ok, bf16_small, masses_close, say, shifted_log2_sums, tiny,
                       to_np)
from workload.device import codes_to_device, summaries_to_device

pytestmark = pytest.mark.gpu
RUN = 16

CASES = [
    ("tiny-r4", lambda: tiny()),
    ("tiny-r16", lambda: tiny(rank=16)),
    ("tiny-G4-r3-ragged", lambda: tiny(num_q_heads=4, num_kv_heads=1, rank=3, seq_lens=[1000])),
    ("bf16-G16-r8", lambda: bf16_small()),
    ("bf16-G16-r2", lambda: bf16_small(rank=2)),
    ("bf16-G4-r16-offset", lambda: bf16_small(num_kv_heads=8, rank=16, page_offset_std=1.0)),
    ("bf16-G1-r5", lambda: bf16_small(num_q_heads=2, rank=5)),
    # several runs per (b, g), workgroups spanning two (b, g), ragged last
    # pages (d 128 and d 64)
    ("bf16-G16-r8-long", lambda: bf16_small(seq_lens=[64 * 130 + 5, 64 * 64])),
    ("tiny-long-ragged", lambda: tiny(seq_lens=[16 * 150 + 3])),
    # the other two (page size, head dim) instantiations
    ("bf16-G16-r8-d64", lambda: bf16_small(head_dim=64)),
    ("tiny-P16-d128-r8", lambda: tiny(head_dim=128, rank=8, seq_lens=[16 * 70 + 9])),
]


def _host_run_max(pm, lens, P):
    B, H, MP = pm.shape
    out = np.full((B, H, -(-MP // RUN)), -np.inf, np.float32)
    for b in range(B):
        n = min(int(lens[b]) // P, MP)
        for r in range(-(-n // RUN)):
            out[b, :, r] = pm[b, :, r * RUN:min(n, (r + 1) * RUN)].max(axis=-1)
    return out


def _codes_np(summ):
    return [t.cpu().numpy() for t in (summ.mu, summ.basis, summ.coef, summ.scales)]


@pytest.mark.parametrize("name,mk", CASES, ids=[c[0] for c in CASES])
def test_quantize_matches_oracle_bit_exact(name, mk):
    """The oracle's fp32 summaries quantised on the GPU and by the oracle:
    identical codes and scales (both take the decision in float arithmetic)."""
    import kv_cache_page_rank_amd as lk
    case = Case(mk())
    s = case.spec
    mu, basis, coef = case.oracle_summaries()
    ref = oracle.quantize_pool(mu, basis, coef)
    src = summaries_to_device(mu, basis, coef)
    dst = lk.Summaries.empty(s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim, s.rank,
                             dtype=lk.Q8Q4)
    say("quantize", name, s)
    lk.locks_quantize_summaries(src, dst)
    torch.cuda.synchronize()
    for got, want, what in zip(_codes_np(dst), ref, ("mu", "basis", "coef", "scales")):
        np.testing.assert_array_equal(got, want, err_msg=what)


@pytest.mark.parametrize("name,mk", CASES, ids=[c[0] for c in CASES])
def test_scan_codes_match_oracle(name, mk):
    """Scan of the oracle's codes against the oracle's estimate on the
    dequantised summary: per-head and group log-masses within 1e-4, -inf
    exactly where a page is not full, run maxima exact."""
    import kv_cache_page_rank_amd as lk
    case = Case(mk())
    s = case.spec
    codes = oracle.quantize_pool(*case.oracle_summaries())
    deq = oracle.dequantize_pool(*codes)
    head_o, page_o = oracle.scan_pool(case.lay, s.rank, case.layer.q, *deq)
    summ = codes_to_device(*codes)
    pm = torch.full((s.batch, s.num_kv_heads, s.max_pages), 7.0, device=DEV)
    hm = torch.full((s.batch, s.num_q_heads, s.max_pages), 7.0, device=DEV)
    rm = torch.full((s.batch, s.num_kv_heads, -(-s.max_pages // RUN)), 7.0, device=DEV)
    say("scan codes", name, s)
    lk.locks_scan(case.q, summ, case.pages, pm, hm, run_max=rm)
    pm2 = torch.full_like(pm, 7.0)
    lk.locks_scan(case.q, summ, case.pages, pm2)  # the path without per-head output
    torch.cuda.synchronize()
    assert masses_close(to_np(pm), page_o) <= 1e-4
    assert masses_close(to_np(pm2), page_o) <= 1e-4
    assert masses_close(to_np(hm), head_o) <= 1e-4
    np.testing.assert_array_equal(to_np(rm), _host_run_max(to_np(pm), s.seq_lens, s.page_size))


@pytest.mark.parametrize("mk", [lambda: tiny(), lambda: bf16_small(), lambda: bf16_small(rank=5)],
                         ids=["tiny", "bf16-r8", "bf16-r5"])
def test_build_codes_equal_quantised_fp32_build(mk):
    """The builder's quantised output is its fp32 summary quantised: equal,
    bit for bit, to locks_quantize_summaries of an fp32 build, on every unit
    of a full page; a one-page refresh writes the same codes."""
    import kv_cache_page_rank_amd as lk
    case = Case(mk())
    s = case.spec
    shape = (s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim, s.rank)
    f32 = lk.Summaries.empty(*shape)
    q_ref = lk.Summaries.empty(*shape, dtype=lk.Q8Q4)
    q_dir = lk.Summaries.empty(*shape, dtype=lk.Q8Q4)
    for t in (f32.mu, f32.basis, f32.coef):
        t.zero_()
    say("build fp32 + quantise / build codes", s)
    lk.locks_build_summaries(case.kv, case.pages, f32)
    lk.locks_quantize_summaries(f32, q_ref)
    lk.locks_build_summaries(case.kv, case.pages, q_dir)
    torch.cuda.synchronize()
    bt = case.layer.block_table
    full = [int(bt[b, j]) for b in range(s.batch) for j in range(s.seq_lens[b] // s.page_size)]
    for got, want in zip(_codes_np(q_dir), _codes_np(q_ref)):
        np.testing.assert_array_equal(got[full], want[full])
    # refresh of each sequence's last full page into a cleared copy
    q_ref_np = _codes_np(q_ref)
    for t in (q_dir.mu, q_dir.basis, q_dir.coef, q_dir.scales):
        t.zero_()
    last = torch.tensor([n // s.page_size - 1 for n in s.seq_lens], dtype=torch.int32,
                        device=DEV)
    say("refresh codes", s)
    lk.locks_refresh_summaries(case.kv, case.pages, last, 1, q_dir)
    torch.cuda.synchronize()
    blocks = [int(bt[b, s.seq_lens[b] // s.page_size - 1]) for b in range(s.batch)]
    for got, want in zip(_codes_np(q_dir), q_ref_np):
        np.testing.assert_array_equal(got[blocks], want[blocks])


def test_select_codes_band():
    """locks_select over the oracle's codes against the oracle's selection
    from the dequantised summary's masses."""
    import kv_cache_page_rank_amd as lk
    case = Case(bf16_small())
    s = case.spec
    codes = oracle.quantize_pool(*case.oracle_summaries())
    _, page_o = oracle.scan_pool(case.lay, s.rank, case.layer.q, *oracle.dequantize_pool(*codes),
                                 heads=False)
    k = s.k_pages
    sel_o, _ = oracle.select_pool(case.lay, s.budget_tokens, page_o.astype(np.float32), k)
    summ = codes_to_device(*codes)
    sel = torch.empty((s.batch, s.num_kv_heads, k), dtype=torch.int32, device=DEV)
    mass = torch.empty((s.batch, s.num_kv_heads, k), device=DEV)
    ws = lk.workspace(lk.workspace_bytes(lk.OP_SELECT, s.batch, s.max_pages, s.num_q_heads,
                                         s.num_kv_heads, s.page_size, s.head_dim, s.rank, k))
    say("select codes")
    lk.locks_select(case.q, summ, case.pages, s.budget_tokens, sel, mass, ws=ws)
    torch.cuda.synchronize()
    sel_g = sel.cpu().numpy()
    for b in range(s.batch):
        f = s.seq_lens[b] // s.page_size
        for g in range(s.num_kv_heads):
            assert band_ok(sel_g[b, g], sel_o[b, g], page_o[b, g, :f], min(k, f)), (b, g)


@pytest.mark.parametrize("scale", [16.0, 32.0])
def test_scan_codes_large_logits(scale):
    """Logits of tens to hundreds over codes (queries scaled up, page centroids
    offset): masses within 1e-4 of the oracle's estimate on the dequantised
    summary.  The scan sums each page's 2^logit shifted by the page's largest
    centroid term and takes the exact form (the page's max first) where that
    sum leaves [2^-60, 2^60]; at these scales both forms are taken, which the
    oracle's own values confirm below."""
    import kv_cache_page_rank_amd as lk
    case = Case(bf16_small(num_kv_heads=8, page_offset_std=4.0))
    s = case.spec
    codes = oracle.quantize_pool(*case.oracle_summaries())
    deq = oracle.dequantize_pool(*codes)
    q_host = (case.layer.q.astype(np.float64) * scale).astype(np.float32)
    head_o, page_o = oracle.scan_pool(case.lay, s.rank, q_host, *deq)
    shifted = shifted_log2_sums(case, q_host, deq[0], page_o)
    assert (shifted < 56).any()
    if scale >= 32:
        assert (shifted > 64).sum() >= 10
    say("scan codes large logits", scale, "shifted log2-sum range", shifted.min(), shifted.max())
    summ = codes_to_device(*codes)
    q = torch.from_numpy(q_host).to(DEV)
    pm = torch.empty((s.batch, s.num_kv_heads, s.max_pages), device=DEV)
    pm2 = torch.empty_like(pm)
    hm = torch.empty((s.batch, s.num_q_heads, s.max_pages), device=DEV)
    lk.locks_scan(q, summ, case.pages, pm, hm)
    lk.locks_scan(q, summ, case.pages, pm2)
    torch.cuda.synchronize()
    err = (masses_close(to_np(pm), page_o), masses_close(to_np(pm2), page_o),
           masses_close(to_np(hm), head_o))
    say("max |log-mass error|", *err)
    assert max(err) <= 1e-4
