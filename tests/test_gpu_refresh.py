"""Summaries of pages that became final during decoding, built off the
step's critical path (technical summary, section 2: a page's summary is made
once the page is final, off the attention's critical path).  A step whose
new token completes a page attends that page outside the budget (the page
table's count of summarised pages has not reached it); the refresh, on a
side stream, builds the page's summaries and then advances the count, and
later steps see the page as a candidate.  Every stage is checked against the
oracle on the same count, and the captured step against the eager calls."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import DEV, Case, band_ok, bf16_small, masses_close, say, to_np

pytestmark = pytest.mark.gpu


def _build(lk, case):
    s = case.spec
    summ = lk.Summaries.empty(s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim, s.rank)
    lk.locks_build_summaries(case.kv, case.pages, summ)
    return summ


def _oracle_step(case, summ, counts, k, budget):
    """The oracle's scan (of the library's summaries), selection and the
    attention over a given page list, on the device's current lengths."""
    s = case.spec
    lens = case.pages.seq_lens.cpu().numpy().astype(np.int32)
    lay = oracle.Layout(s.num_q_heads, s.num_kv_heads, s.head_dim, s.page_size,
                        case.layer.block_table, lens, summarized=np.asarray(counts, np.int32))
    mu, basis, coef = (t.cpu().numpy() for t in (summ.mu, summ.basis, summ.coef))
    _, page = oracle.scan_pool(lay, s.rank, case.layer.q, mu, basis, coef)
    sel, _ = oracle.select_pool(lay, budget, page.astype(np.float32), k)
    return lay, page, sel


@pytest.mark.parametrize("agg", [0, 1], ids=["lse", "mean-share"])
def test_refresh_off_the_step_path(agg):
    import kv_cache_page_rank_amd as lk
    P = 64
    # one token short of a page boundary in both sequences; the slots past the
    # end hold real keys (no poison) so that the next token's key is present
    case = Case(bf16_small(seq_lens=[P * 40 + 63, P * 23 + 63], poison_tail=False))
    s = case.spec
    k = s.k_pages
    say("refresh: initial build", agg)
    summ = _build(lk, case)
    counts = torch.tensor([40, 23], dtype=torch.int32, device=DEV)
    pages = lk.PageTable(case.pages.block_table, case.pages.seq_lens, counts)
    torch.cuda.synchronize()
    args = (s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads, P, s.head_dim, s.rank, k)
    mk = lambda: dict(sel=torch.empty((s.batch, s.num_kv_heads, k), dtype=torch.int32, device=DEV),
                      mass=torch.empty((s.batch, s.num_kv_heads, k), device=DEV),
                      out=torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.bfloat16,
                                      device=DEV),
                      lse=torch.empty((s.batch, s.num_q_heads), device=DEV),
                      pm=torch.empty((s.batch, s.num_kv_heads, s.max_pages), device=DEV),
                      ws=lk.workspace(lk.workspace_bytes(lk.OP_STEP, *args)))
    g, e = mk(), mk()
    graph = lk.StepGraph(case.q, summ, case.kv, pages, s.budget_tokens, g["sel"], g["mass"],
                         g["out"], g["lse"], page_logmass=g["pm"], ws=g["ws"], agg=agg)
    sel_b = lk.workspace_bytes(lk.OP_SELECT, *args)

    def step_and_check(stage, cnt):
        say("refresh:", stage, cnt)
        graph.launch()
        lk.locks_select(case.q, summ, pages, s.budget_tokens, e["sel"], e["mass"],
                        page_logmass=e["pm"], ws=e["ws"], agg=agg)
        lk.locks_sparse_attend(case.q, case.kv, pages, e["sel"], e["out"], e["lse"],
                               ws=e["ws"][sel_b:])
        torch.cuda.synchronize()
        for key in ("sel", "mass", "out", "lse", "pm"):
            assert torch.equal(g[key], e[key]), (stage, key)
        lay, page, sel_o = _oracle_step(case, summ, cnt, k, s.budget_tokens)
        if agg == 1:
            head, _ = oracle.scan_pool(lay, s.rank, case.layer.q,
                                       *(t.cpu().numpy() for t in (summ.mu, summ.basis, summ.coef)))
            page = oracle.share_pool(lay, head)
            sel_o, _ = oracle.select_pool(lay, s.budget_tokens, page.astype(np.float32), k)
        assert masses_close(to_np(g["pm"]), page) <= 1e-4
        sel = to_np(g["sel"])
        for b in range(s.batch):
            for gg in range(s.num_kv_heads):
                assert band_ok(sel[b, gg], sel_o[b, gg], page[b, gg, :cnt[b]], min(k, cnt[b]))
        o_o, l_o = oracle.attend_pool(lay, case.layer.q, case.k_f32, case.layer.v_f32(), sel)
        got = to_np(g["out"]).astype(np.float64)
        assert np.all(np.abs(got - o_o) <= np.maximum(1e-2, 2.0 ** (np.floor(
            np.log2(np.maximum(np.abs(o_o), 1e-30))) - 7)))
        assert np.abs(to_np(g["lse"]) - l_o).max() <= 1e-4
        return sel

    # the decode step appends one token: both sequences complete a page, whose
    # summary does not exist yet - the step attends it outside the budget
    case.pages.seq_lens += 1
    sel = step_and_check("step with the new pages pending", [40, 23])
    assert np.all(sel[0][sel[0] >= 0] < 40) and np.all(sel[1][sel[1] >= 0] < 23)
    # the refresh on a side stream builds the new pages and then moves the count
    side = torch.cuda.Stream()
    begin = counts.clone()
    with torch.cuda.stream(side):
        say("refresh: side-stream build of the new pages")
        lk.locks_refresh_summaries(case.kv, pages, begin, 1, summ, stream=side)
    side.synchronize()
    assert counts.cpu().tolist() == [41, 24]
    _check_refreshed_against_oracle(case, summ, [(0, 40), (1, 23)])
    step_and_check("step after the refresh", [41, 24])
    # a token inside a page: the refresh finds no new full page, nothing moves
    before = [t.clone() for t in (summ.mu, summ.basis, summ.coef)]
    case.pages.seq_lens += 1
    begin.copy_(counts)
    lk.locks_refresh_summaries(case.kv, pages, begin, 1, summ)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [41, 24]
    for a, b in zip(before, (summ.mu, summ.basis, summ.coef)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    graph.close()


def _check_refreshed_against_oracle(case, summ, pages):
    """The oracle's gap-independent checks (centroid, orthonormal basis,
    coordinate residual, captured energy) and, where the spectral gap allows,
    the reconstructed logits, on the refreshed (b, j) pages of every KV head,
    with the sequence lengths the step left on the device."""
    from test_gpu_build import _check_units
    s = case.spec
    lens = case.pages.seq_lens.cpu().numpy().astype(np.int32)
    view = type("RefreshedCase", (), {})()
    view.spec = s.with_(seq_lens=[int(x) for x in lens])
    view.layer = case.layer
    view.k_f32 = case.k_f32
    view.lay = oracle.Layout(s.num_q_heads, s.num_kv_heads, s.head_dim, s.page_size,
                             case.layer.block_table, lens)
    units = np.array([[b, g, j] for b, j in pages for g in range(s.num_kv_heads)], np.int32)
    say("refresh: refreshed pages against the oracle", units.tolist())
    _check_units(view, summ, units, s.rank)


def test_refresh_entry_builds_only_the_window():
    """locks_refresh_summaries builds pages page_begin[b] .. + max_new_pages - 1
    (bounded by the full pages) and nothing else, identically to the full build."""
    import kv_cache_page_rank_amd as lk
    case = Case(bf16_small())
    s = case.spec
    ref = _build(lk, case)
    summ = lk.Summaries.empty(s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim, s.rank)
    for t in (summ.mu, summ.basis, summ.coef):
        t.fill_(float("nan"))
    begin = torch.tensor([5, 21], dtype=torch.int32, device=DEV)
    say("refresh window")
    lk.locks_refresh_summaries(case.kv, case.pages, begin, 3, summ)
    torch.cuda.synchronize()
    full = [n // s.page_size for n in s.seq_lens]
    bt = case.layer.block_table
    inside = {int(bt[b, j]) for b, lo in enumerate([5, 21]) for j in range(lo, min(lo + 3, full[b]))}
    for blk in range(s.num_blocks):
        got = summ.basis[blk]
        if blk in inside:
            assert torch.equal(got.view(torch.int32), ref.basis[blk].view(torch.int32))
        else:
            assert torch.isnan(got).all()
    _check_refreshed_against_oracle(case, summ, [(b, j) for b, lo in enumerate([5, 21])
                                                 for j in range(lo, min(lo + 3, full[b]))])
