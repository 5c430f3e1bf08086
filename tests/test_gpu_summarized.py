"""Pages whose summaries are not built yet (technical summary, section 2: a
page's summary is made once the page is final, off the attention's critical
path): with a per-sequence count of summarised pages in the page table, the
scan, the mean-of-share totals and the selection see only the pages below
the count, and attention covers the selected pages plus every page from the
count to the end.  Checked against the oracle on the same count, for the
one-workgroup-per-page sparse kernel, the wave-per-run kernel (including a
tail longer than one wave's 64 lanes), fp32 caches, and both group
aggregations."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import DEV, Case, band_ok, bf16_small, masses_close, out_tol, say, tiny, to_np
from workload.device import summaries_to_device

pytestmark = pytest.mark.gpu


def _layout(case, counts):
    s = case.spec
    return oracle.Layout(s.num_q_heads, s.num_kv_heads, s.head_dim, s.page_size,
                         case.layer.block_table, case.layer.seq_lens,
                         summarized=np.asarray(counts, np.int32))


@pytest.mark.parametrize("name,mk,counts", [
    ("per-page kernel, 3 pending + partial, none summarised",
     lambda: bf16_small(), [37, 0]),
    ("wave-per-run kernel, a tail of 71 pages",
     lambda: bf16_small(seq_lens=[64 * 150 + 5, 64 * 100], num_kv_heads=8, num_q_heads=32,
                        budget_tokens=4096), [80, 100]),
    ("fp32 cache", lambda: tiny(num_q_heads=4, seq_lens=[16 * 40 + 3]), [31]),
], ids=["per-page", "wave-per-run-long-tail", "fp32"])
@pytest.mark.parametrize("agg", [0, 1], ids=["lse", "mean-share"])
def test_summarised_count_matches_oracle(name, mk, counts, agg):
    import kv_cache_page_rank_amd as lk
    case = Case(mk())
    s = case.spec
    k = s.k_pages
    G = s.group
    lay_s = _layout(case, counts)
    # the oracle's summaries of every full page (those past the count are
    # present but must not be read)
    mu, basis, coef = case.oracle_summaries()
    summ = summaries_to_device(mu, basis, coef, DEV)
    pages = lk.PageTable(case.pages.block_table, case.pages.seq_lens,
                         torch.tensor(counts, dtype=torch.int32, device=DEV))
    head_o, page_o = oracle.scan_pool(lay_s, s.rank, case.layer.q, mu, basis, coef)
    if agg == 1:
        page_o = oracle.share_pool(lay_s, head_o)
    sel_o, _ = oracle.select_pool(lay_s, s.budget_tokens, page_o.astype(np.float32), k)

    sel = torch.empty((s.batch, s.num_kv_heads, k), dtype=torch.int32, device=DEV)
    mass = torch.empty((s.batch, s.num_kv_heads, k), device=DEV)
    pm = torch.empty((s.batch, s.num_kv_heads, s.max_pages), device=DEV)
    ws = lk.workspace(lk.workspace_bytes(lk.OP_STEP, s.batch, s.max_pages, s.num_q_heads,
                                         s.num_kv_heads, s.page_size, s.head_dim, s.rank, k))
    say("summarised count: select", name, counts, "agg", agg)
    lk.locks_select(case.q, summ, pages, s.budget_tokens, sel, mass, page_logmass=pm, ws=ws,
                    agg=agg)
    torch.cuda.synchronize()
    assert masses_close(to_np(pm), page_o) <= 1e-4
    sel_np = to_np(sel)
    for b in range(s.batch):
        cand = min(counts[b], s.seq_lens[b] // s.page_size)
        for g in range(s.num_kv_heads):
            got = sel_np[b, g]
            assert np.all(got[got >= 0] < cand)
            assert band_ok(got, sel_o[b, g], page_o[b, g, :cand], min(k, cand)), (b, g)

    out = torch.empty((s.batch, s.num_q_heads, s.head_dim),
                      dtype=torch.bfloat16 if s.kv_bf16 else torch.float32, device=DEV)
    lse = torch.empty((s.batch, s.num_q_heads), device=DEV)
    sel_b = lk.workspace_bytes(lk.OP_SELECT, s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads,
                               s.page_size, s.head_dim, s.rank, k)
    say("summarised count: sparse attention", name)
    lk.locks_sparse_attend(case.q, case.kv, pages, sel, out, lse, ws=ws[sel_b:])
    torch.cuda.synchronize()
    o_o, l_o = oracle.attend_pool(lay_s, case.layer.q, case.k_f32, case.layer.v_f32(), sel_np)
    got = to_np(out).astype(np.float64)
    assert np.all(np.abs(got - o_o) <= out_tol(o_o, s.kv_bf16)), float(np.abs(got - o_o).max())
    assert np.abs(to_np(lse) - l_o).max() <= 1e-4
    # the count changes the answer: without it the pending pages would compete
    if counts[0] < s.seq_lens[0] // s.page_size:
        _, page_all = oracle.scan_pool(case.lay, s.rank, case.layer.q, mu, basis, coef)
        assert np.isfinite(page_all[0, 0, counts[0]])
        assert np.isneginf(page_o[0, 0, counts[0]])


def test_summarised_count_graph_equals_eager():
    """The captured step with a count equals the eager calls, replay after
    replay, as the count moves."""
    import kv_cache_page_rank_amd as lk
    case = Case(bf16_small())
    s = case.spec
    k = s.k_pages
    summ = lk.Summaries.empty(s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim, s.rank)
    lk.locks_build_summaries(case.kv, case.pages, summ)
    counts = torch.tensor([40, 23], dtype=torch.int32, device=DEV)
    pages = lk.PageTable(case.pages.block_table, case.pages.seq_lens, counts)
    args = (s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads, s.page_size, s.head_dim, s.rank,
            k)
    mk = lambda: dict(sel=torch.empty((s.batch, s.num_kv_heads, k), dtype=torch.int32, device=DEV),
                      mass=torch.empty((s.batch, s.num_kv_heads, k), device=DEV),
                      out=torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.bfloat16,
                                      device=DEV),
                      lse=torch.empty((s.batch, s.num_q_heads), device=DEV),
                      ws=lk.workspace(lk.workspace_bytes(lk.OP_STEP, *args)))
    g, e = mk(), mk()
    graph = lk.StepGraph(case.q, summ, case.kv, pages, s.budget_tokens, g["sel"], g["mass"],
                         g["out"], g["lse"], ws=g["ws"])
    sel_b = lk.workspace_bytes(lk.OP_SELECT, *args)
    for rep, c in enumerate(([40, 23], [35, 23], [0, 20], [40, 23])):
        counts.copy_(torch.tensor(c, dtype=torch.int32))
        say("summarised count: graph replay", rep, c)
        graph.launch()
        lk.locks_select(case.q, summ, pages, s.budget_tokens, e["sel"], e["mass"], ws=e["ws"])
        lk.locks_sparse_attend(case.q, case.kv, pages, e["sel"], e["out"], e["lse"],
                               ws=e["ws"][sel_b:])
        torch.cuda.synchronize()
        for key in ("sel", "mass", "out", "lse"):
            assert torch.equal(g[key], e[key]), (rep, key)
    graph.close()
