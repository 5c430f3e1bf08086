"""Summaries kept current inside the decode graph: a step whose new token
completes a page refreshes that page's summary before the scan reads it
(technical summary, section 2: a page's summary is made once the page is
final).  The refreshed summaries must equal a full build of the new state,
and the step's selection and attention the eager calls on them."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import DEV, Case, bf16_small, say

pytestmark = pytest.mark.gpu


def _build(lk, case, lens=None):
    s = case.spec
    summ = lk.Summaries.empty(s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim, s.rank)
    lk.locks_build_summaries(case.kv, case.pages, summ)
    return summ


def _full_blocks(case):
    lens = case.pages.seq_lens.cpu().numpy()
    bt = case.layer.block_table
    return np.concatenate([bt[b, :lens[b] // case.spec.page_size] for b in range(len(lens))])


@pytest.mark.parametrize("agg", [0, 1], ids=["lse", "mean-share"])
def test_refresh_in_graph_tracks_page_crossing(agg):
    import kv_cache_page_rank_amd as lk
    P = 64
    # one token short of a page boundary in both sequences; the slots past the
    # end hold real keys (no poison) so that the next token's key is present
    case = Case(bf16_small(seq_lens=[P * 40 + 63, P * 23 + 63], poison_tail=False))
    s = case.spec
    k = s.k_pages
    say("refresh: initial build", agg)
    summ = _build(lk, case)
    torch.cuda.synchronize()
    begin = torch.tensor([40, 23], dtype=torch.int32, device=DEV)  # full pages before the step
    ws_b = lk.workspace_bytes(lk.OP_STEP, s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads,
                              P, s.head_dim, s.rank, k)
    g = dict(sel=torch.empty((s.batch, s.num_kv_heads, k), dtype=torch.int32, device=DEV),
             mass=torch.empty((s.batch, s.num_kv_heads, k), device=DEV),
             out=torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.bfloat16, device=DEV),
             lse=torch.empty((s.batch, s.num_q_heads), device=DEV), ws=lk.workspace(ws_b))
    graph = lk.StepGraph(case.q, summ, case.kv, case.pages, s.budget_tokens, g["sel"], g["mass"],
                         g["out"], g["lse"], ws=g["ws"], agg=agg, refresh_begin=begin,
                         refresh_pages=1)
    # the decode step appends one token: both sequences complete a page
    case.pages.seq_lens += 1
    say("refresh: graph replay across the page boundary")
    graph.launch()
    torch.cuda.synchronize()
    ref = _build(lk, case)
    torch.cuda.synchronize()
    blocks = torch.from_numpy(_full_blocks(case).astype(np.int64)).to(DEV)
    for got, want in ((summ.mu, ref.mu), (summ.basis, ref.basis), (summ.coef, ref.coef)):
        assert torch.equal(got[blocks].view(torch.int32), want[blocks].view(torch.int32))
    # the refreshed pages against the oracle's build of the new state
    _check_refreshed_against_oracle(case, summ, [(0, 40), (1, 23)])
    # the step's outputs equal the eager calls on fully rebuilt summaries
    e = {key: torch.empty_like(v) for key, v in g.items()}
    lk.locks_select(case.q, ref, case.pages, s.budget_tokens, e["sel"], e["mass"], ws=e["ws"],
                    agg=agg)
    sel_b = lk.workspace_bytes(lk.OP_SELECT, s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads,
                               P, s.head_dim, s.rank, k)
    lk.locks_sparse_attend(case.q, case.kv, case.pages, e["sel"], e["out"], e["lse"],
                           ws=e["ws"][sel_b:])
    torch.cuda.synchronize()
    for key in ("sel", "mass", "out", "lse"):
        assert torch.equal(g[key], e[key]), key
    # a step that completes no page leaves every summary as it is
    before = [t.clone() for t in (summ.mu, summ.basis, summ.coef)]
    begin.copy_(torch.tensor([41, 24], dtype=torch.int32))
    case.pages.seq_lens += 1
    say("refresh: graph replay inside a page")
    graph.launch()
    torch.cuda.synchronize()
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
