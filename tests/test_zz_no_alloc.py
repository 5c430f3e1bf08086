"""locks_select_noalloc (no workspace argument; the library's static
per-device scratch) against locks_select with a caller workspace, through
the C ABI: identical selections, selected masses and page masses, bit for
bit, for both group aggregations, with and without a caller page-mass
array, on two calls in a row, the second on a smaller input."""
import numpy as np
import pytest
import torch

from gpu_cases import DEV, Case, bf16_small, say, tiny

pytestmark = pytest.mark.gpu


def _build(lk, case):
    s = case.spec
    summ = lk.Summaries.empty(s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim, s.rank)
    lk.locks_build_summaries(case.kv, case.pages, summ)
    torch.cuda.synchronize()
    return summ


def _select(lk, case, summ, agg, noalloc, with_pm):
    s = case.spec
    k = s.k_pages
    sel = torch.full((s.batch, s.num_kv_heads, k), -7, dtype=torch.int32, device=DEV)
    mass = torch.full((s.batch, s.num_kv_heads, k), 7.0, device=DEV)
    pm = torch.full((s.batch, s.num_kv_heads, s.max_pages), 7.0, device=DEV) if with_pm else None
    if noalloc:
        lk.locks_select_noalloc(case.q, summ, case.pages, s.budget_tokens, sel, mass,
                                page_logmass=pm, agg=agg)
    else:
        ws = lk.workspace(lk.workspace_bytes(lk.OP_SELECT, s.batch, s.max_pages, s.num_q_heads,
                                             s.num_kv_heads, s.page_size, s.head_dim, s.rank, k))
        lk.locks_select(case.q, summ, case.pages, s.budget_tokens, sel, mass, page_logmass=pm,
                        ws=ws, agg=agg)
    torch.cuda.synchronize()
    return sel.cpu(), mass.cpu(), None if pm is None else pm.cpu()


def _same(a, b):
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_select_noalloc_equals_select_with_workspace():
    import kv_cache_page_rank_amd as lk
    big = Case(bf16_small(seq_lens=[64 * 300 + 5, 64 * 180], budget_tokens=2048))
    small = Case(tiny(num_q_heads=4, seq_lens=[16 * 40 + 3]))
    for name, case in (("larger", big), ("smaller", small)):
        summ = _build(lk, case)
        for agg in (lk.AGG_LSE, lk.AGG_MEAN_SHARE):
            for with_pm in (True, False):
                say("no-alloc select", name, case.spec.name, "agg", agg, "page masses", with_pm)
                ref = _select(lk, case, summ, agg, False, with_pm)
                got = _select(lk, case, summ, agg, True, with_pm)
                _same(got, ref)
                sel = got[0].numpy()
                assert np.all(sel[sel >= 0] < case.spec.max_pages)
                assert (sel >= 0).any()
