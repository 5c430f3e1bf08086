"""GPU parity of the whole decode step on a batch of degenerate sequences:
an empty one, one shorter than a page (no full page, so nothing to select and
only the partial page to attend), one ordinary ragged sequence, and one whose
full pages all fit the budget (k = number of full pages).  Selection, sparse
attention on that selection, dense attention and the captured step are each
checked against the oracle or the eager calls."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import DEV, Case, band_ok, bf16_small, masses_close, out_tol, say, tiny, to_np
from workload.device import codes_to_device, summaries_to_device

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16-P64", lambda: bf16_small(batch=4, seq_lens=[0, 37, 64 * 20 + 5, 64 * 3], carriers=0),
     True),
    ("f32-P16-G4", lambda: tiny(batch=4, num_q_heads=4, seq_lens=[0, 9, 16 * 40 + 3, 16 * 2],
                                carriers=0), False),
]


def _check(out_g, lse_g, out_o, lse_o, bf16):
    err = np.abs(out_g - out_o)
    assert np.all(err <= out_tol(out_o, bf16)), float(err.max())
    fin = np.isfinite(lse_o)
    assert np.array_equal(fin, np.isfinite(lse_g))
    assert np.all(np.abs(lse_g[fin] - lse_o[fin]) <= (1e-4 if bf16 else 1e-5))


@pytest.mark.parametrize("name,mk,bf16", CASES, ids=[c[0] for c in CASES])
def test_degenerate_batch_step(name, mk, bf16):
    import kv_cache_page_rank_amd as lk
    case = Case(mk())
    s = case.spec
    P = s.page_size
    k = s.k_pages
    full = [n // P for n in s.seq_lens]
    mu, basis, coef = case.oracle_summaries()
    summ = summaries_to_device(mu, basis, coef)
    _, page_o = oracle.scan_pool(case.lay, s.rank, case.layer.q, mu, basis, coef, heads=False)
    sel_o, _ = oracle.select_pool(case.lay, s.budget_tokens, page_o.astype(np.float32), k)

    args = (s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads, P, s.head_dim, s.rank, k)
    sel = torch.full((s.batch, s.num_kv_heads, k), -9, dtype=torch.int32, device=DEV)
    mass = torch.zeros((s.batch, s.num_kv_heads, k), device=DEV)
    ws = lk.workspace(lk.workspace_bytes(lk.OP_STEP, *args))
    say("degenerate select", name, s.seq_lens)
    lk.locks_select(case.q, summ, case.pages, s.budget_tokens, sel, mass, ws=ws)
    torch.cuda.synchronize()
    sel_g, mass_g = sel.cpu().numpy(), mass.cpu().numpy()
    for b in range(s.batch):
        kb = min(k, full[b])
        for g in range(s.num_kv_heads):
            row = sel_g[b, g]
            # no full page: nothing selected; all full pages fit: all of them, in order
            if kb == 0:
                assert np.all(row == -1) and np.all(np.isneginf(mass_g[b, g])), (b, g)
            elif kb == full[b]:
                assert list(row[:kb]) == list(range(kb)), (b, g)
            assert band_ok(row, sel_o[b, g], page_o[b, g, :full[b]], kb), (b, g)
            assert list(row) == sorted(row[row >= 0]) + [-1] * int((row < 0).sum()), (b, g)

    # sparse attention on the device's own selection, against the oracle on
    # the same list (empty sequence: zero output and lse -inf)
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=case.kv.k.dtype, device=DEV)
    lse = torch.empty((s.batch, s.num_q_heads), device=DEV)
    sel_b = lk.workspace_bytes(lk.OP_SELECT, *args)
    say("degenerate sparse attend", name)
    lk.locks_sparse_attend(case.q, case.kv, case.pages, sel, out, lse, ws=ws[sel_b:])
    torch.cuda.synchronize()
    out_o, lse_o = oracle.attend_pool(case.lay, case.layer.q, case.k_f32, case.layer.v_f32(), sel_g)
    assert np.all(np.isneginf(lse_o[0])) and np.all(out_o[0] == 0.0)
    _check(to_np(out), lse.cpu().numpy(), out_o, lse_o, bf16)
    assert np.all(to_np(out)[0] == 0.0)

    # dense attention over every token
    dout = torch.empty_like(out)
    dlse = torch.empty_like(lse)
    dws = lk.workspace(lk.workspace_bytes(lk.OP_DENSE_ATTEND, *args[:-1], 0))
    say("degenerate dense attend", name)
    lk.locks_dense_attend(case.q, case.kv, case.pages, dout, dlse, ws=dws)
    torch.cuda.synchronize()
    dout_o, dlse_o = oracle.attend_pool(case.lay, case.layer.q, case.k_f32, case.layer.v_f32(), None)
    _check(to_np(dout), dlse.cpu().numpy(), dout_o, dlse_o, bf16)

    # the captured step replays to the eager results
    g = dict(sel=torch.full_like(sel, -9), mass=torch.zeros_like(mass), out=torch.zeros_like(out),
             lse=torch.zeros_like(lse), ws=lk.workspace(lk.workspace_bytes(lk.OP_STEP, *args)))
    graph = lk.StepGraph(case.q, summ, case.kv, case.pages, s.budget_tokens, g["sel"], g["mass"],
                         g["out"], g["lse"], ws=g["ws"])
    for rep in range(3):
        for t in (g["sel"], g["mass"], g["out"], g["lse"]):
            t.zero_()
        torch.cuda.synchronize()
        say("degenerate graph replay", name, rep)
        graph.launch()
        torch.cuda.synchronize()
        for key, ref in (("sel", sel), ("mass", mass), ("out", out), ("lse", lse)):
            assert torch.equal(g[key], ref), (rep, key)
    graph.close()


@pytest.mark.parametrize("sdt", ["bf16", "q8q4"])
@pytest.mark.parametrize("name,mk,bf16", CASES, ids=[c[0] for c in CASES])
def test_degenerate_batch_reduced_summaries(name, mk, bf16, sdt):
    """The same batches with bf16 and integer-code summaries: scan masses
    (per head and per group, -inf exactly where a page is not full) within
    1e-4 of the oracle on the same rounded or dequantised values, and the
    selection within the band of the oracle's selection from those masses."""
    import kv_cache_page_rank_amd as lk
    case = Case(mk())
    s = case.spec
    P, k = s.page_size, s.k_pages
    mu, basis, coef = case.oracle_summaries()
    if sdt == "q8q4":
        codes = oracle.quantize_pool(mu, basis, coef)
        vals = oracle.dequantize_pool(*codes)
        summ = codes_to_device(*codes)
    else:
        t = [torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
             for x in (mu, basis, coef)]
        vals = [x.float().numpy() for x in t]
        summ = lk.Summaries(*(x.to(DEV) for x in t))
    head_o, page_o = oracle.scan_pool(case.lay, s.rank, case.layer.q, *vals)
    pm = torch.full((s.batch, s.num_kv_heads, s.max_pages), 7.0, device=DEV)
    hm = torch.full((s.batch, s.num_q_heads, s.max_pages), 7.0, device=DEV)
    say("degenerate scan", name, sdt, s.seq_lens)
    lk.locks_scan(case.q, summ, case.pages, pm, hm)
    args = (s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads, P, s.head_dim, s.rank, k)
    sel = torch.full((s.batch, s.num_kv_heads, k), -9, dtype=torch.int32, device=DEV)
    mass = torch.zeros((s.batch, s.num_kv_heads, k), device=DEV)
    ws = lk.workspace(lk.workspace_bytes(lk.OP_STEP, *args))
    lk.locks_select(case.q, summ, case.pages, s.budget_tokens, sel, mass, ws=ws)
    torch.cuda.synchronize()
    assert masses_close(to_np(pm), page_o) <= 1e-4
    assert masses_close(to_np(hm), head_o) <= 1e-4
    sel_o, _ = oracle.select_pool(case.lay, s.budget_tokens, page_o.astype(np.float32), k)
    sel_g = sel.cpu().numpy()
    for b in range(s.batch):
        f = s.seq_lens[b] // P
        kb = min(k, f)
        for g in range(s.num_kv_heads):
            if kb == 0:
                assert np.all(sel_g[b, g] == -1), (b, g)
                continue
            assert np.all(sel_g[b, g, kb:] == -1), (b, g)
            assert band_ok(sel_g[b, g], sel_o[b, g], page_o[b, g, :f], kb), (b, g)
