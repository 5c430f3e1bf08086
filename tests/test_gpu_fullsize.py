"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times, on outputs the oracle can compute one by one (sampled
pages, sampled heads) and on properties that hold at any size."""
import math

import numpy as np
import pytest
import torch

import oracle
import workload
from gpu_cases import DEV, SubPool, bf16_ulp, say
from workload.device import upload

pytestmark = pytest.mark.gpu


class Full:
    def __init__(self, idx):
        import kv_cache_page_rank_amd as lk
        self.spec = workload.config(idx)
        say("generate", self.spec.name)
        self.layer = workload.make(self.spec, threads=16)
        self.q, self.kv, self.pages = upload(self.layer, DEV)
        s = self.spec
        self.summ = lk.Summaries.empty(s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim,
                                       s.rank)
        say("build", s.name)
        lk.locks_build_summaries(self.kv, self.pages, self.summ)
        torch.cuda.synchronize()
        self.rng = np.random.default_rng(idx)


@pytest.fixture(scope="module", params=[2, 1, 3, 4], ids=["glm-1m", "llama-128k", "glm-1m-r2",
                                                        "qwen-batch16"])
def full(request):
    f = Full(request.param)
    yield f
    del f
    torch.cuda.empty_cache()


def _sample_pages(f, b, g, n_rand=12):
    s = f.spec
    nfull = s.seq_lens[b] // s.page_size
    pages = set(f.rng.choice(nfull, min(n_rand, nfull), replace=False).tolist())
    pages |= set(int(x) for x in f.layer.carrier_page[b, g][:4])
    pages |= {0, nfull - 1}
    return sorted(pages)


def test_fullsize_build_sampled(full):
    """Factors of sampled pages (random + carrier + first/last): unique
    quantities against the oracle (see test_gpu_build)."""
    from test_gpu_build import _check_units
    f, s = full, full.spec
    for b in sorted({0, s.batch - 1}):
        for g in sorted({0, s.num_kv_heads - 1}):
            sub = SubPool(f.layer, s, b, g)
            pages = _sample_pages(f, b, g, 6)

            class _C:  # the view _check_units expects, on the sub-pool
                pass
            c = _C()
            c.spec = s.with_(batch=1, num_kv_heads=1, num_q_heads=s.group,
                             seq_lens=[s.seq_lens[b]])
            c.layer = type("L", (), {})()
            c.layer.block_table = np.arange(len(sub.blocks), dtype=np.int32)[None]
            c.layer.q = sub.q
            c.k_f32 = sub.k
            c.lay = sub.lay
            blk = sub.blocks

            class _S:
                pass
            summ = _S()
            summ.mu = f.summ.mu[torch.from_numpy(blk.astype(np.int64)).to(DEV), g][:, None]
            summ.basis = f.summ.basis[torch.from_numpy(blk.astype(np.int64)).to(DEV), g][:, None]
            summ.coef = f.summ.coef[torch.from_numpy(blk.astype(np.int64)).to(DEV), g][:, None]
            say("fullsize build check", s.name, b, g, pages)
            _check_units(c, summ, sub.units(pages), s.rank)


def test_fullsize_scan_sampled(full):
    """Scan over every page of the layer, with the oracle's summaries placed
    at sampled pages: those pages' masses (per head and per group) match the
    oracle within 1e-4; every page past the full ones is -inf."""
    import kv_cache_page_rank_amd as lk
    f, s = full, full.spec
    summ = lk.Summaries(f.summ.mu.clone(), f.summ.basis.clone(), f.summ.coef.clone())
    checks = []
    for b in sorted({0, s.batch - 1}):
        for g in range(s.num_kv_heads):
            sub = SubPool(f.layer, s, b, g)
            pages = _sample_pages(f, b, g)
            mu, basis, coef, _ = oracle.build_units(sub.lay, s.rank, sub.k, sub.units(pages))
            mu32, basis32, coef32 = (x.astype(np.float32) for x in (mu, basis, coef))
            idx = torch.from_numpy(f.layer.block_table[b, pages].astype(np.int64)).to(DEV)
            summ.mu[idx, g] = torch.from_numpy(mu32).to(DEV)
            summ.basis[idx, g] = torch.from_numpy(basis32).to(DEV)
            summ.coef[idx, g] = torch.from_numpy(coef32).to(DEV)
            # oracle scan of exactly those fp32 summaries (compact single-group layout)
            n = len(pages)
            lay = oracle.Layout(s.group, 1, s.head_dim, s.page_size,
                                np.arange(n, dtype=np.int32)[None],
                                np.array([n * s.page_size], np.int32))
            head_o, page_o = oracle.scan_pool(lay, s.rank, sub.q, mu32[:, None], basis32[:, None],
                                              coef32[:, None])
            checks.append((b, g, pages, head_o[0, :, :n], page_o[0, 0, :n]))
    pm = torch.empty((s.batch, s.num_kv_heads, s.max_pages), device=DEV)
    hm = torch.empty((s.batch, s.num_q_heads, s.max_pages), device=DEV)
    say("fullsize scan", s.name)
    lk.locks_scan(f.q, summ, f.pages, pm, hm)
    torch.cuda.synchronize()
    pm, hm = pm.cpu().numpy(), hm.cpu().numpy()
    G = s.group
    for b, g, pages, head_o, page_o in checks:
        assert np.abs(pm[b, g, pages] - page_o).max() <= 1e-4
        assert np.abs(hm[b, g * G:(g + 1) * G][:, pages] - head_o).max() <= 1e-4
    for b in range(s.batch):
        nfull = s.seq_lens[b] // s.page_size
        assert np.all(np.isneginf(pm[b, :, nfull:]))
        assert np.all(np.isfinite(pm[b, :, :nfull]))


def test_fullsize_scan_codes_sampled(full):
    """Scan of int8 / int4 codes (the layer's summaries quantised on the
    device) over every page of the layer, in the launch configuration the
    benchmark times: sampled pages' masses, per head and per group, with and
    without per-head output, within 1e-4 of the oracle's estimate on the same
    codes dequantised; every page past the full ones is -inf."""
    import kv_cache_page_rank_amd as lk
    f, s = full, full.spec
    codes = lk.Summaries.empty(s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim, s.rank,
                               dtype=lk.Q8Q4)
    say("fullsize quantise", s.name)
    lk.locks_quantize_summaries(f.summ, codes)
    pm = torch.empty((s.batch, s.num_kv_heads, s.max_pages), device=DEV)
    hm = torch.empty((s.batch, s.num_q_heads, s.max_pages), device=DEV)
    pm2 = torch.empty_like(pm)
    say("fullsize scan of codes", s.name)
    lk.locks_scan(f.q, codes, f.pages, pm, hm)
    lk.locks_scan(f.q, codes, f.pages, pm2)
    torch.cuda.synchronize()
    pm, hm, pm2 = pm.cpu().numpy(), hm.cpu().numpy(), pm2.cpu().numpy()
    G = s.group
    for b in sorted({0, s.batch - 1}):
        for g in range(s.num_kv_heads):
            sub = SubPool(f.layer, s, b, g)
            pages = _sample_pages(f, b, g)
            idx = torch.from_numpy(f.layer.block_table[b, pages].astype(np.int64)).to(DEV)
            unit = [t[idx, g][:, None].cpu().numpy()
                    for t in (codes.mu, codes.basis, codes.coef, codes.scales)]
            n = len(pages)
            lay = oracle.Layout(s.group, 1, s.head_dim, s.page_size,
                                np.arange(n, dtype=np.int32)[None],
                                np.array([n * s.page_size], np.int32))
            head_o, page_o = oracle.scan_pool(lay, s.rank, sub.q, *oracle.dequantize_pool(*unit))
            assert np.abs(pm[b, g, pages] - page_o[0, 0, :n]).max() <= 1e-4
            assert np.abs(pm2[b, g, pages] - page_o[0, 0, :n]).max() <= 1e-4
            assert np.abs(hm[b, g * G:(g + 1) * G][:, pages] - head_o[0, :, :n]).max() <= 1e-4
    for b in range(s.batch):
        nfull = s.seq_lens[b] // s.page_size
        assert np.all(np.isneginf(pm[b, :, nfull:]))
        assert np.all(np.isfinite(pm[b, :, :nfull]))


def _brute_topk(mass, k):
    order = np.lexsort((np.arange(mass.size), -mass.astype(np.float64)))
    return np.sort(order[:k])


def test_fullsize_select_is_topk_of_masses(full):
    """At full size, for every budget: the selection is exactly the top-k of
    the page masses the same call produced (ties to the lower page), in
    ascending order, with those masses.  The carriers' rank is reported."""
    import kv_cache_page_rank_amd as lk
    f, s = full, full.spec
    for budget in (s.budgets or [s.budget_tokens]):
        k = budget // s.page_size
        sel = torch.empty((s.batch, s.num_kv_heads, k), dtype=torch.int32, device=DEV)
        mass = torch.empty((s.batch, s.num_kv_heads, k), device=DEV)
        pm = torch.empty((s.batch, s.num_kv_heads, s.max_pages), device=DEV)
        say("fullsize select", s.name, budget)
        lk.locks_select(f.q, f.summ, f.pages, budget, sel, mass, page_logmass=pm)
        torch.cuda.synchronize()
        sel, mass, pm = sel.cpu().numpy(), mass.cpu().numpy(), pm.cpu().numpy()
        kept = total = 0
        for b in range(s.batch):
            nfull = s.seq_lens[b] // s.page_size
            for g in range(s.num_kv_heads):
                ref = _brute_topk(pm[b, g, :nfull], min(k, nfull))
                np.testing.assert_array_equal(sel[b, g, :ref.size], ref)
                np.testing.assert_array_equal(mass[b, g, :ref.size], pm[b, g, ref])
                kept += len(set(f.layer.carrier_page[b, g].tolist()) & set(ref.tolist()))
                total += f.layer.carrier_page.shape[-1]
        print(f"[carrier recall] {s.name} budget {budget}: {kept}/{total}", flush=True)


def test_fullsize_attend_sampled(full):
    """Sparse attention over a seeded page list and dense attention over every
    token, at full size, against the oracle for sampled sequences/groups."""
    import kv_cache_page_rank_amd as lk
    f, s = full, full.spec
    k = s.k_pages
    sel = np.full((s.batch, s.num_kv_heads, k), -1, np.int32)
    for b in range(s.batch):
        nfull = s.seq_lens[b] // s.page_size
        for g in range(s.num_kv_heads):
            sel[b, g] = np.sort(f.rng.choice(nfull, k, replace=False))
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((s.batch, s.num_q_heads), device=DEV)
    ws = lk.workspace(lk.workspace_bytes(lk.OP_SPARSE_ATTEND, s.batch, s.max_pages, s.num_q_heads,
                                         s.num_kv_heads, s.page_size, s.head_dim, s.rank, k))
    say("fullsize sparse attend", s.name)
    lk.locks_sparse_attend(f.q, f.kv, f.pages, torch.from_numpy(sel).to(DEV), out, lse, ws=ws)
    dout = torch.empty_like(out)
    dlse = torch.empty_like(lse)
    dws = lk.workspace(lk.workspace_bytes(lk.OP_DENSE_ATTEND, s.batch, s.max_pages,
                                          s.num_q_heads, s.num_kv_heads, s.page_size, s.head_dim,
                                          s.rank, 0))
    say("fullsize dense attend", s.name)
    lk.locks_dense_attend(f.q, f.kv, f.pages, dout, dlse, ws=dws)
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    dout, dlse = dout.float().cpu().numpy(), dlse.cpu().numpy()
    G = s.group
    for b in sorted({0, s.batch - 1}):
        for g in sorted({0, s.num_kv_heads - 1}):
            sub = SubPool(f.layer, s, b, g)
            o_s, l_s = oracle.attend_pool(sub.lay, sub.q, sub.k, sub.v,
                                          sel[b:b + 1, g:g + 1], threads=16)
            o_d, l_d = oracle.attend_pool(sub.lay, sub.q, sub.k, sub.v, None, threads=16)
            hs = slice(g * G, (g + 1) * G)
            for got, ref in ((out[b, hs], o_s[0]), (dout[b, hs], o_d[0])):
                assert np.all(np.abs(got - ref) <= np.maximum(1e-2, bf16_ulp(ref)))
            assert np.abs(lse[b, hs] - l_s[0]).max() <= 1e-4
            assert np.abs(dlse[b, hs] - l_d[0]).max() <= 1e-4


def test_fullsize_graph_step_equals_eager(full):
    """The benchmark's step (one captured graph) equals the eager calls."""
    import kv_cache_page_rank_amd as lk
    f, s = full, full.spec
    k = s.k_pages
    args = (s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads, s.page_size, s.head_dim, s.rank,
            k)
    bufs = [dict(sel=torch.empty((s.batch, s.num_kv_heads, k), dtype=torch.int32, device=DEV),
                 mass=torch.empty((s.batch, s.num_kv_heads, k), device=DEV),
                 out=torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=torch.bfloat16,
                                 device=DEV),
                 lse=torch.empty((s.batch, s.num_q_heads), device=DEV),
                 ws=lk.workspace(lk.workspace_bytes(lk.OP_STEP, *args))) for _ in range(2)]
    e, g = bufs
    say("fullsize eager step", s.name)
    lk.locks_select(f.q, f.summ, f.pages, s.budget_tokens, e["sel"], e["mass"], ws=e["ws"])
    sel_b = lk.workspace_bytes(lk.OP_SELECT, *args)
    lk.locks_sparse_attend(f.q, f.kv, f.pages, e["sel"], e["out"], e["lse"], ws=e["ws"][sel_b:])
    graph = lk.StepGraph(f.q, f.summ, f.kv, f.pages, s.budget_tokens, g["sel"], g["mass"],
                         g["out"], g["lse"], ws=g["ws"])
    for rep in range(3):
        say("fullsize graph replay", s.name, rep)
        graph.launch()
        torch.cuda.synchronize()
        for key in ("sel", "mass", "out", "lse"):
            assert torch.equal(g[key], e[key]), (rep, key)
    graph.close()


def _lse(x):
    x = np.asarray(x, np.float64)
    m = x.max()
    return m + math.log(np.exp(x - m).sum())


def test_fullsize_agreement_with_exact_selection(full):
    """Reported, not gated: for each budget, how the summary-based selection
    compares with the selection that reads every key (the exact page LSE,
    aggregated over the group the same way): recall of the exact top-k, the
    share of the exact top-k's mass that the selection captures, carrier
    recall, and the largest difference between sparse and dense outputs
    (every sequence of the batch)."""
    import kv_cache_page_rank_amd as lk
    f, s = full, full.spec
    B = s.batch
    say("exact page masses (oracle, every key)", s.name)
    _, exact = oracle.exact_pool(oracle.Layout(s.num_q_heads, s.num_kv_heads, s.head_dim,
                                               s.page_size, f.layer.block_table, f.layer.seq_lens),
                                 f.layer.q, f.layer.k_f32(), threads=16)
    dout = torch.empty((B, s.num_q_heads, s.head_dim), dtype=torch.bfloat16, device=DEV)
    dlse = torch.empty((B, s.num_q_heads), device=DEV)
    dws = lk.workspace(lk.workspace_bytes(lk.OP_DENSE_ATTEND, B, s.max_pages, s.num_q_heads,
                                          s.num_kv_heads, s.page_size, s.head_dim, s.rank, 0))
    lk.locks_dense_attend(f.q, f.kv, f.pages, dout, dlse, ws=dws)
    for budget in (s.budgets or [s.budget_tokens]):
        k = budget // s.page_size
        sel = torch.empty((B, s.num_kv_heads, k), dtype=torch.int32, device=DEV)
        mass = torch.empty((B, s.num_kv_heads, k), device=DEV)
        ws = lk.workspace(lk.workspace_bytes(lk.OP_STEP, B, s.max_pages, s.num_q_heads,
                                             s.num_kv_heads, s.page_size, s.head_dim, s.rank, k))
        say("agreement", s.name, budget)
        lk.locks_select(f.q, f.summ, f.pages, budget, sel, mass, ws=ws)
        out = torch.empty_like(dout)
        lse = torch.empty_like(dlse)
        sel_b = lk.workspace_bytes(lk.OP_SELECT, B, s.max_pages, s.num_q_heads, s.num_kv_heads,
                                   s.page_size, s.head_dim, s.rank, k)
        lk.locks_sparse_attend(f.q, f.kv, f.pages, sel, out, lse, ws=ws[sel_b:])
        torch.cuda.synchronize()
        sel_np = sel.cpu().numpy()
        recall, captured, carriers = [], [], 0
        for b in range(B):
            nfull = s.seq_lens[b] // s.page_size
            kk = min(k, nfull)
            for g in range(s.num_kv_heads):
                a = exact[b, g, :nfull]
                best = _brute_topk(a.astype(np.float32), kk)
                got = sel_np[b, g][sel_np[b, g] >= 0]
                recall.append(len(set(best.tolist()) & set(got.tolist())) / max(kk, 1))
                captured.append(math.exp(_lse(a[got]) - _lse(a[best])))
                carriers += len(set(f.layer.carrier_page[b, g].tolist()) & set(got.tolist()))
        diff = float((out.float() - dout.float()).abs().max())
        print(f"[agreement] {s.name} r={s.rank} budget {budget}: recall@k "
              f"{np.mean(recall):.3f} (min {np.min(recall):.3f}), captured exact mass "
              f"{np.mean(captured):.3f} (min {np.min(captured):.3f}), carriers "
              f"{carriers}/{f.layer.carrier_page.size}, max|o_sparse - o_dense| {diff:.4f}",
              flush=True)
        assert all(0.0 <= r <= 1.0 for r in recall)
        assert all(0.0 < c <= 1.0 + 1e-6 for c in captured)
        assert math.isfinite(diff)
