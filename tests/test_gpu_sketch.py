"""Shared-basis sketch, the ablation baseline (technical summary, section 3:
a projection shared by every page is blind to page-specific directions).
Parity of the GPU sketch builder against the oracle's sketch on the same
shared basis, and - reported, not gated - the selection agreement of page
summaries and of the sketch at equal storage against the selection that reads
every key."""
import math

import numpy as np
import pytest
import torch

import oracle
import workload
from gpu_cases import DEV, Case, bf16_small, masses_close, say, tiny, to_np
from workload.device import upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mk,rho,begin", [(lambda: tiny(), 6, None),
                                          (lambda: bf16_small(), 12, None),
                                          (lambda: bf16_small(num_kv_heads=8), 16, [10, 5])],
                         ids=["tiny-rho6", "bf16-rho12", "bf16-G4-rho16-begin"])
def test_sketch_matches_oracle(mk, rho, begin):
    """Centroids and coordinates within 1e-5 (relative to the page's scale) of
    the oracle's on the same shared basis, the basis copied exactly, other
    blocks untouched; the scan of the result matches the oracle's masses."""
    import kv_cache_page_rank_amd as lk
    case = Case(mk())
    s = case.spec
    basis, _ = oracle.shared_basis(case.lay, rho, case.k_f32)
    mu_o, rep_o, coef_o = oracle.sketch_pool(case.lay, rho, case.k_f32, basis, s.num_blocks)
    summ = lk.Summaries.empty(s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim, rho)
    for t in (summ.mu, summ.basis, summ.coef):
        t.fill_(np.nan)
    pb = None if begin is None else torch.tensor(begin, dtype=torch.int32, device=DEV)
    say("sketch build", s.name, rho, begin)
    lk.locks_build_sketch_summaries(case.kv, case.pages,
                                    torch.from_numpy(basis.astype(np.float32)).to(DEV), summ,
                                    page_begin=pb)
    torch.cuda.synchronize()
    mu, rep, coef = (to_np(t) for t in (summ.mu, summ.basis, summ.coef))
    bt = case.layer.block_table
    for b in range(s.batch):
        lo = 0 if begin is None else begin[b]
        for j in range(-(-s.seq_lens[b] // s.page_size)):
            blk = bt[b, j]
            built = lo <= j < s.seq_lens[b] // s.page_size
            assert np.isfinite(mu[blk]).all() == built, (b, j)
            if not built:
                continue
            scale = np.abs(coef_o[blk]).max() + 1e-30
            np.testing.assert_allclose(mu[blk], mu_o[blk], atol=1e-5 * np.abs(mu_o[blk]).max())
            assert np.abs(coef[blk] - coef_o[blk]).max() <= 1e-5 * scale, (b, j)
            np.testing.assert_array_equal(rep[blk], rep_o[blk])
    if begin is None:
        _, page_o = oracle.scan_pool(case.lay, rho, case.layer.q, mu_o, rep_o, coef_o)
        pm = torch.empty((s.batch, s.num_kv_heads, s.max_pages), device=DEV)
        say("sketch scan", s.name, rho)
        lk.locks_scan(case.q, summ, case.pages, pm)
        torch.cuda.synchronize()
        assert masses_close(to_np(pm), page_o) <= 1e-4


def _lse(x):
    x = np.asarray(x, np.float64)
    m = x.max()
    return m + math.log(np.exp(x - m).sum())


def _topk(mass, k):
    order = np.lexsort((np.arange(mass.size), -mass.astype(np.float64)))
    return np.sort(order[:k])


@pytest.mark.parametrize("idx,gain", [(1, 1.0), (3, 1.0), (1, 3.0)],
                         ids=["llama-128k", "glm-1m", "llama-128k-carrier-gain3"])
def test_shared_basis_ablation_at_equal_storage(idx, gain):
    """Reported, not gated: page summaries of rank r against the shared-basis
    sketch of rank rho = r (1 + d / P) (the same values per page), both
    selecting with the same estimator, each compared with the selection that
    reads every key: recall of the exact top-k, the share of the exact top-k's
    mass captured, carrier pages kept."""
    import kv_cache_page_rank_amd as lk
    spec = workload.config(idx).with_(carrier_gain=gain)
    say("generate", spec.name, "carrier gain", gain)
    layer = workload.make(spec, threads=16)
    q, kv, pages = upload(layer, DEV)
    s = spec
    lay = oracle.Layout(s.num_q_heads, s.num_kv_heads, s.head_dim, s.page_size,
                        layer.block_table, layer.seq_lens)
    kf = layer.k_f32()
    say("exact page masses (oracle, every key)", s.name)
    _, exact = oracle.exact_pool(lay, layer.q, kf, threads=16)
    nfull = s.seq_lens[0] // s.page_size
    lines = []
    for r in (2, 4):
        rho = r * (1 + s.head_dim // s.page_size)
        say("shared basis", s.name, rho)
        basis, eig = oracle.shared_basis(lay, rho, kf, threads=16)
        captured_energy = float(np.mean(eig[:, :rho].sum(1) / eig.sum(1)))
        for label, rank in (("page summaries", r), ("shared basis", rho)):
            summ = lk.Summaries.empty(s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim, rank)
            say("build", label, rank)
            if label == "page summaries":
                lk.locks_build_summaries(kv, pages, summ)
            else:
                lk.locks_build_sketch_summaries(
                    kv, pages, torch.from_numpy(basis.astype(np.float32)).to(DEV), summ)
            for budget in (512, 2048):
                k = budget // s.page_size
                sel = torch.empty((1, s.num_kv_heads, k), dtype=torch.int32, device=DEV)
                mass = torch.empty((1, s.num_kv_heads, k), device=DEV)
                ws = lk.workspace(lk.workspace_bytes(lk.OP_SELECT, 1, s.max_pages, s.num_q_heads,
                                                     s.num_kv_heads, s.page_size, s.head_dim,
                                                     rank, k))
                lk.locks_select(q, summ, pages, budget, sel, mass, ws=ws)
                torch.cuda.synchronize()
                sel_np = sel.cpu().numpy()
                recall, captured, carriers = [], [], 0
                for g in range(s.num_kv_heads):
                    a = exact[0, g, :nfull]
                    best = _topk(a.astype(np.float32), k)
                    got = sel_np[0, g][sel_np[0, g] >= 0]
                    recall.append(len(set(best.tolist()) & set(got.tolist())) / k)
                    captured.append(math.exp(_lse(a[got]) - _lse(a[best])))
                    carriers += len(set(layer.carrier_page[0, g].tolist()) & set(got.tolist()))
                    assert 0.0 < captured[-1] <= 1.0 + 1e-6
                line = (f"[ablation] {s.name} gain {gain} {label} rank {rank} (values per page "
                        f"{s.head_dim + rank * s.head_dim + s.page_size * rank if label == 'page summaries' else s.head_dim + s.page_size * rank}) "
                        f"budget {budget}: recall@k {np.mean(recall):.3f}, captured exact mass "
                        f"{np.mean(captured):.3f}, carriers {carriers}/{layer.carrier_page[0].size}"
                        + (f", shared-basis energy share {captured_energy:.3f}"
                           if label == "shared basis" else ""))
                print(line, flush=True)
                lines.append(line)
            del summ
    assert lines
