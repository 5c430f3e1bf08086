"""GPU parity over seeded random shapes: page size, head dim, rank, GQA
group, batch, budget, ragged lengths and page offsets drawn at random; for
each, the scan of fp32, bf16 and integer-code summaries (per head and per
group, -inf where a page is not full) within 1e-4 of the oracle on the same
values, the selection within the band of the oracle's selection, sparse
(over the library's selection) and dense attention at the attention bars,
the builder against the oracle's build and the quantiser bit for bit
against the oracle's, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import DEV, Case, band_ok, bf16_small, masses_close, say, tiny, to_np
from test_gpu_attend import _check as check_attention, _run_dense, _run_sparse
from test_gpu_build import _build_gpu, _check_units
from workload.device import codes_to_device, summaries_to_device

pytestmark = pytest.mark.gpu


def _shape(i):
    rng = np.random.default_rng(9000 + i)
    seed = int(rng.integers(1, 10**6))
    if i % 3 == 2:  # 16-token pages, d 64
        lens = [int(rng.integers(1, 16 * 90))]
        return tiny(seed=seed, num_q_heads=int(rng.choice([1, 2, 4])),
                    rank=int(rng.choice([2, 4, 8])), seq_lens=lens, carriers=min(3, lens[0] // 16))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    lens = [int(rng.integers(1, 64 * 60)) for _ in range(int(rng.integers(1, 4)))]
    return bf16_small(seed=seed, num_kv_heads=hkv, num_q_heads=hkv * g,
                      rank=int(rng.choice([2, 5, 8, 16])), head_dim=int(rng.choice([64, 128])),
                      budget_tokens=int(rng.choice([512, 2048, 4096])), batch=len(lens), seq_lens=lens, carriers=min(4, min(n // 64 for n in lens)),
                      page_offset_std=float(rng.choice([0.0, 1.0, 4.0])))


def _summaries(sdt, mu, basis, coef):
    import kv_cache_page_rank_amd as lk
    if sdt == "q8q4":
        codes = oracle.quantize_pool(mu, basis, coef)
        return codes_to_device(*codes), oracle.dequantize_pool(*codes)
    if sdt == "bf16":
        t = [torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
             for x in (mu, basis, coef)]
        return lk.Summaries(*(x.to(DEV) for x in t)), [x.float().numpy() for x in t]
    return summaries_to_device(mu, basis, coef), (mu, basis, coef)


@pytest.mark.parametrize("i", range(9))
def test_random_shape_scan_and_select(i):
    import kv_cache_page_rank_amd as lk
    case = Case(_shape(i))
    s = case.spec
    mu, basis, coef = case.oracle_summaries()
    k = s.k_pages
    args = (s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads, s.page_size, s.head_dim, s.rank, k)
    for sdt in ("f32", "bf16", "q8q4"):
        summ, vals = _summaries(sdt, mu, basis, coef)
        head_o, page_o = oracle.scan_pool(case.lay, s.rank, case.layer.q, *vals)
        pm = torch.full((s.batch, s.num_kv_heads, s.max_pages), 7.0, device=DEV)
        hm = torch.full((s.batch, s.num_q_heads, s.max_pages), 7.0, device=DEV)
        say("random shape", i, sdt, s)
        lk.locks_scan(case.q, summ, case.pages, pm, hm)
        sel = torch.full((s.batch, s.num_kv_heads, k), -9, dtype=torch.int32, device=DEV)
        mass = torch.zeros((s.batch, s.num_kv_heads, k), device=DEV)
        lk.locks_select(case.q, summ, case.pages, s.budget_tokens, sel, mass,
                        ws=lk.workspace(lk.workspace_bytes(lk.OP_STEP, *args)))
        torch.cuda.synchronize()
        assert masses_close(to_np(pm), page_o) <= 1e-4, sdt
        assert masses_close(to_np(hm), head_o) <= 1e-4, sdt
        sel_o, _ = oracle.select_pool(case.lay, s.budget_tokens, page_o.astype(np.float32), k)
        sg = sel.cpu().numpy()
        for b in range(s.batch):
            f = s.seq_lens[b] // s.page_size
            kb = min(k, f)
            for g in range(s.num_kv_heads):
                assert np.all(sg[b, g, kb:] == -1), (sdt, b, g)
                if kb:
                    assert band_ok(sg[b, g], sel_o[b, g], page_o[b, g, :f], kb), (sdt, b, g)


@pytest.mark.parametrize("i", range(9))
def test_random_shape_attention(i):
    """Sparse attention over the library's own selection (fp32 summaries) and
    dense attention, against the oracle's attention over the same pages."""
    import kv_cache_page_rank_amd as lk
    case = Case(_shape(i))
    s = case.spec
    k = s.k_pages
    summ = summaries_to_device(*case.oracle_summaries())
    args = (s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads, s.page_size, s.head_dim, s.rank, k)
    sel = torch.full((s.batch, s.num_kv_heads, k), -9, dtype=torch.int32, device=DEV)
    mass = torch.zeros((s.batch, s.num_kv_heads, k), device=DEV)
    say("random shape attention", i, s)
    lk.locks_select(case.q, summ, case.pages, s.budget_tokens, sel, mass,
                    ws=lk.workspace(lk.workspace_bytes(lk.OP_STEP, *args)))
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    v = case.layer.v_f32()
    out_o, lse_o = oracle.attend_pool(case.lay, case.layer.q, case.k_f32, v, sel_np)
    out_g, lse_g = _run_sparse(case, sel_np)
    check_attention(out_g, lse_g, out_o, lse_o, s.kv_bf16)
    out_o, lse_o = oracle.attend_pool(case.lay, case.layer.q, case.k_f32, v, None)
    out_g, lse_g = _run_dense(case)
    check_attention(out_g, lse_g, out_o, lse_o, s.kv_bf16)


@pytest.mark.parametrize("i", range(9))
def test_random_shape_build(i):
    """The builder on every full page against the oracle's build: centroid,
    orthonormal basis, coordinate residual, captured energy, and the
    reconstructed logits on every page whose spectral gap passes the gate
    (random ranks may leave none above it here)."""
    case = Case(_shape(i))
    s = case.spec
    say("random shape build", i, s)
    summ = _build_gpu(case)
    units = np.array([[b, g, j] for b in range(s.batch) for g in range(s.num_kv_heads)
                      for j in range(s.seq_lens[b] // s.page_size)], np.int32)
    if len(units):
        _check_units(case, summ, units, s.rank)


@pytest.mark.parametrize("i", range(9))
def test_random_shape_quantise(i):
    """The oracle's fp32 summaries quantised on the device and by the oracle:
    identical codes and scales."""
    import kv_cache_page_rank_amd as lk
    case = Case(_shape(i))
    s = case.spec
    mu, basis, coef = case.oracle_summaries()
    ref = oracle.quantize_pool(mu, basis, coef)
    src = summaries_to_device(mu, basis, coef)
    dst = lk.Summaries.empty(s.num_blocks, s.num_kv_heads, s.page_size, s.head_dim, s.rank,
                             dtype=lk.Q8Q4)
    say("random shape quantise", i, s)
    lk.locks_quantize_summaries(src, dst)
    torch.cuda.synchronize()
    for got, want, what in zip((dst.mu, dst.basis, dst.coef, dst.scales), ref,
                               ("mu", "basis", "coef", "scales")):
        np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=what)
