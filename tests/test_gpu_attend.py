"""GPU parity of sparse (selected pages + partial last page) and dense paged
flash-decode against the oracle, on the same page lists."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import DEV, Case, bf16_small, out_tol, say, tiny, to_np

pytestmark = pytest.mark.gpu


def _lk():
    import kv_cache_page_rank_amd as lk
    return lk


def _run_sparse(case, sel_np):
    lk = _lk()
    s = case.spec
    k = sel_np.shape[-1]
    sel = torch.from_numpy(np.ascontiguousarray(sel_np, np.int32)).to(DEV)
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=case.kv.k.dtype, device=DEV)
    lse = torch.empty((s.batch, s.num_q_heads), device=DEV)
    ws = lk.workspace(lk.workspace_bytes(lk.OP_SPARSE_ATTEND, s.batch, s.max_pages, s.num_q_heads,
                                         s.num_kv_heads, s.page_size, s.head_dim, s.rank, k))
    lk.locks_sparse_attend(case.q, case.kv, case.pages, sel, out, lse, ws=ws)
    torch.cuda.synchronize()
    return to_np(out), lse.cpu().numpy()


def _run_dense(case):
    lk = _lk()
    s = case.spec
    out = torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=case.kv.k.dtype, device=DEV)
    lse = torch.empty((s.batch, s.num_q_heads), device=DEV)
    ws = lk.workspace(lk.workspace_bytes(lk.OP_DENSE_ATTEND, s.batch, s.max_pages, s.num_q_heads,
                                         s.num_kv_heads, s.page_size, s.head_dim, s.rank, 0))
    lk.locks_dense_attend(case.q, case.kv, case.pages, out, lse, ws=ws)
    torch.cuda.synchronize()
    return to_np(out), lse.cpu().numpy()


def _check(out_g, lse_g, out_o, lse_o, bf16):
    err = np.abs(out_g - out_o)
    assert np.all(err <= out_tol(out_o, bf16)), float(err.max())
    fin = np.isfinite(lse_o)
    assert np.array_equal(fin, np.isfinite(lse_g))
    assert np.all(np.abs(lse_g[fin] - lse_o[fin]) <= (1e-4 if bf16 else 1e-5))


def _random_sel(case, k, seed):
    rng = np.random.default_rng(seed)
    s = case.spec
    sel = np.full((s.batch, s.num_kv_heads, k), -1, np.int32)
    for b in range(s.batch):
        f = s.seq_lens[b] // s.page_size
        for g in range(s.num_kv_heads):
            n = min(k, f)
            sel[b, g, :n] = np.sort(rng.choice(f, n, replace=False))
    return sel


CASES = [
    ("tiny-f32", lambda: tiny(), False),
    ("tiny-f32-G4-ragged", lambda: tiny(num_q_heads=4, num_kv_heads=1, seq_lens=[1000]), False),
    # fp32 caches at the other (page size, head dim) instantiations
    ("tiny-f32-d128", lambda: tiny(head_dim=128, rank=8, seq_lens=[16 * 70 + 9]), False),
    ("f32-P64-G16", lambda: bf16_small(kv_bf16=False), False),
    ("f32-P64-G4-d64", lambda: bf16_small(kv_bf16=False, head_dim=64, num_kv_heads=8), False),
    ("bf16-G16", lambda: bf16_small(), True),
    ("bf16-G4", lambda: bf16_small(num_kv_heads=8), True),
    ("bf16-G1", lambda: bf16_small(num_q_heads=2), True),
    ("bf16-G16-d64", lambda: bf16_small(head_dim=64), True),
    # many (sequence, KV head, page) items: the wave-per-run kernel (2 and 4 pages per wave)
    ("bf16-batch16-G4-runs2", lambda: bf16_small(batch=16, num_kv_heads=8,
                                                 seq_lens=[64 * 40 + (7 * i) % 64 for i in range(16)]),
     True),
    ("bf16-batch16-G4-k64-d64", lambda: bf16_small(batch=16, num_kv_heads=8, head_dim=64,
                                                   budget_tokens=4096,
                                                   seq_lens=[64 * (36 + i) + 5 * i for i in range(16)]),
     True),
    # 32 (sequence, KV head) groups of 65 slots: the wave-per-run kernel with
    # 4-page runs and partial pages at the end of every run
    ("bf16-batch4-G4-k64-runs", lambda: bf16_small(batch=4, num_kv_heads=8, budget_tokens=4096,
                                                   seq_lens=[64 * (70 + 3 * i) + 9 * i
                                                             for i in range(4)]),
     True),
]


@pytest.mark.parametrize("name,mk,bf16", CASES, ids=[c[0] for c in CASES])
def test_sparse_attend_matches_oracle(name, mk, bf16):
    case = Case(mk())
    sel = _random_sel(case, case.spec.k_pages, 5)
    out_o, lse_o = oracle.attend_pool(case.lay, case.layer.q, case.k_f32, case.layer.v_f32(), sel)
    say("sparse attend", name)
    out_g, lse_g = _run_sparse(case, sel)
    _check(out_g, lse_g, out_o, lse_o, bf16)


@pytest.mark.parametrize("name,mk,bf16", CASES, ids=[c[0] for c in CASES])
def test_dense_attend_matches_oracle(name, mk, bf16):
    case = Case(mk())
    out_o, lse_o = oracle.attend_pool(case.lay, case.layer.q, case.k_f32, case.layer.v_f32(), None)
    say("dense attend", name)
    out_g, lse_g = _run_dense(case)
    _check(out_g, lse_g, out_o, lse_o, bf16)


@pytest.mark.parametrize("mk,bf16", [(lambda: tiny(seq_lens=[1000]), False),
                                     (lambda: bf16_small(), True)])
def test_select_all_equals_dense(mk, bf16):
    """Every full page selected (+ the partial page) reproduces dense attention."""
    case = Case(mk())
    s = case.spec
    width = s.max_pages
    sel = np.full((s.batch, s.num_kv_heads, width), -1, np.int32)
    for b in range(s.batch):
        f = s.seq_lens[b] // s.page_size
        sel[b, :, :f] = np.arange(f)
    say("select-all vs dense")
    out_s, lse_s = _run_sparse(case, sel)
    out_d, lse_d = _run_dense(case)
    tol = 2e-2 if bf16 else 1e-5
    assert np.abs(out_s - out_d).max() <= tol
    assert np.abs(lse_s - lse_d).max() <= 1e-4


def test_empty_selection_and_partial_page():
    """k = 0: only the partial last page is attended; a page-aligned sequence
    with nothing selected gives zero output and lse -inf.  Invalid slots
    (-1, pages past the full ones) are ignored."""
    case = Case(bf16_small())
    s = case.spec
    sel = np.full((s.batch, s.num_kv_heads, 3), -1, np.int32)
    sel[0, 0, 1] = 10_000  # not a page of the sequence: ignored
    sel[1, 1, 2] = 23      # first non-full index of sequence 1 (page-aligned): ignored
    out_o, lse_o = oracle.attend_pool(case.lay, case.layer.q, case.k_f32, case.layer.v_f32(), sel)
    say("empty selection")
    out_g, lse_g = _run_sparse(case, sel)
    assert np.all(np.isneginf(lse_g[1])) and not out_g[1].any()
    _check(out_g, lse_g, out_o, lse_o, True)


def test_attend_deterministic():
    case = Case(bf16_small())
    sel = _random_sel(case, 8, 1)
    say("attend determinism")
    a = _run_sparse(case, sel)
    b = _run_sparse(case, sel)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = _run_dense(case)
    d = _run_dense(case)
    assert np.array_equal(c[0], d[0]) and np.array_equal(c[1], d[1])


@pytest.mark.parametrize("mk,bf16", [(lambda: tiny(num_q_heads=4, num_kv_heads=1, seq_lens=[1000]),
                                      False),
                                     (lambda: bf16_small(seq_lens=[64 * 20 + 17, 64 * 9 + 63]),
                                      True)])
def test_zero_pages_attends_partial_page_only(mk, bf16):
    """k_pages = 0 (a budget below one page): each sequence attends only its
    partial last page (the list passed to the kernels is then a stand-in that
    is read but never used)."""
    case = Case(mk())
    s = case.spec
    sel = np.zeros((s.batch, s.num_kv_heads, 0), np.int32)
    out_o, lse_o = oracle.attend_pool(case.lay, case.layer.q, case.k_f32, case.layer.v_f32(), sel)
    say("zero selected pages")
    out_g, lse_g = _run_sparse(case, sel)
    _check(out_g, lse_g, out_o, lse_o, bf16)


@pytest.mark.parametrize("scale", [16.0])
def test_attend_large_logits(scale):
    """Logits of tens (queries scaled up, keys offset per page): outputs within
    the bf16 bar and lse within 1e-4 of the oracle, on the sparse (one
    workgroup per page and wave-per-run) and dense kernels."""
    lk = _lk()
    for mk in (lambda: bf16_small(page_offset_std=4.0),
               lambda: bf16_small(batch=16, num_kv_heads=8, page_offset_std=4.0,
                                  seq_lens=[64 * 40 + (7 * i) % 64 for i in range(16)])):
        case = Case(mk())
        s = case.spec
        q_host = (case.layer.q.astype(np.float64) * scale).astype(np.float32)
        case.q = torch.from_numpy(q_host).to(DEV)
        sel = _random_sel(case, case.spec.k_pages, 9)
        out_o, lse_o = oracle.attend_pool(case.lay, q_host, case.k_f32, case.layer.v_f32(), sel)
        assert float(np.abs(lse_o).max()) > 8.0  # the regime this case is for
        say("attend large logits", scale, s)
        out_g, lse_g = _run_sparse(case, sel)
        say("sparse max |lse error|", float(np.abs(lse_g - lse_o).max()))
        _check(out_g, lse_g, out_o, lse_o, True)
        outd_o, lsed_o = oracle.attend_pool(case.lay, q_host, case.k_f32, case.layer.v_f32(), None)
        outd_g, lsed_g = _run_dense(case)
        say("dense max |lse error|", float(np.abs(lsed_g - lsed_o).max()))
        _check(outd_g, lsed_g, outd_o, lsed_o, True)
