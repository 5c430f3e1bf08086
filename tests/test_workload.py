"""The seeded input generator: determinism, structure and the stated recipe."""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_deterministic_and_thread_independent(wl):
    spec = wl.config(0).with_(seq_lens=[1000, 517], batch=2, num_q_heads=4, num_kv_heads=2,
                              carriers=2)
    a = wl.make(spec, threads=1)
    b = wl.make(spec, threads=5)
    for name in ("q", "k", "v", "block_table", "carrier_page", "carrier_slot"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name), err_msg=name)
    c = wl.make(spec.with_(seed=spec.seed + 1))
    assert not np.array_equal(a.q, c.q)


def test_block_table_is_a_permutation(wl):
    spec = wl.config(0).with_(seq_lens=[1000, 517, 16], batch=3, carriers=1)
    L = wl.make(spec)
    pages = spec.pages_per_seq
    used = np.concatenate([L.block_table[b, :pages[b]] for b in range(3)])
    assert sorted(used.tolist()) == list(range(spec.num_blocks))
    for b in range(3):
        assert np.all(L.block_table[b, pages[b]:] == -1)
    assert not np.array_equal(used, np.arange(spec.num_blocks))  # shuffled


def test_partial_page_is_poisoned(wl):
    spec = wl.config(0).with_(seq_lens=[1000])
    L = wl.make(spec)
    last = L.block_table[0, 62]
    assert np.all(np.isnan(L.k[last, 0, 1000 - 62 * 16:]))
    assert np.all(np.isfinite(L.k[last, 0, :1000 - 62 * 16]))
    assert np.all(np.isfinite(L.v[last, 0, :1000 - 62 * 16]))


def test_pages_are_locally_low_rank(wl):
    """Keys of a page = m-dim subspace signal (std 2^-t) + noise 0.05: the
    centred block has m large singular values then a noise floor."""
    spec = wl.config(0).with_(carriers=0, head_dim=128, subspace_rank=4, page_size=64,
                              seq_lens=[64 * 8])
    L = wl.make(spec)
    K = L.k_f32()[L.block_table[0, 3], 0].astype(np.float64)
    s = np.linalg.svd(K - K.mean(0), compute_uv=False)
    noise_top = 0.05 * (math.sqrt(64) + math.sqrt(128))
    assert s[0] > 4 and s[1] > 2  # sqrt(64) * 2^-t for t = 0, 1
    assert s[4] < 1.15 * noise_top
    # different pages have different subspaces (globally high-rank)
    K2 = L.k_f32()[L.block_table[0, 4], 0].astype(np.float64)
    u1 = np.linalg.svd(K - K.mean(0))[2][:2]
    u2 = np.linalg.svd(K2 - K2.mean(0))[2][:2]
    assert np.linalg.norm(u1 @ u2.T) < 0.8


def test_carriers_aligned_with_group_query(wl):
    spec = wl.config(0).with_(num_q_heads=4, num_kv_heads=2, carriers=3)
    L = wl.make(spec)
    K = L.k_f32()
    for g in range(2):
        qhat = L.q[0, 2 * g:2 * g + 2].astype(np.float64).sum(0)
        qhat /= np.linalg.norm(qhat)
        for page, slot in zip(L.carrier_page[0, g], L.carrier_slot[0, g]):
            k = K[L.block_table[0, page], g, slot].astype(np.float64)
            assert k @ qhat / np.linalg.norm(k) == pytest.approx(0.9, abs=1e-6)
    assert np.all(np.diff(L.carrier_page[0, 0]) > 0)


def test_bf16_rounding_is_nearest_even(wl):
    lib = wl.lib()
    x = np.float32(1.0) + np.float32(2.0 ** -8)  # halfway between two bf16 values
    assert lib.wl_f32_to_bf16(float(x)) == 0x3f80  # ties to even
    y = np.float32(1.0) + np.float32(3 * 2.0 ** -8)
    assert lib.wl_f32_to_bf16(float(y)) == 0x3f82
    spec = wl.config(1).with_(seq_lens=[64 * 4], carriers=1, num_q_heads=4, num_kv_heads=1)
    L = wl.make(spec)
    assert L.k.dtype == np.uint16
    assert np.all(np.isfinite(L.k_f32()))


def test_normal_statistics(wl):
    lib = wl.lib()
    z = np.array([lib.wl_normal(lib.wl_hash(7, 1, 0, 0, 0, i)) for i in range(20000)])
    assert abs(z.mean()) < 0.03 and abs(z.std() - 1) < 0.03


def test_config_shapes(wl):
    s2 = wl.config(2)
    assert (s2.num_q_heads, s2.num_kv_heads, s2.head_dim, s2.page_size) == (32, 2, 128, 64)
    assert s2.seq_lens == [1 << 20] and s2.max_pages == 16384 and s2.k_pages == 32
    s4 = wl.config(4)
    assert s4.batch == 16 and all(32768 <= n <= 262144 for n in s4.seq_lens)
    assert any(n % 64 for n in s4.seq_lens)  # partial last pages exist
    assert wl.config(3).rank == 2 and wl.config(3).budgets == [512, 1024, 2048, 4096]


def test_oracle_regression_fixture(wl, orc):
    """Oracle outputs on the tiny workload equal the stored fixture written by
    tests/golden/make_golden.py (a change to the oracle's arithmetic must
    regenerate it deliberately)."""
    with open(os.path.join(GOLDEN, "tiny_oracle_outputs.json")) as f:
        g = json.load(f)
    spec = wl.config(0)
    L = wl.make(spec)
    lay = orc.Layout(1, 1, 64, 16, L.block_table, L.seq_lens)
    mu, basis, coef = orc.build_pool(lay, spec.rank, L.k_f32(), spec.num_blocks)
    _, page = orc.scan_pool(lay, spec.rank, L.q, mu, basis, coef)
    np.testing.assert_allclose(page[0, 0], g["page_mass"], atol=1e-12)
    sel, _ = orc.select_pool(lay, spec.budget_tokens, page.astype(np.float32), spec.k_pages)
    assert sel[0, 0].tolist() == g["selected"]
    assert set(g["carriers"]) <= set(g["selected"])
    out, lse = orc.attend_pool(lay, L.q, L.k_f32(), L.v_f32(), sel)
    np.testing.assert_allclose(out[0, 0], g["sparse_out"], atol=1e-12)
