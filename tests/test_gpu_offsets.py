"""GPU parity of the summary scan on pools whose summary arrays span more than
4 GiB, where the library addresses them with 64-bit offsets, against the
oracle on the same seeded layer, through the C ABI.

The layer's summaries are planted at physical blocks spread over a large
pool (every other block near its end, beyond the 4 GiB byte offset of the
basis and coefficient arrays, the rest near its start) and the block table is
remapped to match; the oracle scans the layer in its own compact layout.  The
pool's other blocks hold zeros and are never referenced."""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import DEV, Case, bf16_small, masses_close, say, to_np
from workload.device import codes_to_device, summaries_to_device

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32


def _spread(ids, nb_big):
    """Physical block o of the compact layer -> its block in the large pool."""
    ids = np.asarray(ids, np.int64)
    return np.where(ids % 2 == 0, nb_big - 1 - ids, ids)


def _plant(small, nb_big, ids_small, ids_big):
    """A zeroed tensor of nb_big blocks with small's blocks copied in."""
    big = torch.zeros((nb_big,) + tuple(small.shape[1:]), dtype=small.dtype, device=DEV)
    big[torch.from_numpy(ids_big).to(DEV)] = small[torch.from_numpy(ids_small).to(DEV)]
    return big


def _remapped_pages(case, nb_big):
    import kv_cache_page_rank_amd as lk
    bt = case.layer.block_table
    new = np.where(bt >= 0, _spread(np.maximum(bt, 0), nb_big), bt).astype(np.int32)
    return lk.PageTable(torch.from_numpy(np.ascontiguousarray(new)).to(DEV),
                        torch.from_numpy(case.layer.seq_lens).to(DEV))


# (summary type, bytes per (block, KV head) of the basis and of the
# coefficients at r 8, d 128, P 64)
KINDS = [("f32", 8 * 128 * 4, 64 * 8 * 4), ("bf16", 8 * 128 * 2, 64 * 8 * 2),
         ("q8q4", 8 * 64, 64 * 8)]


@pytest.mark.parametrize("kind,basis_b,coef_b", KINDS, ids=[k[0] for k in KINDS])
def test_scan_pool_beyond_4gib(kind, basis_b, coef_b):
    """Per-head and group log-masses within 1e-4 of the oracle, -inf where a
    page is not full, on a pool whose basis and coefficient arrays both reach
    past 4 GiB (runs with and without missing pages: 41 and 23 pages)."""
    import kv_cache_page_rank_amd as lk
    case = Case(bf16_small())
    s = case.spec
    H = s.num_kv_heads
    # smallest block count whose high blocks sit beyond 4 GiB in both arrays
    nb_big = max(-(-GIB4 // (H * basis_b)), -(-GIB4 // (H * coef_b))) + 256
    ids_small = np.arange(s.num_blocks, dtype=np.int64)
    ids_big = _spread(ids_small, nb_big)
    high = ids_big[ids_big >= nb_big - 64]
    assert high.size > 0 and (high * H * basis_b).min() >= GIB4
    assert (high * H * coef_b).min() >= GIB4

    mu, basis, coef = case.oracle_summaries()
    if kind == "q8q4":
        codes = oracle.quantize_pool(mu, basis, coef)
        head_o, page_o = oracle.scan_pool(case.lay, s.rank, case.layer.q,
                                          *oracle.dequantize_pool(*codes))
        small = codes_to_device(*codes)
        parts = (small.mu, small.basis, small.coef, small.scales)
    else:
        dt = torch.bfloat16 if kind == "bf16" else torch.float32
        small = summaries_to_device(mu, basis, coef, dtype=dt)
        wide = [x.float().cpu().numpy() for x in (small.mu, small.basis, small.coef)]
        head_o, page_o = oracle.scan_pool(case.lay, s.rank, case.layer.q, *wide)
        parts = (small.mu, small.basis, small.coef)
    big = lk.Summaries(*(_plant(t, nb_big, ids_small, ids_big) for t in parts))
    assert big.basis.numel() * big.basis.element_size() > GIB4
    assert big.coef.numel() * big.coef.element_size() > GIB4
    pages = _remapped_pages(case, nb_big)

    pm = torch.full((s.batch, H, s.max_pages), 7.0, device=DEV)
    hm = torch.full((s.batch, s.num_q_heads, s.max_pages), 7.0, device=DEV)
    say("scan beyond 4 GiB", kind, nb_big, "blocks")
    lk.locks_scan(case.q, big, pages, pm, hm)
    pm2 = torch.full_like(pm, 7.0)
    lk.locks_scan(case.q, big, pages, pm2)
    torch.cuda.synchronize()
    try:
        assert masses_close(to_np(pm), page_o) <= 1e-4
        assert masses_close(to_np(pm2), page_o) <= 1e-4
        assert masses_close(to_np(hm), head_o) <= 1e-4
    finally:
        del big, pm, hm, pm2
        torch.cuda.empty_cache()
