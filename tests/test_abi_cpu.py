"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments on the host
before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "locks.h")


@pytest.fixture(scope="module")
def lk():
    import kv_cache_page_rank_amd as lk
    if not os.path.exists(lk.LIB_PATH):
        from kv_cache_page_rank_amd import build
        build.build()
    lk.lib()
    return lk


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(locks_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported(lk):
    names = _declared()
    assert "locks_select" in names and "locks_build_summaries" in names
    lib = lk.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert isinstance(getattr(lib, n), ctypes._CFuncPtr)
    assert set(lk.EXPORTED) == set(names)


def test_version_and_status_strings(lk):
    lib = lk.lib()
    assert lib.locks_version() == 106
    assert lib.locks_status_string(0) == b"ok"
    assert b"workspace" in lib.locks_status_string(3)
    assert lib.locks_status_string(99) == b"unknown status"


def test_workspace_sizes(lk):
    ws = lk.workspace_bytes
    # select: page masses [B][Hkv][max_pages] fp32, run maxima
    # [B][Hkv][ceil(max_pages / 16)], per-head estimates [B][Hq][max_pages] and
    # per-head totals [B][Hq], each 256-byte aligned
    assert ws(lk.OP_SELECT, 1, 16384, 32, 2, 64, 128, 8, 32) == \
        2 * 16384 * 4 + 2 * 1024 * 4 + 32 * 16384 * 4 + 256
    assert ws(lk.OP_SELECT, 1, 100, 32, 2, 64, 128, 8, 32) == 1024 + 256 + 12800 + 256
    # sparse attend: (k + 1) splits of (2 + d) floats per query head
    assert ws(lk.OP_SPARSE_ATTEND, 1, 16384, 32, 2, 64, 128, 8, 32) == \
        256 * ((32 * 33 * 2 * 4 + 255) // 256) + 32 * 33 * 128 * 4
    assert ws(lk.OP_STEP, 1, 16384, 32, 2, 64, 128, 8, 32) == \
        ws(lk.OP_SELECT, 1, 16384, 32, 2, 64, 128, 8, 32) + \
        ws(lk.OP_SPARSE_ATTEND, 1, 16384, 32, 2, 64, 128, 8, 32)
    assert ws(lk.OP_BUILD, 1, 16384, 32, 2, 64, 128, 8, 32) == 0
    assert ws(lk.OP_DENSE_ATTEND, 1, 16384, 32, 2, 64, 128, 8, 32) > 0
    assert ws(lk.OP_SELECT, 0, 16384, 32, 2, 64, 128, 8, 32) == 0


def _fake(lk, P=64, d=128, r=8, H=2, NB=4, B=1, MP=4, dtype=1, sdtype=0, scales=True):
    # non-null "device" addresses: validation never dereferences them
    addr = 0x1000
    kv = lk.CKVCache(dtype, NB, H, P, d, addr, addr)
    sm = lk.CSummaries(sdtype, NB, H, P, d, r, addr, addr, addr, addr if scales else None)
    pt = lk.CPageTable(B, MP, addr, addr)
    return kv, sm, pt, ctypes.c_void_p(addr)


def test_host_validation_rejects_without_launch(lk):
    lib = lk.lib()
    by = ctypes.byref
    kv, sm, pt, p = _fake(lk)
    # null query
    assert lib.locks_select(None, 32, by(sm), by(pt), 2048, 0, p, p, p, p, 1 << 20, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    # H_q not a multiple of H_kv
    assert lib.locks_scan(p, 31, by(sm), by(pt), p, None, None, None) == lk.LOCKS_ERR_INVALID_ARG
    # group wider than 16
    assert lib.locks_scan(p, 64, by(sm), by(pt), p, None, None, None) == lk.LOCKS_ERR_INVALID_ARG
    # rank above min(P, d, 16)
    _, sm_bad, _, _ = _fake(lk, r=17)
    assert lib.locks_scan(p, 32, by(sm_bad), by(pt), p, None, None, None) == lk.LOCKS_ERR_UNSUPPORTED
    # unsupported page size / head dim
    _, sm_p, _, _ = _fake(lk, P=32)
    assert lib.locks_scan(p, 32, by(sm_p), by(pt), p, None, None, None) == lk.LOCKS_ERR_UNSUPPORTED
    kv_p, _, _, _ = _fake(lk, P=16, dtype=1)
    assert lib.locks_dense_attend(p, 32, by(kv_p), by(pt), p, None, p, 1 << 30, None) == \
        lk.LOCKS_ERR_UNSUPPORTED
    # workspace missing / too small
    assert lib.locks_select(p, 32, by(sm), by(pt), 2048, 0, p, p, None, None, 0, None) == \
        lk.LOCKS_ERR_WORKSPACE
    assert lib.locks_sparse_attend(p, 32, by(kv), by(pt), p, 32, p, None, p, 16, None) == \
        lk.LOCKS_ERR_WORKSPACE
    # too many pages for the selection kernel
    _, _, pt_big, _ = _fake(lk, MP=40000)
    assert lib.locks_scan(p, 32, by(sm), by(pt_big), p, None, None, None) == lk.LOCKS_ERR_UNSUPPORTED
    # negative budget, bad dtype, mismatched build shapes
    assert lib.locks_select(p, 32, by(sm), by(pt), -1, 0, p, p, p, p, 1 << 20, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    kv_bad, _, _, _ = _fake(lk, dtype=7)
    assert lib.locks_dense_attend(p, 32, by(kv_bad), by(pt), p, None, p, 1 << 30, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    # refresh without page_begin or pages
    assert lib.locks_refresh_summaries(by(kv), by(pt), None, 1, by(sm), None) == \
        lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_refresh_summaries(by(kv), by(pt), p, 0, by(sm), None) == \
        lk.LOCKS_ERR_INVALID_ARG
    # unknown aggregation; mean-of-share without workspace
    assert lib.locks_select(p, 32, by(sm), by(pt), 2048, 7, p, p, p, p, 1 << 20, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_select(p, 32, by(sm), by(pt), 2048, 1, p, p, p, None, 0, None) == \
        lk.LOCKS_ERR_WORKSPACE
    assert lib.locks_mean_share(p, 32, 2, by(pt), 64, p, None, None, 0, None) == \
        lk.LOCKS_ERR_WORKSPACE
    assert lib.locks_mean_share(None, 32, 2, by(pt), 64, p, None, p, 1024, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    _, sm_dt, _, _ = _fake(lk, sdtype=5)  # not a summary dtype
    assert lib.locks_scan(p, 32, by(sm_dt), by(pt), p, None, None, None) == lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_build_summaries(by(kv), by(pt), None, by(sm_dt), None, 0, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    _, sm_d, _, _ = _fake(lk, d=64)
    assert lib.locks_build_summaries(by(kv), by(pt), None, by(sm_d), None, 0, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    # integer-code summaries need their scales; quantise wants fp32 -> Q8Q4 of one shape
    _, sm_q, _, _ = _fake(lk, sdtype=lk.LOCKS_Q8Q4)
    _, sm_qn, _, _ = _fake(lk, sdtype=lk.LOCKS_Q8Q4, scales=False)
    assert lib.locks_scan(p, 32, by(sm_qn), by(pt), p, None, None, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_build_summaries(by(kv), by(pt), None, by(sm_qn), None, 0, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_quantize_summaries(by(sm_q), by(sm_q), None) == lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_quantize_summaries(by(sm), by(sm), None) == lk.LOCKS_ERR_INVALID_ARG
    _, sm_q4, _, _ = _fake(lk, sdtype=lk.LOCKS_Q8Q4, r=4)
    assert lib.locks_quantize_summaries(by(sm), by(sm_q4), None) == lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_quantize_summaries(None, by(sm_q), None) == lk.LOCKS_ERR_INVALID_ARG
    # sketch: needs the shared basis and fp32 output
    assert lib.locks_build_sketch_summaries(by(kv), by(pt), None, None, by(sm), None) == \
        lk.LOCKS_ERR_INVALID_ARG
    _, sm_bf, _, _ = _fake(lk, sdtype=lk.LOCKS_BF16)
    assert lib.locks_build_sketch_summaries(by(kv), by(pt), None, p, by(sm_bf), None) == \
        lk.LOCKS_ERR_INVALID_ARG
    # sparse attend with pages requested but no list
    assert lib.locks_sparse_attend(p, 32, by(kv), by(pt), None, 4, p, None, p, 1 << 30, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    # measurement probes: sizes and shapes checked on the host
    assert lib.locks_probe_stream_read(p, 1000, p, 64, None) == lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_probe_stream_read(p, 1024, p, 6, None) == lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_probe_stream_read(p, 1024, p, 4 * 65537, None) == lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_probe_stream_read(None, 1024, p, 64, None) == lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_probe_summary_read(p, 32, by(sm_bf), by(pt), p, None) == \
        lk.LOCKS_ERR_UNSUPPORTED
    _, sm_r4, _, _ = _fake(lk, r=4)
    assert lib.locks_probe_summary_read(p, 32, by(sm_r4), by(pt), p, None) == \
        lk.LOCKS_ERR_UNSUPPORTED
    assert lib.locks_probe_summary_read(p, 32, by(sm), by(pt), None, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    # the allocation-free selection refuses shapes whose workspace exceeds its
    # 16 MiB scratch, and bad arguments, on the host
    _, _, pt_wide, _ = _fake(lk, B=64, MP=32768)
    assert lib.locks_select_noalloc(p, 32, by(sm), by(pt_wide), 2048, 0, p, p, None, None) == \
        lk.LOCKS_ERR_WORKSPACE
    assert lib.locks_select_noalloc(None, 32, by(sm), by(pt), 2048, 0, p, p, None, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    assert lib.locks_select_noalloc(p, 32, by(sm), by(pt), -5, 0, p, p, None, None) == \
        lk.LOCKS_ERR_INVALID_ARG
    # graph creation validates before capturing
    h = ctypes.c_void_p()
    assert lib.locks_step_graph_create(None, by(h)) == lk.LOCKS_ERR_INVALID_ARG
    args = lk.CStepArgs(0x1000, 32, 2048, 0, sm, kv, pt, 0x1000, 0x1000, None, 0x1000, None, None, 0)
    assert lib.locks_step_graph_create(by(args), by(h)) == lk.LOCKS_ERR_WORKSPACE
    assert lib.locks_step_graph_launch(None, None) == lk.LOCKS_ERR_INVALID_ARG
    lib.locks_step_graph_destroy(None)


def test_python_binding_fails_loudly_without_library(lk, tmp_path, monkeypatch):
    monkeypatch.setattr(lk, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(lk, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        lk.lib()
