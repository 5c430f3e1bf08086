"""Python binding of liblocks.so, the gfx950 library for the decode-step hot
path of page-local key summaries (see include/locks.h for the C ABI).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblocks.so")

LOCKS_OK, LOCKS_ERR_INVALID_ARG, LOCKS_ERR_UNSUPPORTED, LOCKS_ERR_WORKSPACE, LOCKS_ERR_HIP = \
    range(5)
LOCKS_F32, LOCKS_BF16, LOCKS_Q8Q4 = 0, 1, 2
# Summary storage with integer codes (LOCKS_Q8Q4): int8 centroid and
# coefficients, int4 basis, fp32 scales.  Pass as Summaries.empty(dtype=...).
Q8Q4 = "q8q4"
OP_BUILD, OP_SELECT, OP_SPARSE_ATTEND, OP_DENSE_ATTEND, OP_STEP = range(5)
RUN_PAGES = 16  # pages per run maximum (LOCKS_RUN_PAGES)
AGG_LSE, AGG_MEAN_SHARE = 0, 1  # locks_agg

EXPORTED = ("locks_workspace_bytes", "locks_build_summaries", "locks_select", "locks_scan",
            "locks_topk", "locks_mean_share", "locks_refresh_summaries",
            "locks_quantize_summaries", "locks_build_sketch_summaries", "locks_sparse_attend",
            "locks_dense_attend",
            "locks_step_graph_create",
            "locks_step_graph_launch", "locks_step_graph_destroy", "locks_status_string",
            "locks_last_hip_error", "locks_version", "locks_probe_stream_read",
            "locks_probe_summary_read", "locks_select_noalloc")


class LocksError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.locks_status_string(status).decode() if _lib else str(status)
        extra = f" (hipError {_lib.locks_last_hip_error()})" if _lib and status == LOCKS_ERR_HIP \
            else ""
        super().__init__(f"{where}: {msg}{extra}")
        self.status = status


class CKVCache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p)]


class CSummaries(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("mu", ctypes.c_void_p), ("basis", ctypes.c_void_p),
                ("coef", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class CPageTable(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("summarized", ctypes.c_void_p)]


class CStepArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("num_q_heads", ctypes.c_int32),
                ("budget_tokens", ctypes.c_int32), ("agg", ctypes.c_int32),
                ("summaries", CSummaries),
                ("cache", CKVCache), ("pages", CPageTable), ("sel_pages", ctypes.c_void_p),
                ("sel_logmass", ctypes.c_void_p), ("page_logmass", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("out_lse", ctypes.c_void_p), ("ws", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblocks.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run python -m kv_cache_page_rank_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
        P = ctypes.POINTER
        L.locks_workspace_bytes.argtypes = [i32] * 9
        L.locks_workspace_bytes.restype = sz
        L.locks_build_summaries.argtypes = [P(CKVCache), P(CPageTable), vp, P(CSummaries), vp, sz,
                                            vp]
        L.locks_select.argtypes = [vp, i32, P(CSummaries), P(CPageTable), i32, i32, vp, vp, vp,
                                   vp, sz, vp]
        L.locks_select_noalloc.argtypes = [vp, i32, P(CSummaries), P(CPageTable), i32, i32, vp,
                                           vp, vp, vp]
        L.locks_mean_share.argtypes = [vp, i32, i32, P(CPageTable), i32, vp, vp, vp, sz, vp]
        L.locks_refresh_summaries.argtypes = [P(CKVCache), P(CPageTable), vp, i32, P(CSummaries),
                                              vp]
        L.locks_quantize_summaries.argtypes = [P(CSummaries), P(CSummaries), vp]
        L.locks_build_sketch_summaries.argtypes = [P(CKVCache), P(CPageTable), vp, vp,
                                                   P(CSummaries), vp]
        L.locks_scan.argtypes = [vp, i32, P(CSummaries), P(CPageTable), vp, vp, vp, vp]
        L.locks_topk.argtypes = [vp, P(CPageTable), i32, i32, i32, i32, vp, vp, vp, vp]
        L.locks_sparse_attend.argtypes = [vp, i32, P(CKVCache), P(CPageTable), vp, i32, vp, vp,
                                          vp, sz, vp]
        L.locks_dense_attend.argtypes = [vp, i32, P(CKVCache), P(CPageTable), vp, vp, vp, sz, vp]
        L.locks_probe_stream_read.argtypes = [vp, sz, vp, i32, vp]
        L.locks_probe_summary_read.argtypes = [vp, i32, P(CSummaries), P(CPageTable), vp, vp]
        L.locks_step_graph_create.argtypes = [P(CStepArgs), P(vp)]
        L.locks_step_graph_launch.argtypes = [vp, vp]
        L.locks_step_graph_destroy.argtypes = [vp]
        L.locks_step_graph_destroy.restype = None
        L.locks_status_string.argtypes = [i32]
        L.locks_status_string.restype = ctypes.c_char_p
        L.locks_last_hip_error.restype = i32
        L.locks_version.restype = i32
        for fn in ("locks_build_summaries", "locks_select", "locks_scan", "locks_topk",
                   "locks_mean_share", "locks_refresh_summaries", "locks_quantize_summaries",
                   "locks_build_sketch_summaries",
                   "locks_sparse_attend", "locks_dense_attend", "locks_step_graph_create",
                   "locks_step_graph_launch", "locks_probe_stream_read",
                   "locks_probe_summary_read", "locks_select_noalloc"):
            getattr(L, fn).restype = i32
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != LOCKS_OK:
        raise LocksError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------- containers

@dataclass
class PagedKV:
    """K pool [NB][H_kv][P][d] and V pool [NB][H_kv][d][P] (bf16 or float32)."""
    k: torch.Tensor
    v: torch.Tensor | None

    def c(self) -> CKVCache:
        NB, H, P, d = self.k.shape
        dt = {torch.bfloat16: LOCKS_BF16, torch.float32: LOCKS_F32}[self.k.dtype]
        if self.v is not None:
            assert self.v.shape == (NB, H, d, P) and self.v.dtype == self.k.dtype
            assert self.v.is_contiguous()
        assert self.k.is_contiguous()
        return CKVCache(dt, NB, H, P, d, self.k.data_ptr(),
                        self.v.data_ptr() if self.v is not None else None)


@dataclass
class PageTable:
    block_table: torch.Tensor  # [B][max_pages] int32
    seq_lens: torch.Tensor     # [B] int32
    summarized: torch.Tensor | None = None  # [B] int32: leading pages with summaries

    def c(self) -> CPageTable:
        assert self.block_table.dtype == torch.int32 and self.seq_lens.dtype == torch.int32
        assert self.block_table.is_contiguous() and self.seq_lens.is_contiguous()
        if self.summarized is not None:
            assert self.summarized.dtype == torch.int32 and self.summarized.is_contiguous()
        B, MP = self.block_table.shape
        return CPageTable(B, MP, self.block_table.data_ptr(), self.seq_lens.data_ptr(),
                          None if self.summarized is None else self.summarized.data_ptr())


@dataclass
class Summaries:
    mu: torch.Tensor     # [NB][H_kv][d]          (int8 codes for Q8Q4)
    basis: torch.Tensor  # [NB][H_kv][r][d]       (Q8Q4: [NB][H_kv][r][d/2] uint8, int4 pairs)
    coef: torch.Tensor   # [NB][H_kv][P][r]       (int8 codes for Q8Q4)
    scales: torch.Tensor | None = None  # Q8Q4: [NB][H_kv][1 + 2r] float32

    @staticmethod
    def empty(num_blocks, num_kv_heads, page_size, head_dim, rank, device="cuda",
              dtype=torch.float32):
        if dtype == Q8Q4:
            i8 = dict(dtype=torch.int8, device=device)
            return Summaries(torch.empty(num_blocks, num_kv_heads, head_dim, **i8),
                             torch.empty(num_blocks, num_kv_heads, rank, head_dim // 2,
                                         dtype=torch.uint8, device=device),
                             torch.empty(num_blocks, num_kv_heads, page_size, rank, **i8),
                             torch.empty(num_blocks, num_kv_heads, 1 + 2 * rank,
                                         dtype=torch.float32, device=device))
        f = dict(dtype=dtype, device=device)
        return Summaries(torch.empty(num_blocks, num_kv_heads, head_dim, **f),
                         torch.empty(num_blocks, num_kv_heads, rank, head_dim, **f),
                         torch.empty(num_blocks, num_kv_heads, page_size, rank, **f))

    @property
    def quantised(self) -> bool:
        return self.scales is not None

    def c(self) -> CSummaries:
        if self.quantised:
            NB, H, d = self.mu.shape
            r, P = self.basis.shape[2], self.coef.shape[2]
            assert self.mu.dtype == torch.int8 and self.basis.dtype == torch.uint8
            assert self.coef.dtype == torch.int8 and self.scales.dtype == torch.float32
            assert self.basis.shape[3] * 2 == d and self.scales.shape[2] == 1 + 2 * r
            for t in (self.mu, self.basis, self.coef, self.scales):
                assert t.is_contiguous()
            return CSummaries(LOCKS_Q8Q4, NB, H, P, d, r, self.mu.data_ptr(),
                              self.basis.data_ptr(), self.coef.data_ptr(),
                              self.scales.data_ptr())
        NB, H, r, d = self.basis.shape
        P = self.coef.shape[2]
        dt = self.mu.dtype
        assert dt in (torch.float32, torch.bfloat16)
        for t in (self.mu, self.basis, self.coef):
            assert t.dtype == dt and t.is_contiguous()
        return CSummaries(LOCKS_BF16 if dt == torch.bfloat16 else LOCKS_F32, NB, H, P, d, r,
                          self.mu.data_ptr(), self.basis.data_ptr(), self.coef.data_ptr(), None)


def workspace_bytes(op, batch, max_pages, num_q_heads, num_kv_heads, page_size, head_dim, rank,
                    k_pages) -> int:
    return lib().locks_workspace_bytes(op, batch, max_pages, num_q_heads, num_kv_heads, page_size,
                                       head_dim, rank, k_pages)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- entry points

def locks_build_summaries(cache: PagedKV, pages: PageTable, out: Summaries, page_begin=None,
                          stream=None):
    cc, pc, sc = cache.c(), pages.c(), out.c()
    _check(lib().locks_build_summaries(ctypes.byref(cc), ctypes.byref(pc), _ptr(page_begin),
                                       ctypes.byref(sc), None, 0, _stream(stream)),
           "locks_build_summaries")


def locks_scan(q, summaries: Summaries, pages: PageTable, page_logmass, head_logmass=None,
               run_max=None, stream=None):
    sc, pc = summaries.c(), pages.c()
    _check(lib().locks_scan(_ptr(q), q.shape[1], ctypes.byref(sc), ctypes.byref(pc),
                            _ptr(page_logmass), _ptr(head_logmass), _ptr(run_max),
                            _stream(stream)), "locks_scan")


def locks_topk(page_logmass, pages: PageTable, page_size, budget_tokens, sel_pages,
               sel_logmass=None, run_max=None, stream=None):
    pc = pages.c()
    _check(lib().locks_topk(_ptr(page_logmass), ctypes.byref(pc), page_logmass.shape[1],
                            page_size, budget_tokens, sel_pages.shape[-1], _ptr(sel_pages),
                            _ptr(sel_logmass), _ptr(run_max), _stream(stream)), "locks_topk")


def locks_select(q, summaries: Summaries, pages: PageTable, budget_tokens, sel_pages, sel_logmass,
                 page_logmass=None, ws=None, stream=None, agg=AGG_LSE):
    sc, pc = summaries.c(), pages.c()
    _check(lib().locks_select(_ptr(q), q.shape[1], ctypes.byref(sc), ctypes.byref(pc),
                              budget_tokens, agg, _ptr(sel_pages), _ptr(sel_logmass),
                              _ptr(page_logmass), _ptr(ws), 0 if ws is None else ws.numel(),
                              _stream(stream)), "locks_select")


def locks_select_noalloc(q, summaries: Summaries, pages: PageTable, budget_tokens, sel_pages,
                         sel_logmass, page_logmass=None, stream=None, agg=AGG_LSE):
    """locks_select with the library's static per-device scratch instead of a
    workspace (for callers that cannot allocate; calls on one device must not
    overlap)."""
    sc, pc = summaries.c(), pages.c()
    _check(lib().locks_select_noalloc(_ptr(q), q.shape[1], ctypes.byref(sc), ctypes.byref(pc),
                                      budget_tokens, agg, _ptr(sel_pages), _ptr(sel_logmass),
                                      _ptr(page_logmass), _stream(stream)),
           "locks_select_noalloc")


def locks_refresh_summaries(cache: PagedKV, pages: PageTable, page_begin, max_new_pages,
                            out: Summaries, stream=None):
    cc, pc, sc = cache.c(), pages.c(), out.c()
    _check(lib().locks_refresh_summaries(ctypes.byref(cc), ctypes.byref(pc), _ptr(page_begin),
                                         max_new_pages, ctypes.byref(sc), _stream(stream)),
           "locks_refresh_summaries")


def locks_build_sketch_summaries(cache: PagedKV, pages: PageTable, shared_basis, out: Summaries,
                                 page_begin=None, stream=None):
    """Shared-basis sketch (ablation baseline): shared_basis [H_kv][rho][d]
    float32 on the device; out made with rank rho, float32."""
    assert shared_basis.dtype == torch.float32 and shared_basis.is_contiguous()
    cc, pc, sc = cache.c(), pages.c(), out.c()
    _check(lib().locks_build_sketch_summaries(ctypes.byref(cc), ctypes.byref(pc),
                                              _ptr(page_begin), _ptr(shared_basis),
                                              ctypes.byref(sc), _stream(stream)),
           "locks_build_sketch_summaries")


def locks_quantize_summaries(src: Summaries, dst: Summaries, stream=None):
    """fp32 summaries -> int8 / int4 codes and scales (dst made with dtype=Q8Q4)."""
    a, b = src.c(), dst.c()
    _check(lib().locks_quantize_summaries(ctypes.byref(a), ctypes.byref(b), _stream(stream)),
           "locks_quantize_summaries")


def locks_mean_share(head_logmass, num_kv_heads, pages: PageTable, page_size, page_logmass,
                     run_max=None, ws=None, stream=None):
    pc = pages.c()
    _check(lib().locks_mean_share(_ptr(head_logmass), head_logmass.shape[1], num_kv_heads,
                                  ctypes.byref(pc), page_size, _ptr(page_logmass), _ptr(run_max),
                                  _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "locks_mean_share")


def locks_sparse_attend(q, cache: PagedKV, pages: PageTable, sel_pages, out, out_lse=None, ws=None,
                        stream=None):
    cc, pc = cache.c(), pages.c()
    k = sel_pages.shape[-1]
    _check(lib().locks_sparse_attend(_ptr(q), q.shape[1], ctypes.byref(cc), ctypes.byref(pc),
                                     _ptr(sel_pages), k, _ptr(out), _ptr(out_lse), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream(stream)),
           "locks_sparse_attend")


def locks_probe_stream_read(buf, sink, stream=None):
    """Measurement probe: one contiguous read of the device tensor buf
    (its bytes a multiple of 16); sink: float32 device tensor of 4 * blocks
    checksums (blocks = workgroups of 256 threads)."""
    assert sink.dtype == torch.float32
    _check(lib().locks_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                         sink.numel(), _stream(stream)), "locks_probe_stream_read")


def locks_probe_summary_read(q, summaries: Summaries, pages: PageTable, page_out, stream=None):
    """Measurement probe: the fp32 summary scan's reads, in its access
    pattern, without its arithmetic (page_out [B][H_kv][max_pages] float32)."""
    sc, pc = summaries.c(), pages.c()
    _check(lib().locks_probe_summary_read(_ptr(q), q.shape[1], ctypes.byref(sc),
                                          ctypes.byref(pc), _ptr(page_out), _stream(stream)),
           "locks_probe_summary_read")


def locks_dense_attend(q, cache: PagedKV, pages: PageTable, out, out_lse=None, ws=None,
                       stream=None):
    cc, pc = cache.c(), pages.c()
    _check(lib().locks_dense_attend(_ptr(q), q.shape[1], ctypes.byref(cc), ctypes.byref(pc),
                                    _ptr(out), _ptr(out_lse), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(stream)),
           "locks_dense_attend")


class StepGraph:
    """One decode step (select + sparse attend) captured as a HIP graph."""

    def __init__(self, q, summaries: Summaries, cache: PagedKV, pages: PageTable, budget_tokens,
                 sel_pages, sel_logmass, out, out_lse=None, page_logmass=None, ws=None,
                 agg=AGG_LSE):
        self._keep = (q, summaries, cache, pages, sel_pages, sel_logmass, out, out_lse,
                      page_logmass, ws)
        a = CStepArgs(q.data_ptr(), q.shape[1], budget_tokens, agg, summaries.c(), cache.c(),
                      pages.c(), sel_pages.data_ptr(), sel_logmass.data_ptr(),
                      None if page_logmass is None else page_logmass.data_ptr(), out.data_ptr(),
                      None if out_lse is None else out_lse.data_ptr(),
                      None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel())
        h = ctypes.c_void_p()
        _check(lib().locks_step_graph_create(ctypes.byref(a), ctypes.byref(h)),
               "locks_step_graph_create")
        self._h = h

    def launch(self, stream=None):
        _check(lib().locks_step_graph_launch(self._h, _stream(stream)), "locks_step_graph_launch")

    def close(self):
        if self._h:
            lib().locks_step_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
