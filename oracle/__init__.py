"""ctypes binding of the CPU oracle (``locks_oracle.c``).

TEST INFRASTRUCTURE ONLY: the oracle is the plain, slow, double-precision
reference the GPU library is checked against.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg import this package.  It shares
no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "locks_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblocks_oracle.so")
_lib = None

_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")


def build() -> str:
    """Compile the oracle with gcc (plain IEEE double, no fast-math)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                           "-Wextra", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("summarized", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        c_int, c_double = ctypes.c_int, ctypes.c_double
        lay = ctypes.POINTER(_Layout)
        L.orc_lse.argtypes = [c_int, _f64p]
        L.orc_lse.restype = c_double
        L.orc_page_summary.argtypes = [c_int, c_int, c_int, _f64p, _f64p, _f64p, _f64p, _f64p]
        L.orc_page_summary.restype = c_int
        L.orc_page_estimate.argtypes = [c_int, c_int, c_int, _f64p, _f64p, _f64p, _f64p]
        L.orc_page_estimate.restype = c_double
        L.orc_page_exact_lse.argtypes = [c_int, c_int, _f64p, _f64p]
        L.orc_page_exact_lse.restype = c_double
        L.orc_select_topk.argtypes = [c_int, _f32p, c_int, c_int, _i32p, _f32p]
        L.orc_select_topk.restype = c_int
        L.orc_attend_tokens.argtypes = [c_int, c_int, _f64p, _f64p, _f64p, _f64p,
                                        ctypes.POINTER(c_double)]
        L.orc_attend_tokens.restype = None
        L.orc_build_pool.argtypes = [lay, c_int, _f32p, _f32p, _f32p, _f32p, ctypes.c_void_p,
                                     c_int]
        L.orc_build_units.argtypes = [lay, c_int, _f32p, c_int, _i32p, _i32p, _i32p, _f64p,
                                      _f64p, _f64p, _f64p, c_int]
        L.orc_scan_pool.argtypes = [lay, c_int, _f32p, _f32p, _f32p, _f32p, ctypes.c_void_p,
                                    ctypes.c_void_p, c_int]
        L.orc_scan_units.argtypes = [lay, c_int, _f32p, _f32p, _f32p, _f32p, c_int, _i32p,
                                     _i32p, _i32p, _f64p, _f64p]
        L.orc_exact_pool.argtypes = [lay, _f32p, _f32p, ctypes.c_void_p, ctypes.c_void_p, c_int]
        L.orc_share_pool.argtypes = [lay, _f64p, _f64p]
        L.orc_select_pool.argtypes = [lay, c_int, _f32p, c_int, _i32p, ctypes.c_void_p]
        L.orc_attend_pool.argtypes = [lay, _f32p, _f32p, _f32p, ctypes.c_void_p, c_int, _f64p,
                                      ctypes.c_void_p, c_int]
        vp = ctypes.c_void_p
        L.orc_pooled_covariance.argtypes = [lay, vp, vp, c_int]
        L.orc_sketch_pool.argtypes = [lay, c_int, vp, vp, vp, vp, c_int]
        L.orc_quantize_vec.argtypes = [c_int, c_int, vp, c_int, vp, vp]
        L.orc_quantize_vec.restype = None
        L.orc_quantize_pool.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp,
                                        vp, vp]
        L.orc_dequantize_pool.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp,
                                          vp, vp]
        for fn in ("orc_build_pool", "orc_build_units", "orc_scan_pool", "orc_scan_units",
                   "orc_exact_pool", "orc_select_pool", "orc_attend_pool", "orc_quantize_pool",
                   "orc_dequantize_pool", "orc_pooled_covariance", "orc_sketch_pool"):
            getattr(L, fn).restype = c_int
        _lib = L
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


# ------------------------------------------------------------------ single page

def lse(x) -> float:
    x = _f64(x).ravel()
    return lib().orc_lse(x.size, x)


def page_summary(keys, r: int):
    """Summary of one page: (mu[d], basis[r][d], coef[P][r], sigma[min(P,d)], sweeps)."""
    keys = _f64(keys)
    P, d = keys.shape
    mu = np.zeros(d)
    basis = np.zeros((max(r, 0), d))
    coef = np.zeros((P, max(r, 0)))
    sigma = np.zeros(min(P, d))
    sweeps = lib().orc_page_summary(P, d, r, keys, mu, basis.reshape(-1) if r else np.zeros(1),
                                    coef.reshape(-1) if r else np.zeros(1), sigma)
    if sweeps < 0:
        raise ValueError("invalid rank")
    return mu, basis, coef, sigma, sweeps


def page_estimate(q, mu, basis, coef) -> float:
    q, mu = _f64(q), _f64(mu)
    basis, coef = _f64(basis), _f64(coef)
    P = coef.shape[0]
    r = basis.shape[0]
    return lib().orc_page_estimate(P, q.size, r, q, mu, basis.reshape(-1) if r else np.zeros(1),
                                   coef.reshape(-1) if r else np.zeros(1))


def page_exact_lse(q, keys) -> float:
    q, keys = _f64(q), _f64(keys)
    return lib().orc_page_exact_lse(keys.shape[0], q.size, q, keys.reshape(-1) if keys.size
                                    else np.zeros(1))


def select_topk(mass, k: int, width: int | None = None):
    mass = _f32(mass).ravel()
    width = k if width is None else width
    sel = np.zeros(max(width, 1), np.int32)
    sm = np.zeros(max(width, 1), np.float32)
    kk = lib().orc_select_topk(mass.size, mass, k, width, sel, sm)
    return sel[:width], sm[:width], kk


def attend_tokens(q, keys, vals):
    q, keys, vals = _f64(q), _f64(keys), _f64(vals)
    d = q.size
    out = np.zeros(d)
    l = ctypes.c_double()
    n = keys.shape[0]
    lib().orc_attend_tokens(n, d, q, keys.reshape(-1) if n else np.zeros(1),
                            vals.reshape(-1) if n else np.zeros(1), out, ctypes.byref(l))
    return out, l.value


# ------------------------------------------------------------------ paged cache

@dataclass
class Layout:
    """Paged layout: block_table [B][max_pages] int32, seq_lens [B] int32;
    summarized [B] int32 or None: the leading pages of each sequence whose
    summaries exist (None: every full page)."""
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    block_table: np.ndarray
    seq_lens: np.ndarray
    summarized: np.ndarray | None = None

    def __post_init__(self):
        self.block_table = _i32(self.block_table)
        self.seq_lens = _i32(self.seq_lens)
        if self.summarized is not None:
            self.summarized = _i32(self.summarized)

    @property
    def batch(self):
        return self.block_table.shape[0]

    @property
    def max_pages(self):
        return self.block_table.shape[1]

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    def c(self):
        s = _Layout(self.batch, self.num_q_heads, self.num_kv_heads, self.head_dim,
                    self.page_size, self.max_pages, self.block_table.ctypes.data,
                    self.seq_lens.ctypes.data,
                    None if self.summarized is None else self.summarized.ctypes.data)
        return ctypes.byref(s), s


def build_pool(L: Layout, r: int, k_pool, num_blocks: int, threads: int = 0,
               with_sigma: bool = False):
    """fp32 summaries (mu, basis, coef) of every full page at its physical
    block; with_sigma also returns the singular values [NB][Hkv][min(P,d)]
    (double; zero for blocks that hold no full page)."""
    k_pool = _f32(k_pool)
    H, P, d = L.num_kv_heads, L.page_size, L.head_dim
    mu = np.zeros((num_blocks, H, d), np.float32)
    basis = np.zeros((num_blocks, H, max(r, 1), d), np.float32)[:, :, :r]
    basis = np.ascontiguousarray(basis)
    coef = np.zeros((num_blocks, H, P, r), np.float32)
    sigma = np.zeros((num_blocks, H, min(P, d))) if with_sigma else None
    ref, _keep = L.c()
    _check(lib().orc_build_pool(ref, r, k_pool.reshape(-1), mu.reshape(-1),
                                basis.reshape(-1) if basis.size else np.zeros(1, np.float32),
                                coef.reshape(-1) if coef.size else np.zeros(1, np.float32),
                                _ptr(sigma), threads), "build_pool")
    return (mu, basis, coef, sigma) if with_sigma else (mu, basis, coef)


def build_units(L: Layout, r: int, k_pool, units, threads: int = 0):
    """units: int array [n][3] of (b, g, j). Returns double mu, basis, coef, sigma."""
    units = _i32(units).reshape(-1, 3)
    n = units.shape[0]
    P, d = L.page_size, L.head_dim
    mu = np.zeros((n, d))
    basis = np.zeros((n, r, d))
    coef = np.zeros((n, P, r))
    sigma = np.zeros((n, min(P, d)))
    ref, _keep = L.c()
    _check(lib().orc_build_units(ref, r, _f32(k_pool).reshape(-1), n,
                                 _i32(units[:, 0]), _i32(units[:, 1]), _i32(units[:, 2]),
                                 mu.reshape(-1), basis.reshape(-1) if basis.size else np.zeros(1),
                                 coef.reshape(-1) if coef.size else np.zeros(1),
                                 sigma.reshape(-1), threads), "build_units")
    return mu, basis, coef, sigma


def _ptr(a):
    return None if a is None else a.ctypes.data


def scan_pool(L: Layout, r: int, q, mu, basis, coef, threads: int = 0, heads: bool = True):
    q, mu, basis, coef = _f32(q), _f32(mu), _f32(basis), _f32(coef)
    head = np.zeros((L.batch, L.num_q_heads, L.max_pages)) if heads else None
    page = np.zeros((L.batch, L.num_kv_heads, L.max_pages))
    ref, _keep = L.c()
    _check(lib().orc_scan_pool(ref, r, q.reshape(-1), mu.reshape(-1),
                               basis.reshape(-1) if basis.size else np.zeros(1, np.float32),
                               coef.reshape(-1) if coef.size else np.zeros(1, np.float32),
                               _ptr(head), _ptr(page), threads), "scan_pool")
    return head, page


def scan_units(L: Layout, r: int, q, mu, basis, coef, units):
    units = _i32(units).reshape(-1, 3)
    n = units.shape[0]
    head = np.zeros((n, L.group))
    page = np.zeros(n)
    ref, _keep = L.c()
    _check(lib().orc_scan_units(ref, r, _f32(q).reshape(-1), _f32(mu).reshape(-1),
                                _f32(basis).reshape(-1), _f32(coef).reshape(-1), n,
                                _i32(units[:, 0]), _i32(units[:, 1]), _i32(units[:, 2]),
                                head.reshape(-1), page), "scan_units")
    return head, page


def exact_pool(L: Layout, q, k_pool, threads: int = 0):
    head = np.zeros((L.batch, L.num_q_heads, L.max_pages))
    page = np.zeros((L.batch, L.num_kv_heads, L.max_pages))
    ref, _keep = L.c()
    _check(lib().orc_exact_pool(ref, _f32(q).reshape(-1), _f32(k_pool).reshape(-1),
                                _ptr(head), _ptr(page), threads), "exact_pool")
    return head, page


def share_pool(L: Layout, head_mass):
    """Mean-of-share group scores [B][Hkv][max_pages] (log of the group's mean
    share) from per-head estimates [B][Hq][max_pages]."""
    hm = np.ascontiguousarray(head_mass, np.float64)
    out = np.zeros((L.batch, L.num_kv_heads, L.max_pages))
    ref, _keep = L.c()
    _check(lib().orc_share_pool(ref, hm.reshape(-1), out.reshape(-1)), "share_pool")
    return out


def select_pool(L: Layout, budget_tokens: int, page_mass_f32, width: int):
    pm = _f32(page_mass_f32)
    sel = np.zeros((L.batch, L.num_kv_heads, max(width, 1)), np.int32)
    sm = np.zeros((L.batch, L.num_kv_heads, max(width, 1)), np.float32)
    ref, _keep = L.c()
    _check(lib().orc_select_pool(ref, budget_tokens, pm.reshape(-1), width, sel.reshape(-1),
                                 sm.ctypes.data), "select_pool")
    return sel[:, :, :width], sm[:, :, :width]


def attend_pool(L: Layout, q, k_pool, v_pool, sel_pages=None, threads: int = 0):
    out = np.zeros((L.batch, L.num_q_heads, L.head_dim))
    lse_ = np.zeros((L.batch, L.num_q_heads))
    width = 0
    sel = None
    if sel_pages is not None:
        sel = _i32(sel_pages)
        width = sel.shape[-1]
    ref, _keep = L.c()
    _check(lib().orc_attend_pool(ref, _f32(q).reshape(-1), _f32(k_pool).reshape(-1),
                                 _f32(v_pool).reshape(-1), _ptr(sel), width, out.reshape(-1),
                                 lse_.ctypes.data, threads), "attend_pool")
    return out, lse_


# ------------------------------------------------------------------ quantised summaries
def quantize_vec(x, qmax: int):
    """Symmetric absmax quantisation of one float32 vector (technical summary,
    section 2, "Kwantisatie"; reading in locks_oracle.h): (scale, int8 codes)."""
    xs = _f32(x).reshape(-1)
    code = np.zeros(xs.shape, np.int8)
    scale = np.zeros(1, np.float32)
    lib().orc_quantize_vec(xs.size, 1, xs.ctypes.data, qmax, scale.ctypes.data, code.ctypes.data)
    return float(scale[0]), code


def quantize_pool(mu, basis, coef):
    """fp32 summary arrays mu [NB][Hkv][d], basis [NB][Hkv][r][d], coef
    [NB][Hkv][P][r] -> (mu_q int8, basis_q packed uint8 [NB][Hkv][r][d/2],
    coef_q int8, scales float32 [NB][Hkv][1+2r])."""
    mu, basis, coef = _f32(mu), _f32(basis), _f32(coef)
    NB, H, r, d = basis.shape
    P = coef.shape[2]
    mu_q = np.zeros((NB, H, d), np.int8)
    basis_q = np.zeros((NB, H, r, d // 2), np.uint8)
    coef_q = np.zeros((NB, H, P, r), np.int8)
    scales = np.zeros((NB, H, 1 + 2 * r), np.float32)
    _check(lib().orc_quantize_pool(NB, H, P, d, r, mu.ctypes.data, basis.ctypes.data,
                                   coef.ctypes.data, mu_q.ctypes.data, basis_q.ctypes.data,
                                   coef_q.ctypes.data, scales.ctypes.data), "quantize_pool")
    return mu_q, basis_q, coef_q, scales


def dequantize_pool(mu_q, basis_q, coef_q, scales):
    """Inverse of quantize_pool up to the codes: float32 (mu, basis, coef)."""
    mu_q = np.ascontiguousarray(mu_q, np.int8)
    basis_q = np.ascontiguousarray(basis_q, np.uint8)
    coef_q = np.ascontiguousarray(coef_q, np.int8)
    scales = _f32(scales)
    NB, H, r, dh = basis_q.shape
    d, P = 2 * dh, coef_q.shape[2]
    mu = np.zeros((NB, H, d), np.float32)
    basis = np.zeros((NB, H, r, d), np.float32)
    coef = np.zeros((NB, H, P, r), np.float32)
    _check(lib().orc_dequantize_pool(NB, H, P, d, r, mu_q.ctypes.data, basis_q.ctypes.data,
                                     coef_q.ctypes.data, scales.ctypes.data, mu.ctypes.data,
                                     basis.ctypes.data, coef.ctypes.data), "dequantize_pool")
    return mu, basis, coef


# ------------------------------------------------------------------ shared-basis sketch
def pooled_covariance(L: Layout, k_pool, threads: int = 0):
    """sum over every full page of Kc^T Kc, per KV head: [Hkv][d][d] float64."""
    kp = _f32(k_pool)
    cov = np.zeros((L.num_kv_heads, L.head_dim, L.head_dim))
    ref, _keep = L.c()
    _check(lib().orc_pooled_covariance(ref, kp.ctypes.data, cov.ctypes.data, threads),
           "pooled_covariance")
    return cov


def shared_basis(L: Layout, rho: int, k_pool, threads: int = 0):
    """One rank-rho basis per KV head for the shared-basis ablation (reading in
    locks_oracle.h): the top rho eigenvectors of the pooled within-page
    covariance, eigenvalues descending (LAPACK eigh as the eigensolver).
    Returns (basis [Hkv][rho][d] float64 rows, eigenvalues [Hkv][d] descending)."""
    cov = pooled_covariance(L, k_pool, threads)
    H, d = L.num_kv_heads, L.head_dim
    basis = np.zeros((H, rho, d))
    eig = np.zeros((H, d))
    for g in range(H):
        w, v = np.linalg.eigh(cov[g])
        order = np.argsort(-w, kind="stable")
        eig[g] = w[order]
        basis[g] = v[:, order[:rho]].T
    return basis, eig


def sketch_pool(L: Layout, rho: int, k_pool, basis, num_blocks: int, threads: int = 0):
    """Summaries of the shared-basis sketch in the page-summary layout, for the
    same estimator: mu [NB][Hkv][d], the shared basis copied to every block
    [NB][Hkv][rho][d], coordinates [NB][Hkv][P][rho] (float32)."""
    kp = _f32(k_pool)
    B = np.ascontiguousarray(basis, np.float64)
    H, d, P = L.num_kv_heads, L.head_dim, L.page_size
    mu = np.zeros((num_blocks, H, d), np.float32)
    coef = np.zeros((num_blocks, H, P, rho), np.float32)
    ref, _keep = L.c()
    _check(lib().orc_sketch_pool(ref, rho, kp.ctypes.data, B.ctypes.data, mu.ctypes.data,
                                 coef.ctypes.data, threads), "sketch_pool")
    rep = np.broadcast_to(B.astype(np.float32)[None], (num_blocks, H, rho, d)).copy()
    return mu, rep, coef
