"""Seeded synthetic decode-step workloads (ctypes binding of ``locks_workload.c``).

Inputs only: this package holds none of the method's arithmetic.  Both the
oracle and the GPU library read the buffers it makes.

The five workloads are attention layers of a paged KV cache with locally
low-rank keys and planted carrier tokens, shaped like the models the pages
evaluate (Llama-3.1-8B, GLM-4-9B-Chat-1M, Qwen3-4B); there are no weights and
no datasets, so synthetic inputs stand in for the pages' evaluation suites.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "locks_workload.c")
_LIB_PATH = os.path.join(_HERE, "liblocks_workload.so")
_lib = None


def build() -> str:
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                           "-Wextra", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Params(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("subspace_rank", ctypes.c_int32),
                ("carriers", ctypes.c_int32), ("kv_bf16", ctypes.c_int32),
                ("poison_tail", ctypes.c_int32), ("num_threads", ctypes.c_int32),
                ("noise_std", ctypes.c_double), ("page_offset_std", ctypes.c_double),
                ("carrier_gain", ctypes.c_double), ("carrier_cos", ctypes.c_double),
                ("q_std", ctypes.c_double), ("v_std", ctypes.c_double),
                ("seed", ctypes.c_uint64)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.wl_generate.argtypes = [ctypes.POINTER(_Params), ctypes.c_void_p, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p]
        L.wl_generate.restype = ctypes.c_int
        L.wl_hash.argtypes = [ctypes.c_uint64] * 6
        L.wl_hash.restype = ctypes.c_uint64
        L.wl_uniform.argtypes = [ctypes.c_uint64]
        L.wl_uniform.restype = ctypes.c_double
        L.wl_normal.argtypes = [ctypes.c_uint64]
        L.wl_normal.restype = ctypes.c_double
        L.wl_splitmix64.argtypes = [ctypes.c_uint64]
        L.wl_splitmix64.restype = ctypes.c_uint64
        L.wl_f32_to_bf16.argtypes = [ctypes.c_float]
        L.wl_f32_to_bf16.restype = ctypes.c_uint16
        _lib = L
    return _lib


TAG_LENGTHS = 11


@dataclass
class Spec:
    """One synthetic attention layer plus the method's parameters for it."""
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    seq_lens: list
    rank: int
    budget_tokens: int
    subspace_rank: int
    carriers: int
    kv_bf16: bool
    seed: int
    noise_std: float = 0.05
    page_offset_std: float = 0.0
    carrier_gain: float = 1.0
    carrier_cos: float = 0.9
    q_std: float | None = None  # default 1/sqrt(d)
    v_std: float = 1.0
    poison_tail: bool = True
    budgets: list = field(default_factory=list)

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def pages_per_seq(self):
        return [-(-n // self.page_size) for n in self.seq_lens]

    @property
    def max_pages(self):
        return max(self.pages_per_seq)

    @property
    def num_blocks(self):
        return sum(self.pages_per_seq)

    @property
    def k_pages(self):
        return self.budget_tokens // self.page_size

    def with_(self, **kw) -> "Spec":
        return replace(self, **kw)


def uniform_lengths(seed: int, n: int, lo: int, hi: int) -> list:
    """n lengths drawn uniformly from {lo, ..., hi} with the counter-based hash."""
    L = lib()
    return [lo + int(L.wl_uniform(L.wl_hash(seed, TAG_LENGTHS, b, 0, 0, 0)) * (hi - lo + 1))
            for b in range(n)]


def config(idx: int) -> Spec:
    """The five workloads (seed 1000 + index).

    0: tiny CPU-checkable layer: 1 query head, 1 KV head, d 64, P 16, 64 pages,
       r 4, fp32, budget 8 pages, 6-dim page subspaces, 3 carriers.
    1: Llama-3.1-8B-shaped layer: 32/8 heads, d 128, P 64, 128K tokens, bf16 K/V,
       r 8, budget 2048, 12-dim subspaces, 16 carriers per KV head.
    2: GLM-4-9B-shaped layer at 1M tokens: 32/2 heads (GQA 16), r 8, budget 2048,
       64 carriers per KV head.
    3: workload 2 at r 2, budgets 512/1024/2048/4096.
    4: Qwen3-4B-shaped batch of 16 sequences of 32K..256K tokens: 32/8 heads, r 8,
       budget 2048 per sequence, 16 carriers per KV head.
    """
    if idx == 0:
        return Spec("tiny-1h-d64-p16-1k", 1, 1, 1, 64, 16, [1024], 4, 128, 6, 3, False, 1000)
    if idx == 1:
        return Spec("llama31-8b-layer-128k", 1, 32, 8, 128, 64, [131072], 8, 2048, 12, 16, True,
                    1001)
    if idx == 2:
        return Spec("glm4-9b-layer-1m", 1, 32, 2, 128, 64, [1048576], 8, 2048, 12, 64, True, 1002)
    if idx == 3:
        return Spec("glm4-9b-layer-1m-r2", 1, 32, 2, 128, 64, [1048576], 2, 2048, 12, 64, True,
                    1003, budgets=[512, 1024, 2048, 4096])
    if idx == 4:
        lens = uniform_lengths(1004, 16, 32768, 262144)
        return Spec("qwen3-4b-batch16-32k-256k", 16, 32, 8, 128, 64, lens, 8, 2048, 12, 16, True,
                    1004)
    raise ValueError(idx)


@dataclass
class Layer:
    spec: Spec
    q: np.ndarray            # [B][Hq][d] float32
    k: np.ndarray            # [NB][Hkv][P][d] uint16 (bf16 bits) or float32
    v: np.ndarray
    block_table: np.ndarray  # [B][max_pages] int32
    seq_lens: np.ndarray     # [B] int32
    carrier_page: np.ndarray  # [B][Hkv][n_c] int32
    carrier_slot: np.ndarray

    def k_f32(self) -> np.ndarray:
        return bf16_to_f32(self.k) if self.k.dtype == np.uint16 else self.k

    def v_f32(self) -> np.ndarray:
        return bf16_to_f32(self.v) if self.v.dtype == np.uint16 else self.v


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def make(spec: Spec, threads: int = 0) -> Layer:
    B, Hq, Hkv, d, P = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, \
        spec.page_size
    seq = np.asarray(spec.seq_lens, np.int32)
    NB, MP = spec.num_blocks, spec.max_pages
    kv_dtype = np.uint16 if spec.kv_bf16 else np.float32
    q = np.zeros((B, Hq, d), np.float32)
    k = np.empty((NB, Hkv, P, d), kv_dtype)
    v = np.empty((NB, Hkv, P, d), kv_dtype)
    bt = np.zeros((B, MP), np.int32)
    nc = spec.carriers
    cp = np.zeros((B, Hkv, max(nc, 1)), np.int32)
    cs = np.zeros((B, Hkv, max(nc, 1)), np.int32)
    p = _Params(B, Hq, Hkv, d, P, spec.subspace_rank, nc, int(spec.kv_bf16),
                int(spec.poison_tail), threads, spec.noise_std, spec.page_offset_std,
                spec.carrier_gain, spec.carrier_cos,
                spec.q_std if spec.q_std is not None else 1.0 / math.sqrt(d), spec.v_std,
                spec.seed)
    rc = lib().wl_generate(ctypes.byref(p), seq.ctypes.data, MP, NB, q.ctypes.data,
                           k.ctypes.data, v.ctypes.data, bt.ctypes.data, cp.ctypes.data,
                           cs.ctypes.data)
    if rc != 0:
        raise ValueError(f"workload generation failed ({rc})")
    return Layer(spec, q, k, v, bt, seq, cp[:, :, :nc], cs[:, :, :nc])
