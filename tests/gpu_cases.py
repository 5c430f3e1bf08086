"""Shared set-up of the GPU parity tests: seeded workloads, the oracle on the
same inputs, device copies in the library's layout."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import workload
from workload.device import summaries_to_device, upload

DEV = "cuda"


def say(*a):
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def tiny(**kw) -> workload.Spec:
    return workload.config(0).with_(**kw)


def bf16_small(**kw) -> workload.Spec:
    """bf16, P 64, d 128 layer small enough for the full oracle (several tiles,
    ragged partial pages, two sequences)."""
    base = workload.Spec("bf16-small", 2, 32, 2, 128, 64, [64 * 40 + 17, 64 * 23], 8, 512, 12, 4,
                         True, 77)
    return base.with_(**kw)


class Case:
    """A layer with its oracle layout and device copies."""

    def __init__(self, spec: workload.Spec, threads: int = 0):
        self.spec = spec
        self.layer = workload.make(spec, threads=threads)
        self.lay = oracle.Layout(spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                                 spec.page_size, self.layer.block_table, self.layer.seq_lens)
        self.q, self.kv, self.pages = upload(self.layer, DEV)
        self._kf = None

    @property
    def k_f32(self):
        if self._kf is None:
            self._kf = self.layer.k_f32()
        return self._kf

    def oracle_summaries(self, rank=None):
        r = self.spec.rank if rank is None else rank
        return oracle.build_pool(self.lay, r, self.k_f32, self.spec.num_blocks)

    def full_pages(self):
        return [n // self.spec.page_size for n in self.spec.seq_lens]


def shifted_log2_sums(case, q_host, mu, page_o):
    """log2 of each full page's sum of 2^logit after the shift by the page's
    largest centroid term over the group's heads, from the oracle's masses
    (mass / ln 2 minus that term): where the scan's shifted form holds
    (inside [-60, 60]) and where it takes the exact form."""
    s = case.spec
    H, G, d, P = s.num_kv_heads, s.group, s.head_dim, s.page_size
    mu = np.asarray(mu).reshape(s.num_blocks, H, d)
    out = []
    for b in range(s.batch):
        for g in range(H):
            for j in range(s.seq_lens[b] // P):
                m = mu[case.layer.block_table[b, j], g].astype(np.float64)
                beta = q_host[b, g * G:(g + 1) * G].astype(np.float64) @ m / np.sqrt(d)
                out.append((page_o[b, g, j] - beta.max()) / np.log(2))
    return np.array(out)


def masses_close(gpu, orc, atol=1e-4):
    """|a_gpu - a_orc| <= atol in the log domain (relative 1e-4 on the mass),
    with identical -inf entries."""
    gpu = np.asarray(gpu, np.float64)
    orc = np.asarray(orc, np.float64)
    inf_g, inf_o = np.isneginf(gpu), np.isneginf(orc)
    assert np.array_equal(inf_g, inf_o), "-inf pattern differs"
    fin = ~inf_o
    err = np.abs(gpu[fin] - orc[fin])
    return float(err.max()) if err.size else 0.0


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (2^(floor(log2|x|) - 7))."""
    ax = np.maximum(np.abs(x), 1e-30)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def out_tol(orc_out, is_bf16):
    if is_bf16:
        return np.maximum(1e-2, bf16_ulp(orc_out))
    return 1e-5


def band_ok(gpu_sel, orc_sel, orc_mass, k, band=1e-3):
    """Selected sets equal except for pages whose oracle mass lies within
    `band` of the oracle's k-th largest value."""
    g = set(int(x) for x in gpu_sel if x >= 0)
    o = set(int(x) for x in orc_sel if x >= 0)
    if g == o:
        return True
    if len(g) != len(o):
        return False
    kth = np.sort(orc_mass)[::-1][k - 1]
    for j in g ^ o:
        if abs(orc_mass[j] - kth) > band:
            return False
    return True


def to_np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


class SubPool:
    """One sequence b and one KV group g of a layer, re-laid out as a compact
    pool (pages in logical order, block table 0..n-1) for the oracle.  Data
    slicing only.  Keys/values are widened to float32 for the pages kept."""

    def __init__(self, layer, spec, b, g):
        P = spec.page_size
        n = int(layer.seq_lens[b])
        npg = -(-n // P)
        blocks = layer.block_table[b, :npg]
        G = spec.group
        k = layer.k[blocks, g][:, None]  # [npg][1][P][d]
        v = layer.v[blocks, g][:, None]
        self.k = workload.bf16_to_f32(k) if k.dtype == np.uint16 else np.ascontiguousarray(k)
        self.v = workload.bf16_to_f32(v) if v.dtype == np.uint16 else np.ascontiguousarray(v)
        self.q = np.ascontiguousarray(layer.q[b:b + 1, g * G:(g + 1) * G])
        self.blocks = blocks
        self.lay = oracle.Layout(G, 1, spec.head_dim, P, np.arange(npg, dtype=np.int32)[None],
                                 np.array([n], np.int32))

    def units(self, pages):
        return np.array([[0, 0, j] for j in pages], np.int32)
