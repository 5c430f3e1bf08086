"""Upload a generated layer to the GPU in the library's cache layout.

Layout marshalling only: K pool [NB][H_kv][P][d], V pool stored per page
transposed as [NB][H_kv][d][P], int32 page table, float32 queries.
"""
from __future__ import annotations

import numpy as np
import torch


def kv_tensor(arr: np.ndarray, device) -> torch.Tensor:
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(arr).to(device)


def upload(layer, device="cuda"):
    """Returns (q, PagedKV, PageTable) for a workload.Layer."""
    import kv_cache_page_rank_amd as lk
    q = torch.from_numpy(layer.q).to(device)
    k = kv_tensor(layer.k, device)
    v = kv_tensor(layer.v, device).transpose(-1, -2).contiguous()
    pages = lk.PageTable(torch.from_numpy(layer.block_table).to(device),
                         torch.from_numpy(layer.seq_lens).to(device))
    return q, lk.PagedKV(k, v), pages


def summaries_to_device(mu, basis, coef, device="cuda", dtype=torch.float32):
    """Host summaries (float arrays) as device tensors of the given dtype
    (bf16: torch's round-to-nearest-even of the fp32 values)."""
    import kv_cache_page_rank_amd as lk
    return lk.Summaries(*(torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device).to(dtype)
                          for x in (mu, basis, coef)))


def codes_to_device(mu_q, basis_q, coef_q, scales, device="cuda"):
    """Host int8 / int4 summary codes and fp32 scales as device Summaries
    (dtype Q8Q4 in the library's layout)."""
    import kv_cache_page_rank_amd as lk
    return lk.Summaries(torch.from_numpy(np.ascontiguousarray(mu_q, np.int8)).to(device),
                        torch.from_numpy(np.ascontiguousarray(basis_q, np.uint8)).to(device),
                        torch.from_numpy(np.ascontiguousarray(coef_q, np.int8)).to(device),
                        torch.from_numpy(np.ascontiguousarray(scales, np.float32)).to(device))
