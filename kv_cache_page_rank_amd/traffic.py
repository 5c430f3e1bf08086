"""Algorithmic byte counts of the decode step (host-side arithmetic for
reporting; no kernel work).

Units: a summary unit is one (full page, KV head); it stores the centroid
(d floats), the basis (r x d floats) and the coefficients (P x r floats).
An attended unit is one (page, KV head) of K and V.
"""
from __future__ import annotations


def summary_unit_bytes(d: int, P: int, r: int, elem=4) -> int:
    """elem: bytes per value (4 fp32, 2 bf16), or "q8q4" for integer codes:
    int8 centroid and coefficients, int4 basis, 1 + 2r fp32 scales."""
    if elem == "q8q4":
        return d + r * d // 2 + P * r + 4 * (1 + 2 * r)
    return elem * (d + r * d + P * r)


def kv_unit_bytes(d: int, P: int, elem: int = 2) -> int:
    return 2 * P * d * elem


def summary_to_cache_ratio(d: int, P: int, r: int, summary_elem: int = 4, kv_elem: int = 2) -> float:
    """Resident summary bytes over the page's K+V bytes."""
    return summary_unit_bytes(d, P, r, summary_elem) / kv_unit_bytes(d, P, kv_elem)


def scan_bytes(batch, num_q_heads, num_kv_heads, max_pages, full_pages, d, P, r,
               summary_elem: int = 4) -> int:
    """Bytes one scan launch must move: every full page's summary, the
    queries, and the page-mass output row."""
    return (full_pages * num_kv_heads * summary_unit_bytes(d, P, r, summary_elem)
            + batch * num_q_heads * d * 4 + batch * num_kv_heads * max_pages * 4)


def step_bytes(full_pages, partial_pages, num_kv_heads, d, P, r, k_pages_total,
               summary_elem: int = 4) -> int:
    """Bytes of one decode step: all summaries + the K/V of the selected pages
    and of each sequence's partial last page."""
    return (full_pages * num_kv_heads * summary_unit_bytes(d, P, r, summary_elem)
            + (k_pages_total + partial_pages * num_kv_heads) * kv_unit_bytes(d, P))


def dense_bytes(total_pages, num_kv_heads, d, P) -> int:
    return total_pages * num_kv_heads * kv_unit_bytes(d, P)


def byte_reduction(summary_fraction: float, budget_tokens: int, context: int) -> float:
    """Per-step KV-read reduction when the summary (a fraction of the cache)
    is read in full and budget_tokens of K/V are attended."""
    return 1.0 / (summary_fraction + budget_tokens / context)
