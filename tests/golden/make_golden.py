"""Writes the stored fixtures under tests/golden/.

Run from the repository root: ``python tests/golden/make_golden.py``.
Stored expected values come only from closed forms or from the CPU oracle
(``oracle/``) on inputs made by ``workload/``; nothing here touches the GPU
library.
"""
import json
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workload  # noqa: E402


def exact_lse_worked_example():
    """Closed form: d = 4, q = (2, 0, 0, 0) = (sqrt(d), 0, 0, 0), so the logit of
    token i is its first coordinate; first coordinates log(1), ..., log(P) give
    the page LSE log(P (P + 1) / 2)."""
    P, d = 12, 4
    keys = [[math.log(i + 1), 0.25 * (i % 3), -0.5, float(i)] for i in range(P)]
    return {"source": "closed form, see make_golden.py", "q": [2.0, 0.0, 0.0, 0.0],
            "keys": keys, "expected": math.log(P * (P + 1) / 2)}


def tiny_oracle_outputs():
    """Oracle outputs on the tiny workload (1 head, d 64, P 16, 64 pages, r 4,
    budget 8 pages): regression fixture for the oracle itself."""
    spec = workload.config(0)
    layer = workload.make(spec)
    lay = oracle.Layout(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        layer.block_table, layer.seq_lens)
    mu, basis, coef = oracle.build_pool(lay, spec.rank, layer.k_f32(), spec.num_blocks)
    _, page = oracle.scan_pool(lay, spec.rank, layer.q, mu, basis, coef)
    _, exact = oracle.exact_pool(lay, layer.q, layer.k_f32())
    sel, sm = oracle.select_pool(lay, spec.budget_tokens, page.astype(np.float32), spec.k_pages)
    out, lse = oracle.attend_pool(lay, layer.q, layer.k_f32(), layer.v_f32(), sel)
    dense, dlse = oracle.attend_pool(lay, layer.q, layer.k_f32(), layer.v_f32(), None)
    return {"source": "oracle/ on workload.config(0), see make_golden.py",
            "page_mass": page[0, 0].tolist(), "exact_page_lse": exact[0, 0].tolist(),
            "selected": sel[0, 0].tolist(), "carriers": layer.carrier_page[0, 0].tolist(),
            "sparse_out": out[0, 0].tolist(), "sparse_lse": float(lse[0, 0]),
            "dense_out": dense[0, 0].tolist(), "dense_lse": float(dlse[0, 0])}


if __name__ == "__main__":
    for name, fn in [("exact_lse_worked_example.json", exact_lse_worked_example),
                     ("tiny_oracle_outputs.json", tiny_oracle_outputs)]:
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(fn(), f, indent=1)
        print("wrote", name)
