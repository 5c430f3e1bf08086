"""The decode step captured as one HIP graph: replays equal eager runs
bitwise, also with eager work and synchronisation between replays."""
import numpy as np
import pytest
import torch

from gpu_cases import DEV, Case, bf16_small, say, tiny
import oracle
from workload.device import codes_to_device, summaries_to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mk,sdt,agg", [(lambda: tiny(), torch.float32, 0),
                                        (lambda: bf16_small(), torch.float32, 0),
                                        (lambda: bf16_small(), torch.bfloat16, 0),
                                        (lambda: bf16_small(), "q8q4", 0),
                                        (lambda: bf16_small(), torch.float32, 1)],
                         ids=["tiny", "bf16", "bf16-summaries", "code-summaries", "mean-share"])
def test_graph_replay_equals_eager(mk, sdt, agg):
    import kv_cache_page_rank_amd as lk
    case = Case(mk())
    s = case.spec
    if sdt == "q8q4":
        summ = codes_to_device(*oracle.quantize_pool(*case.oracle_summaries()))
    else:
        summ = summaries_to_device(*case.oracle_summaries(), dtype=sdt)
    k = s.k_pages
    ws_b = lk.workspace_bytes(lk.OP_STEP, s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads,
                              s.page_size, s.head_dim, s.rank, k)

    def bufs():
        return dict(sel=torch.full((s.batch, s.num_kv_heads, k), -9, dtype=torch.int32,
                                   device=DEV),
                    mass=torch.zeros((s.batch, s.num_kv_heads, k), device=DEV),
                    out=torch.zeros((s.batch, s.num_q_heads, s.head_dim), dtype=case.kv.k.dtype,
                                    device=DEV),
                    lse=torch.zeros((s.batch, s.num_q_heads), device=DEV),
                    ws=lk.workspace(ws_b))

    e = bufs()
    say("eager step")
    lk.locks_select(case.q, summ, case.pages, s.budget_tokens, e["sel"], e["mass"], ws=e["ws"],
                    agg=agg)
    attn_ws = e["ws"][lk.workspace_bytes(lk.OP_SELECT, s.batch, s.max_pages, s.num_q_heads,
                                         s.num_kv_heads, s.page_size, s.head_dim, s.rank, k):]
    lk.locks_sparse_attend(case.q, case.kv, case.pages, e["sel"], e["out"], e["lse"], ws=attn_ws)
    torch.cuda.synchronize()

    g = bufs()
    say("graph create")
    graph = lk.StepGraph(case.q, summ, case.kv, case.pages, s.budget_tokens, g["sel"], g["mass"],
                         g["out"], g["lse"], ws=g["ws"], agg=agg)
    for rep in range(4):
        for t in (g["sel"], g["mass"], g["out"], g["lse"]):
            t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        say("graph replay", rep)
        graph.launch()
        torch.cuda.synchronize()
        for key in ("sel", "mass", "out", "lse"):
            assert torch.equal(g[key], e[key]), (rep, key)
    graph.close()


def test_graph_replays_follow_new_queries_and_lengths():
    """A decode loop on one captured step: between replays the query is
    rewritten in place and a sequence grows by a token inside its partial
    page (no page completes).  Every replay equals an eager step on the same
    buffers bitwise, and the selection and output change with the query, so
    the graph reads the buffers' current contents rather than its first
    ones."""
    import kv_cache_page_rank_amd as lk
    case = Case(bf16_small())
    s = case.spec
    P = s.page_size
    summ = summaries_to_device(*case.oracle_summaries())
    k = s.k_pages
    ws_b = lk.workspace_bytes(lk.OP_STEP, s.batch, s.max_pages, s.num_q_heads, s.num_kv_heads,
                              P, s.head_dim, s.rank, k)
    sel_b = lk.workspace_bytes(lk.OP_SELECT, s.batch, s.max_pages, s.num_q_heads,
                               s.num_kv_heads, P, s.head_dim, s.rank, k)

    def bufs():
        return dict(sel=torch.empty((s.batch, s.num_kv_heads, k), dtype=torch.int32, device=DEV),
                    mass=torch.empty((s.batch, s.num_kv_heads, k), device=DEV),
                    out=torch.empty((s.batch, s.num_q_heads, s.head_dim), dtype=case.kv.k.dtype,
                                    device=DEV),
                    lse=torch.empty((s.batch, s.num_q_heads), device=DEV),
                    ws=lk.workspace(ws_b))

    q = case.q.clone()
    lens = case.pages.seq_lens.clone()
    pages = lk.PageTable(case.pages.block_table, lens)
    g = bufs()
    graph = lk.StepGraph(q, summ, case.kv, pages, s.budget_tokens, g["sel"], g["mass"], g["out"],
                         g["lse"], ws=g["ws"])
    gen = torch.Generator(device="cpu").manual_seed(5)
    prev = None
    for step in range(4):
        if step > 0:
            q.copy_((torch.randn(q.shape, generator=gen) / s.head_dim ** 0.5).to(DEV))
            host = lens.cpu().numpy()
            grow = (host % P != 0) & (host % P != P - 1)
            lens.copy_(torch.from_numpy(np.where(grow, host + 1, host).astype(np.int32)).to(DEV))
        torch.cuda.synchronize()
        say("decode step", step, lens.tolist())
        graph.launch()
        e = bufs()
        lk.locks_select(q, summ, pages, s.budget_tokens, e["sel"], e["mass"], ws=e["ws"])
        lk.locks_sparse_attend(q, case.kv, pages, e["sel"], e["out"], e["lse"],
                               ws=e["ws"][sel_b:])
        torch.cuda.synchronize()
        for key in ("sel", "mass", "out", "lse"):
            assert torch.equal(g[key], e[key]), (step, key)
        if prev is not None:
            assert not torch.equal(prev["out"], g["out"]), step
            assert not torch.equal(prev["sel"], g["sel"]), step
        prev = {key: g[key].clone() for key in ("sel", "out")}
    graph.close()
