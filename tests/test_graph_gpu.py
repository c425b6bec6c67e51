"""Append and decode captured in a graph (torch.cuda.graph around the
library's C ABI calls) and replayed several times, with eager work between
the replays (new queries written, the output poisoned, a synchronisation):
every replay matches an eager call on the same inputs bit for bit, and the
first, on the seeded inputs, matches the oracle.  The library allocates
nothing and synchronises nothing inside a call, so the capture holds only
its kernels."""
import numpy as np
import pytest
import torch

from paged_kv_cache_405_amd import binding as B
from paged_kv_cache_405_amd import workloads as W
from tests.pa_harness import assert_close, compare, log, oracle_step, upload

pytestmark = pytest.mark.gpu

CTXS = [1, 17, 300, 1000, 2049, 64, 700, 5]
SHAPES = {
    "mha_f16": ("f16", 8, 8),
    "gqa_bf16": ("bf16", 64, 8),
}


@pytest.mark.parametrize("pt", [B.PA_PARTITION_AUTO, B.PA_PARTITION_SINGLE, B.PA_PARTITION_BALANCED, 256])
@pytest.mark.parametrize("shape", list(SHAPES))
def test_graph_replays_match_eager(shape, pt):
    dtype, Hq, Hkv = SHAPES[shape]
    w = W.custom(f"graph_{shape}", dtype, CTXS, Hq, Hkv, 128, 16, seed=40 + Hq, append=True, table_pad=1)
    log(f"[gpu] {w.name} pt={pt}")
    g = upload(w)
    S, _, D = g.q.shape
    code = {"f16": B.PA_F16, "bf16": B.PA_BF16}[dtype]
    nbytes = max(16, B.pa_decode_workspace_bytes(S, Hq, Hkv, D, 16, w.max_blocks_per_seq, code, pt))
    ws_graph = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws_eager = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    qbuf = g.q.clone()
    out_graph = torch.empty_like(qbuf)
    out_eager = torch.empty_like(qbuf)

    def step(out, ws):
        B.pa_reshape_and_cache(g.new_k, g.new_v, g.k_cache, g.v_cache, g.slots, layout=g.layout)
        B.pa_decode_ex(out, qbuf, g.k_cache, g.v_cache, g.tables, g.ctx, w.scale, layout=g.layout,
                       partition_tokens=pt, workspace=ws)

    step(out_eager, ws_eager)          # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out_graph, ws_graph)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(44)
    for i in range(4):
        if i > 0:
            qbuf.copy_(torch.randn(tuple(qbuf.shape), generator=gen, device="cuda", dtype=qbuf.dtype))
        out_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(out_eager, ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(out_graph, out_eager), f"replay {i} differs from the eager call"
        if i == 0:
            assert_close(compare(out_graph, oracle_step(w), dtype), dtype, f"{w.name} pt={pt} replay 0")
