"""The decode inside a captured HIP graph (through torch.cuda.graph): every
launch of a step is an ordinary kernel node -- no allocation, no host
synchronisation, no memset -- so a replayed step gives the eager result bit
for bit.  The graph is replayed several times with eager decodes and host
synchronisations in between, and every replay is checked."""

import numpy as np
import pytest
import torch

from mla_inputs import make_workload, to_torch
from gpu_helpers import make_decoder, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["paged_b32_small", "fp8_b64_small", "mtp2_b128_small", "sparse_topk2048_b64_small"])
def test_graph_replays_match_eager(name):
    w = make_workload(name)
    s = w.spec
    dev = torch.device("cuda:0")
    t = to_torch(w, dev)
    dec = make_decoder(w)
    sparse = w.indices is not None
    ws = dec.alloc_sparse_workspace(s.batch, s.topk) if sparse else dec.alloc_workspace(s.batch)
    shape, lshape = (s.batch, s.s_q, s.n_h, s.d_c), (s.batch, s.s_q, s.n_h)

    def step(out, lse):
        if sparse:
            dec.run_sparse(t["q"], t["kv"], t["block_table"], t["seq_lens"], t["indices"], out, lse, workspace=ws)
        else:
            dec.run(t["q"], t["kv"], t["block_table"], t["seq_lens"], out, lse, workspace=ws)

    say(f"graph capture {name}")
    ref_o = torch.empty(shape, dtype=torch.float32, device=dev)
    ref_l = torch.empty(lshape, dtype=torch.float32, device=dev)
    step(ref_o, ref_l)
    torch.cuda.synchronize()
    out = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full(lshape, float("nan"), dtype=torch.float32, device=dev)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            step(out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    other_o = torch.empty_like(ref_o)
    other_l = torch.empty_like(ref_l)
    for r in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {r}")
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {r} differs from the eager step"
        step(other_o, other_l)             # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other_o, ref_o)
