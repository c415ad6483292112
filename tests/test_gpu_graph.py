"""psa_fwd and psa_bwd inside a captured HIP graph: both only launch kernels on the
caller's stream (no allocation, no copy, no wait), so a captured forward + backward
replays to the same bits as the eager calls.  The graph is replayed several times
with eager work and synchronisations between the replays, and every replay is
checked."""
import numpy as np
import pytest
import torch

from shared_prefix_block_amd import psa
from shared_prefix_block_amd import workloads as wl
from tests.gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("form", ["auto", "nodes"])
def test_graph_replay_matches_eager(form):
    need_gpu()
    lay = wl.tokens_layout([(300, [120, 77, 0]), (64, [200])], pad_multiple=128)
    q, k, v, do = (x.cuda() for x in wl.make_tensors(lay.T, 4, 2, 128, "bf16", 1.0, 21))
    m = psa.layout_tile_map(lay, "cuda", dtype=torch.bfloat16, d=128, form=form)
    say(f"graph replay: T={lay.T} form={m.info['form']}")
    o = torch.empty_like(q)
    lse = torch.empty(4, lay.T, device="cuda")
    grads = (torch.empty(q.shape, device="cuda"), torch.empty(k.shape, device="cuda"),
             torch.empty(v.shape, device="cuda"))
    ws = torch.empty(psa.bwd_workspace_size(m, q, k), dtype=torch.uint8, device="cuda")

    def step():
        psa.fwd(m, q, k, v, out=o, lse=lse)
        psa.bwd(m, q, k, v, o, lse, do, workspace=ws, out=grads)

    step()
    torch.cuda.synchronize()
    want = [x.clone() for x in (o, lse) + grads]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the graph's stream, as capture wants
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for x in (o, lse) + grads:
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "lse", "dq", "dk", "dv"), (o, lse) + grads, want):
            assert torch.equal(got, ref), (rep, name)
        _ = (q.float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
