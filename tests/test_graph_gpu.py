"""The layer captured in a HIP graph (through torch.cuda.graph, on torch's
current stream) replays bit-identically to eager execution, replay after
replay, with eager work and synchronisations in between (the plain forward
and the forward that reroutes over-capacity pairs)."""
import pytest
import torch

import sparse_mixture_experts_04_amd as moe
import workloads
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,d,E,k,F,cap,reroute", [(300, 256, 8, 2, 384, -1, False), (8, 1024, 64, 2, 256, -1, False),
                                                   (500, 256, 16, 4, 256, 100, False),
                                                   (2500, 256, 16, 4, 256, 500, True),
                                                   # the skewed layer's kernels: K-sliced router (gate too large
                                                   # for LDS), two-launch dispatch, gathered up-projection
                                                   (4100, 4096, 64, 2, 128, -1, False)])
def test_graph_replay_matches_eager(T, d, E, k, F, cap, reroute):
    inp = workloads.random_case(3, T, d, E, k, F, "bf16", cap, 0.3, w_scale=0.05)
    cfg = moe.config(T, d, F, E, k, cap, "bf16")
    layer = moe.MoELayer(cfg, to_dev(inp.Wg, "bf16"), to_dev(inp.W1, "bf16"), to_dev(inp.W2, "bf16"),
                         to_dev(inp.bias, "f32"), reroute=reroute)
    X = to_dev(inp.X, "bf16")
    X2 = torch.randn_like(X)
    ref = layer.forward(X).clone()
    ref_ids = layer.buf.topk_ids.clone()
    ref2 = layer.forward(X2).clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(X)
    for rep in range(4):
        layer.buf.out.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.buf.out, ref), f"replay {rep} differs from eager"
        assert torch.equal(layer.buf.topk_ids, ref_ids)
        # eager work with other inputs between replays
        out2 = layer.forward(X2)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref2)
