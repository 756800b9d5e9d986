"""The path on a non-default stream and inside a captured HIP graph.

Every hot entry point only enqueues kernels on the caller's stream, so the
whole path runs on a side stream and can be captured once and replayed: the
fused path (means of Q, permute and pool K, permute V, predict, attend with
raster-order Q and O), the five-pass path (permute Q too, attend, unpermute)
and the FP8 form.  The replays run with eager launches of the same path and host
synchronisations between them, and each replay's output must equal the eager
result bit for bit.
"""
import sys

import pytest
import torch

from image_diffusion_dits_amd import configs, inputs, rf

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _five_pass(q, k, v, plan, s):
    return rf.sparse_attention(q, k, v, plan, s, fused=False)


CASES = [("bf16-fused", rf.sparse_attention), ("bf16-five-pass", _five_pass),
         ("fp8", rf.sparse_attention_fp8)]


@pytest.mark.parametrize("name,path", CASES, ids=[c[0] for c in CASES])
def test_side_stream_and_graph_replays(name, path):
    cfg = configs.VIDEO720
    s = cfg.sparsity[0]
    say(f"[graph] {name} path, {cfg.name}, 4 heads: side stream, capture, 3 replays")
    q, k, v = inputs.make_qkv(cfg, "cuda", H=4)
    plan = rf.Plan(cfg.layout)
    o_ref, kept_ref = path(q, k, v, plan, s)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o_side, kept_side = path(q, k, v, plan, s)      # also the warm-up before capture
    side.synchronize()
    assert torch.equal(o_side, o_ref) and torch.equal(kept_side, kept_ref)
    torch.cuda.current_stream().wait_stream(side)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o_g, kept_g = path(q, k, v, plan, s)
    for rep in range(3):
        o_g.zero_()                                     # the replay must rewrite everything
        kept_g.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_ref), f"replay {rep}: output"
        assert torch.equal(kept_g, kept_ref), f"replay {rep}: kept tiles"
        o_e, _ = path(q, k, v, plan, s)                 # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o_e, o_ref)
    del graph
    plan.close()
