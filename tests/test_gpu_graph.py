"""The layer captured in a HIP graph: every replay equals the eager call bit for bit.

No call of the library records a memset or allocates; moe_backward forks its
side branches onto a second stream with events, which graph capture follows.
Each graph is replayed several times with the program's own eager work and
synchronisations in between, and every replay is checked.
"""

import numpy as np
import pytest
import torch

import routing_token_permute_amd as moe
from gpu_util import dev_tensor, layer_tensors, require_gpu
from workloads import make_config, make_layer, random_bf16_matrix

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _replays(graph, outs, expected, eager_work):
    for r in range(3):
        eager_work()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, o in outs.items():
            assert torch.equal(_bits(o), _bits(expected[name])), f"replay {r}: {name} differs from the eager call"


@pytest.mark.parametrize("name", ["decode_bf16", "olmoe_bf16"])
def test_packed_forward_graph_replays_match_eager(dev, name):
    """moe_forward_packed (GEMM1 from the ids at decode, the gathered GEMM1 at the OLMoE shape) in a graph."""
    w = make_config(name)
    t = layer_tensors(w, dev)
    W13p, W2p = moe.moe_pack_w13(t["W13"]), moe.moe_pack_w2(t["W2"])
    y_eager = moe.moe_forward_packed(t["x"], t["W_gate"], W13p, W2p, w.K, w.renorm)
    ws = torch.empty(moe.moe_forward_workspace_size(w.n, w.H, w.I, w.E, w.K, t["x"].dtype), dtype=torch.uint8,
                     device=dev)
    y = torch.empty_like(y_eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        moe.moe_forward_packed(t["x"], t["W_gate"], W13p, W2p, w.K, w.renorm, y=y, ws=ws)  # warm-up on s
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        moe.moe_forward_packed(t["x"], t["W_gate"], W13p, W2p, w.K, w.renorm, y=y, ws=ws)
    junk = torch.empty_like(y_eager)
    _replays(g, {"y": y}, {"y": y_eager},
             lambda: moe.moe_forward_packed(t["x"], t["W_gate"], W13p, W2p, w.K, w.renorm, y=junk))


@pytest.mark.parametrize("name", ["decode_bf16", "tiny_f32"])
def test_forward_graph_replays_match_eager(dev, name):
    w = make_config(name)
    t = layer_tensors(w, dev)
    y_eager = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm)
    ws = torch.empty(moe.moe_forward_workspace_size(w.n, w.H, w.I, w.E, w.K, t["x"].dtype), dtype=torch.uint8,
                     device=dev)
    y = torch.empty_like(y_eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, y=y, ws=ws)  # warm-up on s
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, y=y, ws=ws)
    junk = torch.empty_like(y_eager)
    _replays(g, {"y": y}, {"y": y_eager},
             lambda: moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, y=junk))


def test_backward_graph_replays_match_eager(dev):
    w = make_layer(300, 128, 128, 8, 4, renorm=True, seed=11)
    t = layer_tensors(w, dev)
    dy = dev_tensor(random_bf16_matrix(np.random.default_rng(3), (w.n, w.H))[0], "bf16", dev)
    _, saved = moe.moe_forward_train(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm)
    g_eager = moe.moe_backward(dy, t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, saved)
    ws = torch.empty(moe.moe_backward_workspace_size(w.n, w.H, w.I, w.E, w.K, torch.bfloat16), dtype=torch.uint8,
                     device=dev)
    grads = {k: torch.empty_like(v) for k, v in g_eager.items()}
    torch.cuda.synchronize()
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        moe.moe_backward(dy, t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, saved, grads=grads, ws=ws)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    for v in grads.values():
        v.zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_backward(dy, t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, saved, grads=grads, ws=ws)
    _replays(g, grads, g_eager,
             lambda: moe.moe_backward(dy, t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, saved))
