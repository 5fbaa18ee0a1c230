"""moe_forward_noalloc (the layer on the library's fixed device scratch, for callers that cannot
allocate) against moe_forward (the same kernels on a caller workspace): bitwise-equal outputs on two
calls in a row, the second with a smaller input, and MOE_ETOOLARGE beyond the scratch."""

import numpy as np
import pytest
import torch

import routing_token_permute_amd as moe
from gpu_util import layer_tensors, require_gpu
from workloads import make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _compare(dev, w):
    t = layer_tensors(w, dev)
    ref = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"], routing_out=True)
    # Poisoned outputs: every element must be written by the call.
    y = torch.full((w.n, w.H), float("nan"), dtype=t["x"].dtype, device=dev)
    got = moe.moe_forward_noalloc(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"], y=y,
                                  routing_out=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("y", "logits", "topk_ids", "topk_w", "counts"), ref, got):
        assert torch.equal(_bits(a), _bits(b)), f"n={w.n}: {name} differs from moe_forward"
    print(f"[noalloc n={w.n} H={w.H} I={w.I} E={w.E} K={w.K} {w.dtype}] bitwise equal to moe_forward", flush=True)


def test_noalloc_matches_forward_twice_shrinking(dev):
    lib = moe.load_library()
    cap = lib.moe_forward_noalloc_max_bytes()
    big = make_layer(1024, 2048, 1024, 64, 8, dtype="bf16", seed=11)  # OLMoE layer shape, 1024 tokens
    assert lib.moe_forward_workspace_size(big.n, big.H, big.I, big.E, big.K, 1) <= cap
    _compare(dev, big)
    _compare(dev, make_layer(32, 2048, 1024, 64, 8, dtype="bf16", seed=12))  # decode batch, smaller
    _compare(dev, make_layer(300, 128, 128, 8, 8, dtype="bf16", renorm=True, seed=13))
    _compare(dev, make_layer(64, 128, 64, 8, 2, dtype="f32", renorm=True, seed=14))


def test_noalloc_rejects_beyond_scratch(dev):
    lib = moe.load_library()
    cap = lib.moe_forward_noalloc_max_bytes()
    n = 2048
    assert lib.moe_forward_workspace_size(n, 2048, 1024, 64, 8, 1) > cap
    w = make_layer(n, 2048, 1024, 64, 8, dtype="bf16", seed=3)
    t = layer_tensors(w, dev)
    with pytest.raises(moe.MoEError, match="MOE_ETOOLARGE"):
        moe.moe_forward_noalloc(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm)
    # After the refusal the scratch still serves a call that fits.
    _compare(dev, make_layer(48, 2048, 1024, 64, 8, dtype="bf16", seed=15))
