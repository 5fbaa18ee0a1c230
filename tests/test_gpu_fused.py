"""moe_forward_persistent (GEMM1 + SwiGLU and GEMM2 in one persistent kernel, the Mega MoE scheduling of
"大模型系统中的通算融合" §4.4) against moe_forward: bitwise-equal outputs (every output element is the same
sequence of fp32 operations), for several warm-up depths and ring-pool sizes, on balanced, skewed, decode
and ragged layers; the scheduler's flag word stays zero (no bounded wait ran out); and the layer against
the fp64 oracle, routed from the device's fp32 logits."""

import numpy as np
import pytest
import torch

import oracle
import routing_token_permute_amd as moe
from gpu_util import assert_close, errors, layer_tensors, require_gpu, to_f64
from workloads import make_config, make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _run(dev, w, t, warm, pool):
    lib = moe.load_library()
    nbytes = lib.moe_forward_persistent_workspace_size(w.n, w.H, w.I, w.E, w.K, pool)
    ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device=dev)  # the counters must be cleared by the call
    y = torch.full((w.n, w.H), float("nan"), dtype=torch.bfloat16, device=dev)
    out = moe.moe_forward_persistent(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"],
                                     warmup_row_tiles=warm, pool_row_tiles=pool, y=y, ws=ws, routing_out=True)
    torch.cuda.synchronize()
    flag = int(ws[nbytes - 4:].view(torch.int32).item())
    assert flag == 0, "a bounded wait of the persistent scheduler ran out"
    return out


CASES = [("olmoe_bf16", 4, 0), ("olmoe_bf16", 4, 8), ("olmoe_bf16", 1, 2), ("olmoe_skewed_bf16", 4, 8),
         ("olmoe_skewed_bf16", 2, 3), ("decode_bf16", 4, 5), ("ragged", 3, 4), ("ragged", 1, 0), ("tiny_e", 2, 3)]


def _layer(name):
    if name == "ragged":  # experts of 0 .. a few hundred rows, partial column blocks (I = 192, H = 320)
        return make_layer(700, 320, 192, 16, 4, dtype="bf16", seed=21)
    if name == "tiny_e":  # fewer row tiles than queues
        return make_layer(90, 128, 128, 4, 2, dtype="bf16", renorm=True, seed=22)
    return make_config(name)


@pytest.mark.parametrize("name,warm,pool", CASES)
def test_persistent_matches_forward_bitwise(dev, name, warm, pool):
    w = _layer(name)
    t = layer_tensors(w, dev)
    ref = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"], routing_out=True)
    got = _run(dev, w, t, warm, pool)
    for what, a, b in zip(("y", "logits", "topk_ids", "topk_w", "counts"), ref, got):
        a = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
        b = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
        assert torch.equal(a, b), f"{name} warm={warm} pool={pool}: {what} differs from moe_forward"
    print(f"[persistent {name} warm={warm} pool={pool}] bitwise equal to moe_forward", flush=True)


@pytest.mark.parametrize("name,warm,pool", [("olmoe_bf16", 4, 0), ("olmoe_skewed_bf16", 4, 8), ("ragged", 3, 4),
                                            ("decode_bf16", 4, 5)])
def test_persistent_packed_matches_forward_bitwise(dev, name, warm, pool):
    """The persistent kernel over packed weights: bit for bit moe_forward (and so moe_forward_packed)."""
    w = _layer(name)
    t = layer_tensors(w, dev)
    ref = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"], routing_out=True)
    W13p, W2p = moe.moe_pack_w13(t["W13"]), moe.moe_pack_w2(t["W2"])
    lib = moe.load_library()
    nbytes = lib.moe_forward_persistent_workspace_size(w.n, w.H, w.I, w.E, w.K, pool)
    ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device=dev)
    got = moe.moe_forward_persistent_packed(t["x"], t["W_gate"], W13p, W2p, w.K, w.renorm, bias=t["bias"],
                                            warmup_row_tiles=warm, pool_row_tiles=pool, ws=ws, routing_out=True)
    torch.cuda.synchronize()
    assert int(ws[nbytes - 4:].view(torch.int32).item()) == 0, "a bounded wait of the persistent scheduler ran out"
    for what, a, b in zip(("y", "logits", "topk_ids", "topk_w", "counts"), ref, got):
        a = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
        b = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
        assert torch.equal(a, b), f"{name} warm={warm} pool={pool}: {what} differs from moe_forward"


def test_persistent_against_oracle(dev):
    w = make_layer(600, 256, 128, 8, 2, dtype="bf16", seed=23)
    t = layer_tensors(w, dev)
    y, logits, ids, wts, counts = _run(dev, w, t, 2, 3)
    L = logits.cpu().numpy()
    ma, rf = errors(L.astype(np.float64), oracle.router_logits(w.x_f32, w.W_gate_f32, w.bias))
    assert rf <= 1e-5 and ma <= 1e-4
    ref = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, w.K, w.renorm, bias=w.bias,
                         routing_logits_f32=L)
    assert (ids.cpu().numpy() == ref["e_top"]).all()
    assert (counts.cpu().numpy() == ref["counts"]).all()
    assert_close(to_f64(y), ref["y"], "bf16", "persistent forward")


def test_persistent_repeated_calls_deterministic(dev):
    w = make_config("olmoe_bf16")
    t = layer_tensors(w, dev)
    a = _run(dev, w, t, 4, 8)[0]
    b = _run(dev, w, t, 4, 8)[0]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_persistent_rejects_bad_arguments(dev):
    w = make_layer(64, 128, 64, 8, 2, dtype="f32", seed=24)
    t = layer_tensors(w, dev)
    with pytest.raises(moe.MoEError):  # bf16 only
        moe.moe_forward_persistent(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm)
