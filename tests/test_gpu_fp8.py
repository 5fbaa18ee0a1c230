"""Parity of the FP8-weight calls against the fp64 CPU oracle (oracle/fp8.py).

The quantizer's codes and scales must match the oracle's bit for bit (both
take every rounding decision in fp32: one division for the scale, one per
weight for the quotient, then the nearest E4M3 value with ties to even). The
GEMMs and the layer are then compared with the oracle's layer on its own
dequantized weights under the bf16 bounds of the forward tests: the FP8
weights are exact in bf16, so the device adds only its fp32 accumulation and
the bf16 roundings of h and y.
"""

import numpy as np
import pytest
import torch

import oracle
import routing_token_permute_amd as moe
from gpu_util import assert_close, dev_tensor, errors, layer_tensors, require_gpu, to_f64
from oracle import fp8 as of8
from oracle import moe_oracle as om
from workloads import make_config, make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _quantize_both(w_f32, w_dev, experts=None):
    """Device codes/scales for the whole stack; oracle codes/scales for `experts` (all by default);
    asserts they agree bit for bit on those experts."""
    codes, scales = moe.moe_quantize_fp8(w_dev)
    torch.cuda.synchronize()
    idx = np.arange(w_f32.shape[0]) if experts is None else np.asarray(experts)
    c_ref, s_ref = of8.quantize_columns(w_f32[idx])
    c_dev = codes.cpu().numpy()[idx]
    s_dev = scales.cpu().numpy()[idx]
    assert (s_dev.view(np.uint32) == s_ref.view(np.uint32)).all(), "scales differ"
    bad = int((c_dev != c_ref).sum())
    assert bad == 0, f"{bad} codes differ"
    return codes, scales


@pytest.mark.parametrize("E,Kd,N,dtype", [(4, 64, 128, "bf16"), (3, 128, 64, "f32"), (2, 192, 260, "bf16"),
                                          (64, 2048, 2048, "bf16")])
def test_quantize_fp8_matches_oracle(dev, E, Kd, N, dtype):
    rng = np.random.default_rng(E * Kd + N)
    W = (rng.standard_normal((E, Kd, N)) * 0.02).astype(np.float32)
    W[0, :, 1] = 0.0  # an all-zero column: scale 1, codes 0
    W[0, 3, 2] = 1e-9  # tiny values next to a large one round to zero or a subnormal
    W[0, 5, 2] = 0.5
    W[-1, :, -1] = np.float32(2.0) ** rng.integers(-12, 4, Kd)  # powers of two: exact codes after scaling
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits, bf16_bits_to_f32

        bits = f32_to_bf16_bits(W)
        W = bf16_bits_to_f32(bits)
        Wd = dev_tensor(bits, "bf16", dev)
    else:
        Wd = dev_tensor(W, "f32", dev)
    experts = None if E <= 4 else [0, 17, E - 1]  # full-size stack: the oracle checks three experts
    _quantize_both(W, Wd, experts)


_ORACLE_Q = {}  # oracle codes/scales of the named full-size layers (about 30 s of numpy each)


def _fp8_layer(w, dev):
    t = layer_tensors(w, dev)
    experts = None if w.E <= 16 else [0, w.E // 2, w.E - 1]
    q13, s13 = _quantize_both(w.W13_f32, t["W13"], experts)
    q2, s2 = _quantize_both(w.W2_f32, t["W2"], experts)
    key = w.name if w.name != "custom" else None
    if key is None or key not in _ORACLE_Q:
        ref = of8.quantize_columns(w.W13_f32) + of8.quantize_columns(w.W2_f32)
        if key is not None:
            _ORACLE_Q[key] = ref
    else:
        ref = _ORACLE_Q[key]
    return t, (q13, s13, q2, s2), ref


@pytest.mark.parametrize("n,H,I,E,K", [(300, 128, 64, 8, 2), (1000, 256, 192, 16, 4), (32, 2048, 1024, 64, 8),
                                       (4096, 2048, 1024, 64, 8), (5, 64, 64, 4, 2)])
def test_fp8_expert_gemms(dev, n, H, I, E, K):  # noqa: E741
    """GEMM1 (+SwiGLU, rows gathered) and GEMM2 with FP8 weights, each alone. The full-size cases use the
    decode and OLMoE layers of the benchmark."""
    if H == 2048:
        w = make_config("decode_bf16" if n == 32 else "olmoe_bf16")
    else:
        w = make_layer(n, H, I, E, K, seed=n + H)
    rng = np.random.default_rng(n)
    L = rng.standard_normal((n, E)).astype(np.float32)
    e_top, _, _ = oracle.route_from_logits(L, K, renorm=False)
    offsets = oracle.offsets_from_counts(oracle.expert_counts(e_top, E))
    perm, _ = oracle.permutation(e_top, E)
    t, (q13, s13, q2, s2), (c13, r13, c2, r2) = _fp8_layer(w, dev)
    off_d = torch.from_numpy(offsets.astype(np.int32)).to(dev)
    perm_d = torch.from_numpy(perm.astype(np.int32)).to(dev)
    h = moe.moe_expert_w13_swiglu_gather_fp8(t["x"], perm_d, K, off_d, q13, s13)
    torch.cuda.synchronize()
    W13d = of8.dequantize_columns(c13, r13)
    ref_h = om.grouped_gate_up(w.x_f32[perm // K], offsets, W13d)
    assert_close(to_f64(h), ref_h, "bf16", f"fp8 gate_up n={n} E={E}", intermediate=True)
    # GEMM2 on the device's h (a bf16 input to both sides), FP8 W2.
    Y = moe.moe_expert_w2_fp8(h, off_d, q2, s2)
    torch.cuda.synchronize()
    W2d = of8.dequantize_columns(c2, r2)
    ref_Y = om.grouped_down(to_f64(h), offsets, W2d)
    assert_close(to_f64(Y), ref_Y, "bf16", f"fp8 down n={n} E={E}")


def _forward_fp8_parity(dev, w, what):
    t, (q13, s13, q2, s2), (c13, r13, c2, r2) = _fp8_layer(w, dev)
    y, logits, ids, wts, counts = moe.moe_forward_fp8(t["x"], t["W_gate"], q13, s13, q2, s2, w.K, w.renorm,
                                                      bias=t["bias"], routing_out=True)
    torch.cuda.synchronize()
    # Router logits against the fp64 product, then both sides route from the
    # device's fp32 logits, so every row is compared.
    ref_logits = oracle.router_logits(w.x_f32, w.W_gate_f32, w.bias)
    L = logits.cpu().numpy()
    fin = np.isfinite(ref_logits)
    assert (np.isfinite(L) == fin).all()
    ma, rf = errors(L[fin].astype(np.float64), ref_logits[fin])
    assert rf <= 1e-5 and ma <= 1e-4
    ref = of8.forward_fp8(w.x_f32, w.W_gate_f32, c13, r13, c2, r2, w.K, w.renorm, bias=w.bias,
                          routing_logits_f32=L)
    print(f"[{what}] rows at a top-K near-tie, all compared: {int((oracle.topk_margin(L, w.K) <= 1e-4).sum())}",
          flush=True)
    assert (ids.cpu().numpy() == ref["e_top"]).all()
    assert (counts.cpu().numpy() == ref["counts"]).all()
    assert_close(to_f64(y), ref["y"], "bf16", what)
    # FP8 weights move the output by about the quantisation error of the weights, not more.
    plain = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, w.K, w.renorm, bias=w.bias,
                           routing_logits_f32=L)
    rel = np.linalg.norm(ref["y"] - plain["y"]) / np.linalg.norm(plain["y"])
    print(f"[{what}] FP8 vs bf16 weights: rel_frob={rel:.3e}", flush=True)
    assert rel < 0.1


@pytest.mark.parametrize("name", ["decode_bf16", "olmoe_bf16", "olmoe_skewed_bf16", "tiny_bf16"])
def test_forward_fp8_configs(dev, name):
    w = make_config(name) if name != "tiny_bf16" else make_layer(64, 128, 64, 8, 2, renorm=True, seed=2)
    _forward_fp8_parity(dev, w, f"forward fp8 {name}")


@pytest.mark.parametrize("n,H,I,E,K,renorm", [(1, 64, 64, 8, 2, False), (257, 128, 64, 1, 1, False),
                                              (45, 256, 192, 32, 4, True), (300, 128, 64, 256, 64, True)])
def test_forward_fp8_small_shapes(dev, n, H, I, E, K, renorm):  # noqa: E741
    w = make_layer(n, H, I, E, K, renorm=renorm, seed=n + I)
    _forward_fp8_parity(dev, w, f"forward fp8 n={n} E={E} K={K}")


@pytest.mark.parametrize("n", [256, 16])
def test_forward_fp8_wide_layer(dev, n):
    """FP8 weights on a wide layer (H = 7168, I = 2048): the gathered GEMM1 (n = 256) and the decode GEMM1
    from the ids (n = 16) over 7168-deep columns, GEMM2 over 28 column blocks; every row against the oracle.
    Weights ~ N(0, 0.01^2), as in the bf16 wide-layer test."""
    w = make_layer(n, 7168, 2048, 8, 2, seed=7 + n, w_std=0.01)
    _forward_fp8_parity(dev, w, f"forward fp8 wide n={n}")


def test_fp8_rejects_fp32_activations(dev):
    w = make_layer(8, 64, 64, 4, 2, dtype="f32", seed=1)
    t = layer_tensors(w, dev)
    q13 = torch.zeros((4, 128, 64), dtype=torch.uint8, device=dev)
    s13 = torch.ones((4, 128), dtype=torch.float32, device=dev)
    q2 = torch.zeros((4, 64, 64), dtype=torch.uint8, device=dev)
    s2 = torch.ones((4, 64), dtype=torch.float32, device=dev)
    with pytest.raises(moe.MoEError):
        moe.moe_forward_fp8(t["x"], t["W_gate"], q13, s13, q2, s2, 2, False)
