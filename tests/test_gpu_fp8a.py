"""Parity of the FP8-activation calls against the fp64 CPU oracle (oracle/fp8.py).

Per-token codes and scales, and the padded FP8 receive buffer (group starts,
row order, codes, scales, perm and inv), must match the oracle's bit for bit:
both sides take each rounding decision in fp32 (one division for a row's
scale, one per element for the quotient, then the nearest E4M3 value with
ties to even) and place rows by the same integer rules. The FP8 x FP8 GEMM and
the layer are compared with the oracle on its own dequantized activations and
weights under the bf16 bounds of the forward tests: the FP8 operands are exact
products of codes and scales, so the device adds only its fp32 accumulation,
the scale multiplications and the bf16 roundings of h and y. Routing is taken
from the device's fp32 logits on both sides (held to the fp64 router product
first), so every row is compared.
"""

import numpy as np
import pytest
import torch

import oracle
import routing_token_permute_amd as moe
from gpu_util import assert_close, dev_tensor, errors, layer_tensors, require_gpu, to_f64
from oracle import fp8 as of8
from oracle import moe_oracle as om
from workloads import make_config, make_layer, random_bf16_matrix

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("n,H,dtype", [(7, 128, "bf16"), (300, 2048, "bf16"), (33, 192, "f32"), (4096, 2048, "bf16"),
                                     (9, 4096, "bf16"), (5, 2184, "f32"), (40, 1024, "bf16")])
def test_quantize_rows_fp8_bit_exact(dev, n, H, dtype):
    rng = np.random.default_rng(n + H)
    if dtype == "bf16":
        xb, xf = random_bf16_matrix(rng, (n, H))
        xf = xf * 1.0
        xb = xb.copy()
        xb[0] = 0  # an all-zero row: scale 1, codes 0
        xf[0] = 0
        x = dev_tensor(xb, "bf16", dev)
    else:
        xf = (rng.standard_normal((n, H)) * rng.uniform(1e-3, 10, (n, 1))).astype(np.float32)
        xf[0] = 0
        x = dev_tensor(xf, "f32", dev)
    codes, scales = moe.moe_quantize_rows_fp8(x)
    torch.cuda.synchronize()
    c_ref, s_ref = of8.quantize_rows(xf.astype(np.float32))
    assert (scales.cpu().numpy().view(np.uint32) == s_ref.view(np.uint32)).all(), "scales differ"
    bad = int((codes.cpu().numpy() != c_ref).sum())
    assert bad == 0, f"{bad} codes differ"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_rows_fp8_ties_subnormals_and_signed_zero(dev, dtype):
    """Rows whose amax is 448 (scale exactly 1) holding every midpoint between consecutive E4M3 values, normal
    and subnormal, both signs, and tiny values that round to zero from either side: the codes must be the
    oracle's bit for bit (ties to the even mantissa, no negative-zero code)."""
    t = of8.e4m3_decode_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    vals = np.concatenate([[448.0], mids, -mids, t, -t[1:], [2.0**-11, -2.0**-11, -2.0**-12, 0.0, -0.0]])
    H = 512
    row = np.zeros(H)
    row[:vals.size] = vals
    x = np.stack([row, np.roll(row, 7), -row]).astype(np.float32)
    if dtype == "bf16":
        bits = x.view(np.uint32)
        assert ((bits & 0xFFFF) == 0).all()  # every value is exact in bf16
        xd = torch.from_numpy((bits >> 16).astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        xd = torch.from_numpy(x).to(dev)
    codes, scales = moe.moe_quantize_rows_fp8(xd)
    torch.cuda.synchronize()
    c_ref, s_ref = of8.quantize_rows(x)
    assert (scales.cpu().numpy() == 1.0).all() and (s_ref == 1.0).all()
    got = codes.cpu().numpy()
    bad = np.argwhere(got != c_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, e.g. value {x[tuple(bad[0])]}: {got[tuple(bad[0])]:#x} vs " \
                          f"{c_ref[tuple(bad[0])]:#x}"


def _route_and_dispatch(dev, w, t):
    logits, ids, wts = moe.moe_route(t["x"], t["W_gate"], t["bias"], w.K, w.renorm)
    meta = moe.moe_permute(ids, None, w.E)
    codes_tok, s_tok = moe.moe_quantize_rows_fp8(t["x"])
    d = moe.moe_dispatch_fp8(meta, codes_tok, s_tok, w.K)
    torch.cuda.synchronize()
    return logits, ids, wts, meta, d


@pytest.mark.parametrize("n,H,E,K", [(70, 128, 8, 3), (300, 256, 16, 4), (4096, 2048, 64, 8), (1, 128, 4, 1),
                                     (513, 128, 256, 8)])
def test_dispatch_fp8_receive_buffer_bit_exact(dev, n, H, E, K):
    w = make_layer(n, H, 64, E, K, dtype="bf16", seed=n + E) if H != 2048 else make_config("olmoe_bf16")
    t = layer_tensors(w, dev)
    logits, ids, wts, meta, d = _route_and_dispatch(dev, w, t)
    ref = of8.dispatch_fp8(w.x_f32, ids.cpu().numpy(), w.E)
    P = ref["offsets"]
    R = int(P[-1])
    assert d["x_q"].shape[0] == moe.moe_fp8_padded_rows(w.n, w.E, w.K) >= R
    np.testing.assert_array_equal(d["offsets_padded"].cpu().numpy(), P)
    np.testing.assert_array_equal(d["perm_padded"].cpu().numpy()[:R], ref["perm"])
    np.testing.assert_array_equal(d["inv_padded"].cpu().numpy(), ref["inv"])
    assert (d["x_scale"].cpu().numpy()[:R].view(np.uint32) == ref["scales"].view(np.uint32)).all()
    bad = int((d["x_q"].cpu().numpy()[:R] != ref["codes"]).sum())
    assert bad == 0, f"{bad} receive-buffer codes differ"


_ORACLE_Q = {}  # oracle codes/scales of the named full-size layers (tens of seconds of numpy each)


def _fp8_weights(w, t):
    """Device codes/scales of W13 and W2 (checked bit-exact against the oracle's), and the oracle's own
    codes/scales, which are what the oracle side of every comparison uses."""
    q13, s13 = moe.moe_quantize_fp8(t["W13"])
    q2, s2 = moe.moe_quantize_fp8(t["W2"])
    torch.cuda.synchronize()
    key = w.name if w.name != "custom" else None
    if key is None or key not in _ORACLE_Q:
        ref = of8.quantize_columns(w.W13_f32) + of8.quantize_columns(w.W2_f32)
        if key is not None:
            _ORACLE_Q[key] = ref
    else:
        ref = _ORACLE_Q[key]
    c13, r13, c2, r2 = ref
    for dv, rv in ((q13, c13), (s13, r13), (q2, c2), (s2, r2)):
        a = dv.cpu().numpy()
        assert (a.view(np.uint8) == rv.view(np.uint8)).all() if a.dtype == np.uint8 else \
            (a.view(np.uint32) == rv.view(np.uint32)).all()
    return (q13, s13, q2, s2), ref


@pytest.mark.parametrize("n,H,I,E,K", [(300, 128, 64, 8, 2), (1000, 256, 192, 16, 4), (32, 2048, 1024, 64, 8),
                                       (4096, 2048, 1024, 64, 8), (5, 128, 128, 4, 2)])
def test_w13_swiglu_fp8a(dev, n, H, I, E, K):  # noqa: E741
    """GEMM1 + SwiGLU on the receive buffer: every real row against the oracle on the dequantized rows and
    weights; padding rows exactly zero."""
    w = make_layer(n, H, I, E, K, dtype="bf16", seed=2 * n + I) if H != 2048 else make_config(
        "decode_bf16" if n == 32 else "olmoe_bf16")
    t = layer_tensors(w, dev)
    logits, ids, wts, meta, d = _route_and_dispatch(dev, w, t)
    (q13, s13, q2, s2), (c13, r13, c2, r2) = _fp8_weights(w, t)
    h = moe.moe_expert_w13_swiglu_fp8a(d["x_q"], d["x_scale"], d["offsets_padded"], q13, s13)
    torch.cuda.synchronize()
    # The oracle's own receive buffer (on the device's routing, from its fp32 logits) and weight codes.
    rd = of8.dispatch_fp8(w.x_f32, ids.cpu().numpy(), w.E)
    P = rd["offsets"]
    R = int(P[-1])
    np.testing.assert_array_equal(d["offsets_padded"].cpu().numpy(), P)
    ref = om.grouped_gate_up(of8.dequantize_rows(rd["codes"], rd["scales"]), P, of8.dequantize_columns(c13, r13))
    got = to_f64(h[:R])
    real = rd["perm"] >= 0
    assert (got[~real] == 0).all(), "padding rows must be zero"
    assert_close(got[real], ref[real], "bf16", f"fp8a gate_up n={n} E={E}", intermediate=True)
    # The in-place form (token rows read through perm, unpadded rows) computes every output the same way.
    codes_tok, s_tok = moe.moe_quantize_rows_fp8(t["x"])
    hg = moe.moe_expert_w13_swiglu_gather_fp8a(codes_tok, s_tok, meta["perm"], K, meta["offsets"], q13, s13)
    torch.cuda.synchronize()
    offs = meta["offsets"].cpu().numpy()
    rows_p = np.concatenate([np.arange(P[e], P[e] + offs[e + 1] - offs[e]) for e in range(E)]).astype(np.int64)
    assert torch.equal(hg.view(torch.int16).cpu(), h.view(torch.int16).cpu()[rows_p]), "gather form differs"


@pytest.mark.parametrize("R_real,E,H,I,skew", [(700, 8, 256, 128, False), (200, 16, 384, 256, True),
                                                (32768, 64, 2048, 1024, False), (248, 62, 2048, 1024, False)])
def test_w2_fp8a(dev, R_real, E, H, I, skew):  # noqa: E741
    """GEMM2 on FP8 activations alone: seeded h rows quantized per row by the oracle, in a receive buffer
    padded to 16-row groups (padding rows code 0, scale 0), against the oracle's dequantized product."""
    rng = np.random.default_rng(R_real + E)
    p = rng.dirichlet(np.full(E, 0.3 if skew else 5.0))
    counts = rng.multinomial(R_real, p)
    P = of8.padded_offsets(counts)
    R = int(P[-1])
    h = (rng.standard_normal((R, I)) * rng.uniform(0.1, 4.0, (R, 1))).astype(np.float32)
    codes, scales = of8.quantize_rows(h)
    real = np.zeros(R, bool)
    for e in range(E):
        real[P[e]:P[e] + counts[e]] = True
    codes[~real] = 0
    scales[~real] = 0
    W2 = (rng.standard_normal((E, I, H)) * 0.02).astype(np.float32)
    c2, r2 = of8.quantize_columns(W2)
    Y = moe.moe_expert_w2_fp8a(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev),
                               torch.from_numpy(P.astype(np.int32)).to(dev), torch.from_numpy(c2).to(dev),
                               torch.from_numpy(r2).to(dev))
    torch.cuda.synchronize()
    ref = om.grouped_down(of8.dequantize_rows(codes, scales), P, of8.dequantize_columns(c2, r2))
    got = to_f64(Y[:R])
    assert (got[~real] == 0).all(), "padding rows must be zero"
    assert_close(got[real], ref[real], "bf16", f"fp8a down R={R} E={E} H={H} I={I}", intermediate=True)


@pytest.mark.parametrize("name", ["decode_bf16", "olmoe_bf16", "olmoe_skewed_bf16", "small", "wide"])
def test_forward_fp8a_configs(dev, name):
    """The layer against the oracle, every row. Two integer decisions are compared given identical
    floating-point inputs, as the routing is: the ids from the device's fp32 logits (held to the fp64 router
    product), and the FP8 codes of h from the device's bf16 h (held to the oracle's fp64 h under the
    intermediate bounds): an h element within a bf16 ulp of an E4M3 midpoint may round either way, and a
    flipped code moves y by up to 2^-3 of that element's share. The rest of the layer is then held to the
    bf16 bounds: y against the oracle's product of those codes and the oracle's combine."""
    if name == "small":
        w = make_layer(200, 256, 128, 16, 4, dtype="bf16", renorm=True, seed=8)
    elif name == "wide":  # H = 7168, I = 2048: GEMM1 56 k-steps of 128 codes and 16 column blocks, GEMM2 28 blocks
        w = make_layer(256, 7168, 2048, 8, 2, dtype="bf16", seed=71, w_std=0.01)
    else:
        w = make_config(name)
    t = layer_tensors(w, dev)
    (q13, s13, q2, s2), (c13, r13, c2, r2) = _fp8_weights(w, t)
    y, logits, ids, wts, counts = moe.moe_forward_fp8a(t["x"], t["W_gate"], q13, s13, q2, s2, w.K, w.renorm,
                                                       bias=t["bias"], routing_out=True)
    # The same kernels stage by stage, for the device's h and its codes.
    meta = moe.moe_permute(ids, None, w.E)
    codes_tok, s_tok = moe.moe_quantize_rows_fp8(t["x"])
    h = moe.moe_expert_w13_swiglu_gather_fp8a(codes_tok, s_tok, meta["perm"], w.K, meta["offsets"], q13, s13)
    hq, hs = moe.moe_quantize_rows_fp8(h)
    torch.cuda.synchronize()
    ref_logits = oracle.router_logits(w.x_f32, w.W_gate_f32, w.bias)
    L = logits.cpu().numpy()
    fin = np.isfinite(ref_logits)
    ma, rf = errors(L[fin].astype(np.float64), ref_logits[fin])
    assert rf <= 1e-5 and ma <= 1e-4
    ref = of8.forward_fp8a(w.x_f32, w.W_gate_f32, c13, r13, c2, r2, w.K, w.renorm, bias=w.bias,
                           routing_logits_f32=L)
    assert (ids.cpu().numpy() == ref["e_top"]).all()
    assert (counts.cpu().numpy() == ref["counts"]).all()
    offsets, perm, inv = ref["offsets"], ref["perm"], ref["inv"]
    ct, st = of8.quantize_rows(w.x_f32)
    h_ref = om.grouped_gate_up(of8.dequantize_rows(ct, st)[perm // w.K], offsets, of8.dequantize_columns(c13, r13))
    h_dev = h.float().cpu().numpy()
    assert_close(h_dev.astype(np.float64), h_ref, "bf16", f"fp8a layer h {name}", intermediate=True)
    hc_ref, hs_ref = of8.quantize_rows(h_dev)
    assert (hs.cpu().numpy().view(np.uint32) == hs_ref.view(np.uint32)).all(), "h scales differ"
    assert int((hq.cpu().numpy() != hc_ref).sum()) == 0, "h codes differ"
    Y_ref = om.grouped_down(of8.dequantize_rows(hc_ref, hs_ref), offsets, of8.dequantize_columns(c2, r2))
    y_ref = om.combine_slot_order(Y_ref, inv, ref["w_top"], w.n, w.K)
    assert_close(to_f64(y), y_ref, "bf16", f"forward fp8a {name}")
    # Against the oracle's own layer (its h rounded from fp64): only the code flips of near-midpoint elements
    # separate the two, and FP8 activations move the output by about their quantization error, not more.
    rel = np.linalg.norm(to_f64(y) - ref["y"]) / np.linalg.norm(ref["y"])
    assert rel < 1e-2
    wq = of8.forward_fp8(w.x_f32, w.W_gate_f32, c13, r13, c2, r2, w.K, w.renorm, bias=w.bias, routing_logits_f32=L)
    rel = np.linalg.norm(ref["y"] - wq["y"]) / np.linalg.norm(wq["y"])
    print(f"[forward fp8a {name}] FP8 vs bf16 activations: rel_frob={rel:.3e}", flush=True)
    assert rel < 0.1


def test_forward_fp8a_deterministic_and_zero_tokens(dev):
    w = make_config("decode_bf16")
    t = layer_tensors(w, dev)
    q13, s13 = moe.moe_quantize_fp8(t["W13"])
    q2, s2 = moe.moe_quantize_fp8(t["W2"])
    y1 = moe.moe_forward_fp8a(t["x"], t["W_gate"], q13, s13, q2, s2, w.K, w.renorm)
    y2 = moe.moe_forward_fp8a(t["x"], t["W_gate"], q13, s13, q2, s2, w.K, w.renorm)
    y0 = moe.moe_forward_fp8a(t["x"][:0], t["W_gate"], q13, s13, q2, s2, w.K, w.renorm)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert y0.shape == (0, w.H)


def test_fp8a_rejects_unsupported_shapes(dev):
    w = make_layer(8, 192, 64, 4, 2, dtype="bf16", seed=1)  # H not a multiple of 128
    t = layer_tensors(w, dev)
    q13, s13 = moe.moe_quantize_fp8(t["W13"])
    q2, s2 = moe.moe_quantize_fp8(t["W2"])
    with pytest.raises(moe.MoEError):
        moe.moe_forward_fp8a(t["x"], t["W_gate"], q13, s13, q2, s2, 2, False)
