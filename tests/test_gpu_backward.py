"""Parity of the backward C-ABI calls against the fp64 CPU oracle's gradient.

Inputs follow the workload recipe (x ~ N(0, 1), weights ~ N(0, 0.02)); the
upstream gradient dy is drawn N(0, 1) with the same generators. Integer and
copy-like outputs must match exactly; floating-point gradients are held to
relative bounds (bf16: relative Frobenius 1e-2 and largest error at most 1e-2
of the largest reference value; fp32: 1e-5 for both), since their absolute
scale differs from the layer output's. The router's fp32 gradients are held
to 1e-4 relative (bf16 inputs) or 1e-5 (fp32).

Every bf16 gradient goes through the roundings the forward stores (gate_up,
h and Y_perm in bf16) and one rounding per backward stage (dY_perm,
dgate_up, dX_perm, then the output), each a relative perturbation of at most
2^-9 per element with random sign, so the relative Frobenius error of the
chain stays near 2^-9 * sqrt(4 / 3) ~ 2.3e-3, well inside 1e-2.
"""

import numpy as np
import pytest
import torch

import oracle
import routing_token_permute_amd as moe
from gpu_util import assert_close, dev_tensor, errors, layer_tensors, require_gpu, to_f64
from workloads import make_config, make_layer, random_bf16_matrix, zipf_bias

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _draw(rng, shape, dtype, std=1.0):
    if dtype == "bf16":
        return random_bf16_matrix(rng, shape, std)
    v = (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    return v, v


def _routing(n, E, K, seed, bias=None):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((n, E)).astype(np.float32)
    if bias is not None:
        L = L + bias
    e_top, w_top, _ = oracle.route_from_logits(L, K, renorm=False)
    perm, inv = oracle.permutation(e_top, E)
    offsets = oracle.offsets_from_counts(oracle.expert_counts(e_top, E))
    return L, e_top, w_top, perm, inv, offsets


def _i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def _f32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


# ---------------------------------------------------------------------------
# moe_combine_backward and moe_dispatch_backward
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("n,H,E,K,dtype", [(300, 128, 8, 2, "bf16"), (4096, 2048, 64, 8, "bf16"), (64, 132, 8, 3, "f32"),
                                           (50, 256, 16, 16, "bf16"), (7, 64, 1, 1, "bf16"), (33, 64, 70, 9, "bf16")])
def test_combine_backward(dev, n, H, E, K, dtype):
    rng = np.random.default_rng(n + H + K)
    _, _, w_top, _, inv, _ = _routing(n, E, K, seed=n)
    yb, yf = _draw(rng, (n * K, H), dtype, 0.05)
    db, dfl = _draw(rng, (n, H), dtype)
    dY, dw = moe.moe_combine_backward(dev_tensor(db, dtype, dev), dev_tensor(yb, dtype, dev), _i32(inv, dev),
                                      _f32(w_top, dev), n, K)
    torch.cuda.synchronize()
    ref_dY, ref_dw = oracle.combine_backward(dfl, yf, inv, w_top.astype(np.float32), n, K)
    assert_close(to_f64(dY), ref_dY, dtype, f"dY_perm n={n} K={K}", intermediate=True)
    ma, rf = errors(dw.cpu().numpy(), ref_dw)
    peak = np.abs(ref_dw).max()
    print(f"[dw n={n} K={K}] max_abs={ma:.2e} rel_frob={rf:.2e} peak={peak:.3g}", flush=True)
    assert rf <= 1e-5 and ma <= 1e-5 * peak + 1e-6


@pytest.mark.parametrize("n,H,E,K,dtype,add", [(300, 128, 8, 2, "bf16", True), (4096, 2048, 64, 8, "bf16", True),
                                               (64, 132, 8, 3, "f32", True), (129, 64, 4, 1, "bf16", False),
                                               (50, 256, 16, 16, "f32", False)])
def test_dispatch_backward(dev, n, H, E, K, dtype, add):
    rng = np.random.default_rng(n * 3 + K)
    _, _, _, perm, inv, _ = _routing(n, E, K, seed=n + 1)
    gb, gf = _draw(rng, (n * K, H), dtype)
    a = rng.standard_normal((n, H)).astype(np.float32) if add else None
    dx = moe.moe_dispatch_backward(dev_tensor(gb, dtype, dev), _i32(inv, dev), n, K,
                                   add=_f32(a, dev) if add else None)
    torch.cuda.synchronize()
    ref = oracle.dispatch_backward(gf, inv, n, K) + (a if add else 0.0)
    assert_close(to_f64(dx), ref, dtype, f"dispatch bwd n={n} K={K}", intermediate=True)
    # Adjoint of the gather: <x[perm/K], g> = <x, dispatch_backward(g)> (on the device result).
    if dtype == "f32" and not add:
        x = rng.standard_normal((n, H))
        lhs = np.sum(x[perm // K] * gf)
        assert abs(lhs - np.sum(x * to_f64(dx))) <= 1e-4 * (1 + abs(lhs))


# ---------------------------------------------------------------------------
# Grouped GEMMs of the backward
# ---------------------------------------------------------------------------


def _segments(kind, rows, E, rng):
    if kind == "random":
        cuts = np.sort(rng.integers(0, rows + 1, size=E - 1))
        counts = np.diff(np.concatenate([[0], cuts, [rows]]))
    elif kind == "edge":  # empty, single row, a full tile plus one, a k-step plus one, the rest
        counts = np.zeros(E, dtype=np.int64)
        counts[1], counts[2], counts[3] = 1, 257, 33
        counts[4] = rows - 291
    elif kind == "hot":
        counts = np.zeros(E, dtype=np.int64)
        counts[E // 2] = rows
    else:
        raise ValueError(kind)
    return counts.astype(np.int64)


BWD_GEMM_CASES = [
    # rows, E, H, I, dtype, kind
    (300, 8, 128, 64, "bf16", "random"),
    (1000, 6, 256, 128, "bf16", "edge"),
    (777, 6, 192, 192, "bf16", "hot"),
    (2500, 16, 512, 256, "bf16", "random"),
    (130, 5, 64, 64, "f32", "random"),
    (600, 8, 128, 64, "f32", "edge"),
    (32768, 64, 2048, 1024, "bf16", "random"),
]


@pytest.mark.parametrize("rows,E,H,I,dtype,kind", BWD_GEMM_CASES)
def test_expert_w2_backward(dev, rows, E, H, I, dtype, kind):  # noqa: E741
    rng = np.random.default_rng(rows + I)
    offsets = oracle.offsets_from_counts(_segments(kind, rows, E, rng))
    db, dfl = _draw(rng, (rows, H), dtype)
    gb, gf = _draw(rng, (rows, 2 * I), dtype)
    wb, wf = _draw(rng, (E, I, H), dtype, 0.02)
    dgu = moe.moe_expert_w2_backward(dev_tensor(db, dtype, dev), _i32(offsets, dev), dev_tensor(wb, dtype, dev),
                                     dev_tensor(gb, dtype, dev))
    torch.cuda.synchronize()
    ref = oracle.swiglu_backward(oracle.grouped_data_grad(dfl, offsets, wf), gf)
    assert_close(to_f64(dgu), ref, dtype, f"dgate_up rows={rows} E={E} {kind}", intermediate=True)


@pytest.mark.parametrize("rows,E,H,I,dtype,kind", BWD_GEMM_CASES)
def test_expert_w13_backward(dev, rows, E, H, I, dtype, kind):  # noqa: E741
    rng = np.random.default_rng(rows + H)
    offsets = oracle.offsets_from_counts(_segments(kind, rows, E, rng))
    gb, gf = _draw(rng, (rows, 2 * I), dtype)
    wb, wf = _draw(rng, (E, H, 2 * I), dtype, 0.02)
    dX = moe.moe_expert_w13_backward(dev_tensor(gb, dtype, dev), _i32(offsets, dev), dev_tensor(wb, dtype, dev))
    torch.cuda.synchronize()
    ref = oracle.grouped_data_grad(gf, offsets, wf)
    assert_close(to_f64(dX), ref, dtype, f"dX_perm rows={rows} E={E} {kind}", intermediate=True)


WGRAD_CASES = [
    # rows, E, M, N, dtype, kind
    (300, 8, 64, 128, "bf16", "random"),
    (1000, 6, 128, 256, "bf16", "edge"),
    (777, 6, 192, 384, "bf16", "hot"),
    (2500, 16, 256, 512, "bf16", "random"),
    (130, 5, 64, 64, "f32", "random"),
    (600, 8, 128, 64, "f32", "edge"),
    (0, 4, 64, 128, "bf16", "random"),
    (32768, 64, 1024, 2048, "bf16", "random"),
    (32768, 64, 2048, 2048, "bf16", "random"),
]


@pytest.mark.parametrize("rows,E,M,N,dtype,kind", WGRAD_CASES)
def test_expert_weight_grad(dev, rows, E, M, N, dtype, kind):
    rng = np.random.default_rng(rows + M + N)
    counts = _segments(kind, rows, E, rng) if rows > 0 else np.zeros(E, dtype=np.int64)
    offsets = oracle.offsets_from_counts(counts)
    ab, af = _draw(rng, (rows, M), dtype)
    bb, bf = _draw(rng, (rows, N), dtype)
    # Poison the output so that a tile left unwritten shows up.
    dW = torch.full((E, M, N), float("nan"), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device=dev)
    moe.moe_expert_weight_grad(dev_tensor(ab, dtype, dev), dev_tensor(bb, dtype, dev), _i32(offsets, dev), dW=dW)
    torch.cuda.synchronize()
    got = to_f64(dW)
    assert np.isfinite(got).all()
    ref = oracle.grouped_weight_grad(af, bf, offsets)
    for e in np.flatnonzero(counts == 0):
        assert (got[e] == 0).all()
    if rows > 0:
        assert_close(got, ref, dtype, f"dW rows={rows} E={E} M={M} N={N} {kind}", intermediate=True)


@pytest.mark.parametrize("n,K,E,M,N,dtype,kind", [(300, 2, 8, 64, 128, "bf16", "routed"), (1000, 4, 16, 192, 256, "bf16", "skewed"),
                                                  (4096, 8, 64, 2048, 2048, "bf16", "routed"), (65, 3, 5, 64, 64, "f32", "routed"),
                                                  (7, 2, 8, 64, 128, "bf16", "routed")])
def test_expert_weight_grad_gather(dev, n, K, E, M, N, dtype, kind):
    """dW13 with the rows of x read through perm equals the weight gradient of the explicitly gathered rows."""
    rng = np.random.default_rng(n + M)
    bias = zipf_bias(E) if kind == "skewed" else None
    _, e_top, _, perm, _, offsets = _routing(n, E, K, seed=n + 5, bias=bias)
    xb, xf = _draw(rng, (n, M), dtype)
    bb, bf = _draw(rng, (n * K, N), dtype)
    dW = torch.full((E, M, N), float("nan"), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device=dev)
    moe.moe_expert_weight_grad_gather(dev_tensor(xb, dtype, dev), _i32(perm, dev), K, dev_tensor(bb, dtype, dev),
                                      _i32(offsets, dev), dW=dW)
    torch.cuda.synchronize()
    got = to_f64(dW)
    assert np.isfinite(got).all()
    ref = oracle.grouped_weight_grad(xf[perm // K], bf, offsets)
    counts = np.diff(offsets)
    for e in np.flatnonzero(counts == 0):
        assert (got[e] == 0).all()
    assert_close(got, ref, dtype, f"dW gathered n={n} K={K} E={E} M={M} N={N}", intermediate=True)


# ---------------------------------------------------------------------------
# moe_route_backward
# ---------------------------------------------------------------------------

ROUTE_BWD_CASES = [
    # n, H, E, K, dtype, renorm, bias
    (300, 256, 64, 8, "bf16", False, None),
    (4096, 2048, 64, 8, "bf16", False, None),
    (4096, 2048, 64, 8, "bf16", True, "zipf"),
    (37, 128, 16, 16, "bf16", True, None),
    (1, 64, 1, 1, "bf16", False, None),
    (130, 192, 100, 7, "bf16", True, None),
    (50, 64, 256, 64, "bf16", False, None),
    (33, 68, 5, 3, "f32", False, None),
    (200, 128, 8, 2, "f32", True, None),
]


@pytest.mark.parametrize("n,H,E,K,dtype,renorm,bias", ROUTE_BWD_CASES)
def test_route_backward(dev, n, H, E, K, dtype, renorm, bias):
    b = zipf_bias(E) if bias == "zipf" else None
    w = make_layer(n, H, 64, E, K, dtype=dtype, renorm=renorm, seed=n + E + 7, bias=b)
    t = layer_tensors(w, dev)
    logits, ids, wts = moe.moe_route(t["x"], t["W_gate"], t["bias"], K, renorm)
    rng = np.random.default_rng(n + K)
    dw_h = rng.standard_normal((n, K)).astype(np.float32)
    out = moe.moe_route_backward(t["x"], t["W_gate"], logits, ids, wts, _f32(dw_h, dev), renorm)
    torch.cuda.synchronize()
    L = logits.cpu().numpy()
    ids_h = ids.cpu().numpy()
    # The oracle ranks the same fp32 logits: the selection must agree exactly.
    e_ref, _, _ = oracle.route_from_logits(L, K, renorm)
    assert (ids_h == e_ref).all()
    ref = oracle.router_backward(L, ids_h, dw_h, K, renorm, x=w.x_f32, W_gate=w.W_gate_f32)
    tol = 1e-5 if dtype == "f32" else 1e-4
    for name in ("dlogits", "dx", "dW_gate", "dbias"):
        got = out["dx_router" if name == "dx" else name].cpu().numpy().astype(np.float64)
        r = ref[name]
        ma, rf = errors(got, r)
        peak = float(np.abs(r).max())
        print(f"[route bwd {name} n={n} E={E} K={K}] max_abs={ma:.2e} rel_frob={rf:.2e} peak={peak:.3g}", flush=True)
        if peak == 0:
            assert ma <= 1e-7
        else:
            assert rf <= tol and ma <= tol * peak


def test_route_backward_dlogits_only_and_empty(dev):
    w = make_layer(40, 64, 64, 8, 2, seed=3)
    t = layer_tensors(w, dev)
    logits, ids, wts = moe.moe_route(t["x"], t["W_gate"], None, 2, False)
    dw = torch.ones((40, 2), dtype=torch.float32, device=dev)
    out = moe.moe_route_backward(None, None, logits, ids, wts, dw, False, want_dx=False, want_weights=False)
    full = moe.moe_route_backward(t["x"], t["W_gate"], logits, ids, wts, dw, False)
    torch.cuda.synchronize()
    assert torch.equal(out["dlogits"], full["dlogits"])
    e = moe.moe_route_backward(t["x"][:0], t["W_gate"], logits[:0], ids[:0], wts[:0], dw[:0], False)
    torch.cuda.synchronize()
    assert (e["dW_gate"].cpu() == 0).all() and (e["dbias"].cpu() == 0).all()


# ---------------------------------------------------------------------------
# Training forward and the whole backward
# ---------------------------------------------------------------------------


def _backward_parity(dev, w, what, dy_seed=0):
    t = layer_tensors(w, dev)
    y, saved = moe.moe_forward_train(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"])
    y_plain = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"])
    db, dfl = _draw(np.random.default_rng(dy_seed + w.n), (w.n, w.H), w.dtype)
    grads = moe.moe_backward(dev_tensor(db, w.dtype, dev), t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm,
                             saved)
    torch.cuda.synchronize()
    # The training forward runs the same arithmetic as moe_forward.
    assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y,
                       y_plain.view(torch.int16) if y.dtype == torch.bfloat16 else y_plain)
    # Both sides route from the device's fp32 logits (held to the fp64 router
    # product first), so every row is compared, near-ties of the top-K
    # boundary included.
    ref_logits = oracle.router_logits(w.x_f32, w.W_gate_f32, w.bias)
    got_logits = saved["logits"].cpu().numpy()
    fin = np.isfinite(ref_logits)
    assert (np.isfinite(got_logits) == fin).all()
    ma, rf = errors(got_logits[fin].astype(np.float64), ref_logits[fin])
    assert rf <= 1e-5 and ma <= 1e-4, f"{what} logits: max_abs={ma:.2e} rel_frob={rf:.2e}"
    ref = oracle.backward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, w.K, w.renorm, dfl, bias=w.bias,
                          routing_logits_f32=got_logits)
    f = ref["fwd"]
    near = int((oracle.topk_margin(got_logits, w.K) <= 1e-4).sum())
    print(f"[{what}] rows at a top-K near-tie, all compared: {near} of {w.n}", flush=True)
    assert (saved["topk_ids"].cpu().numpy() == f["e_top"]).all()
    assert (saved["offsets"].cpu().numpy() == f["offsets"]).all()
    assert (saved["perm"].cpu().numpy() == f["perm"]).all()
    assert (saved["inv"].cpu().numpy() == f["inv"]).all()
    # Saved pre-activations and activations, expert-major.
    assert_close(to_f64(saved["gate_up"]), ref["gate_up"], w.dtype, f"{what} gate_up", intermediate=True)
    assert_close(to_f64(saved["h"]), ref["h"], w.dtype, f"{what} h", intermediate=True)
    assert_close(to_f64(grads["dx"]), ref["dx"], w.dtype, f"{what} dx", intermediate=True)
    tol = 1e-5 if w.dtype == "f32" else 1e-2
    for name in ("dW13", "dW2", "dW_gate", "dbias"):
        got = to_f64(grads[name])
        ma, rf = errors(got, ref[name])
        peak = float(np.abs(ref[name]).max())
        print(f"[{what} {name}] max_abs={ma:.3e} rel_frob={rf:.3e} peak={peak:.3g}", flush=True)
        assert rf <= tol and ma <= tol * peak
    return grads


@pytest.mark.parametrize("n,H,I,E,K,dtype,renorm", [
    (64, 64, 64, 8, 2, "f32", False),
    (100, 128, 64, 16, 4, "f32", True),
    (300, 128, 128, 8, 8, "bf16", True),
    (257, 128, 64, 1, 1, "bf16", False),
    (45, 256, 192, 32, 4, "bf16", True),
    (1, 64, 64, 8, 2, "bf16", False),
    (513, 192, 128, 16, 4, "bf16", False),
])
def test_backward_small_shapes(dev, n, H, I, E, K, dtype, renorm):  # noqa: E741
    w = make_layer(n, H, I, E, K, dtype=dtype, renorm=renorm, seed=n + H + 3 * I)
    _backward_parity(dev, w, f"backward n={n} H={H} I={I} E={E} K={K} {dtype}")


def test_backward_wide_layer(dev):
    """The backward on a wide layer (H = 7168, I = 2048): the data gradients reduce over 2048- and 7168-wide
    rows, dW13 and dW2 are 7168 x 4096 and 2048 x 7168 per expert; every gradient against the oracle.
    Weights ~ N(0, 0.01^2), as in the forward's wide-layer test."""
    w = make_layer(128, 7168, 2048, 8, 2, seed=29, w_std=0.01)
    _backward_parity(dev, w, "backward wide H=7168 I=2048")


@pytest.mark.parametrize("name", ["tiny_f32", "decode_bf16", "olmoe_bf16", "olmoe_skewed_bf16"])
def test_backward_configs(dev, name):
    w = make_config(name)
    g1 = _backward_parity(dev, w, f"backward {name}")
    if name == "olmoe_bf16":  # deterministic: a second backward gives the same bits
        t = layer_tensors(w, dev)
        _, saved = moe.moe_forward_train(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"])
        db, _ = _draw(np.random.default_rng(w.n), (w.n, w.H), w.dtype)
        g2 = moe.moe_backward(dev_tensor(db, w.dtype, dev), t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm,
                              saved)
        torch.cuda.synchronize()
        for k in g1:
            a, b = g1[k], g2[k]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), k


def test_backward_zero_tokens(dev):
    w = make_layer(4, 64, 64, 8, 2, seed=0)
    t = layer_tensors(w, dev)
    x0 = t["x"][:0]
    y, saved = moe.moe_forward_train(x0, t["W_gate"], t["W13"], t["W2"], 2, False)
    grads = moe.moe_backward(x0.clone(), x0, t["W_gate"], t["W13"], t["W2"], 2, False, saved)
    torch.cuda.synchronize()
    for k in ("dW13", "dW2", "dW_gate", "dbias"):
        assert (grads[k].float().cpu() == 0).all(), k
