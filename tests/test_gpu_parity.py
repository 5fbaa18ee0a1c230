"""Parity of every C-ABI call against the fp64 CPU oracle, on seeded inputs.

Inputs follow the workload recipe (x ~ N(0, 1), weights ~ N(0, 0.02)) at
every shape, so that outputs have the OLMoE layer's scale and the absolute
error bound keeps its meaning next to the relative ones.

Integer outputs (expert ids, counts, offsets, splits, perm, inv) and row
copies must be bit-exact; floating-point outputs must stay within the
layer's bounds (bf16: max-abs 2e-2 and relative Frobenius 1e-2; fp32: 1e-5
for both; routing weights 1e-6; router logits relative Frobenius 1e-5). Sizes
span several tiles with ragged tails, empty and hot experts, ties, and the
full OLMoE-layer sizes the benchmark times.
"""

import numpy as np
import pytest
import torch

import oracle
import routing_token_permute_amd as moe
from gpu_util import assert_close, dev_tensor, errors, layer_tensors, require_gpu, to_f64
from oracle import moe_oracle as om
from workloads import make_config, make_layer, random_bf16_matrix, zipf_bias
from workloads.gen import make_ep_share

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _ids_from_random_logits(n, E, K, seed, bias=None):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((n, E)).astype(np.float32)
    if bias is not None:
        L = L + bias
    e_top, w_top, _ = oracle.route_from_logits(L, K, renorm=False)
    return L, e_top, w_top


def _tie_logits(n, E, seed):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((n, E)).astype(np.float32)
    L[0::7] = 0.5  # all equal rows
    L[1::7] = np.round(L[1::7] * 2) / 2  # coarse grid, many ties
    h = E // 2
    L[2::7, :h] = L[2::7, h : 2 * h]  # duplicated halves
    L[3::7] = np.where(np.arange(E) % 2 == 0, np.float32(0.0), np.float32(-0.0))
    L[4::7, ::3] = -np.inf
    return L


# ---------------------------------------------------------------------------
# moe_route
# ---------------------------------------------------------------------------

ROUTE_CASES = [
    # n, H, E, K, dtype, renorm, bias
    (64, 128, 8, 2, "f32", True, None),
    (300, 256, 64, 8, "bf16", False, None),
    (4096, 2048, 64, 8, "bf16", False, None),
    (4096, 2048, 64, 8, "bf16", False, "zipf"),
    (37, 128, 16, 16, "bf16", True, None),
    (1, 64, 1, 1, "bf16", False, None),
    (130, 192, 100, 7, "bf16", True, None),
    (50, 64, 256, 64, "bf16", False, None),
    (33, 68, 5, 3, "f32", False, None),
    (65536, 256, 64, 8, "bf16", False, None),  # 4096 workgroups
    (20000, 512, 128, 8, "bf16", True, None),  # 128 experts: 8 expert tiles, 4 waves over H
    # at most 256 tokens and E = 8 * 2^k: one workgroup per token
    (32, 2048, 64, 8, "bf16", False, None),    # the decode batch
    (17, 64, 8, 2, "bf16", True, None),        # E = 8: 256 rows per step, more than H
    (200, 192, 32, 4, "bf16", False, None),
    (256, 512, 128, 4, "bf16", True, "zipf"),  # -inf experts
    (100, 128, 256, 64, "bf16", False, None),
    (257, 256, 64, 8, "bf16", False, None),    # one token more: the batched router
]


@pytest.mark.parametrize("n,H,E,K,dtype,renorm,bias", ROUTE_CASES)
def test_route(dev, n, H, E, K, dtype, renorm, bias):
    b = zipf_bias(E) if bias == "zipf" else None
    w = make_layer(n, H, 64, E, K, dtype=dtype, renorm=renorm, seed=n + E, bias=b)
    t = layer_tensors(w, dev)
    logits, ids, wts = moe.moe_route(t["x"], t["W_gate"], t["bias"], K, renorm)
    torch.cuda.synchronize()
    ref = oracle.router_logits(w.x_f32, w.W_gate_f32, w.bias)
    got = logits.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref)
    assert (np.isfinite(got) == fin).all() and (got[~fin] == ref[~fin]).all()
    ma, rf = errors(got[fin], ref[fin])
    print(f"[route logits n={n} E={E}] max_abs={ma:.2e} rel_frob={rf:.2e}", flush=True)
    assert rf <= 1e-5 and ma <= 1e-4
    # Routing on every row: the oracle routes from the device's fp32 logits
    # (identical inputs to steps 2-3), so ids must match bit for bit, near-ties
    # of the top-K boundary included.
    L = logits.cpu().numpy()
    e_ref, w_ref, _ = oracle.route_from_logits(L, K, renorm)
    print(f"[route n={n} E={E}] rows at a top-K near-tie: {int((oracle.topk_margin(L, K) <= 1e-4).sum())}",
          flush=True)
    assert (ids.cpu().numpy() == e_ref).all()
    np.testing.assert_allclose(wts.cpu().numpy(), w_ref, atol=1e-6, rtol=0)


@pytest.mark.parametrize("n,E,K,renorm", [(200, 64, 8, False), (200, 64, 8, True), (90, 256, 64, True), (40, 5, 5, False), (70, 130, 9, False), (7, 1, 1, True), (150, 100, 6, True), (60, 128, 17, False)])
def test_topk_from_logits_bit_exact(dev, n, E, K, renorm):
    L = _tie_logits(n, E, seed=E + K)
    logits = torch.from_numpy(L).to(dev)
    _, ids, wts = moe.moe_route(None, None, None, K, renorm, logits=logits)
    torch.cuda.synchronize()
    e_ref, w_ref, _ = oracle.route_from_logits(L, K, renorm)
    assert (ids.cpu().numpy() == e_ref).all()
    np.testing.assert_allclose(wts.cpu().numpy(), w_ref, atol=1e-6, rtol=0)


# ---------------------------------------------------------------------------
# moe_permute
# ---------------------------------------------------------------------------

PERMUTE_CASES = [
    # n, H, E, K, ep, ids
    (300, 128, 8, 2, 4, "routed"),
    (4096, 2048, 64, 8, 8, "routed"),
    (4096, 2048, 64, 8, 8, "skewed"),
    (256, 64, 64, 8, 1, "routed"),  # n*K = 2048: exactly one counting block
    (1, 64, 8, 8, 2, "routed"),
    (513, 192, 16, 4, 16, "random"),  # repeated experts within a row
    (777, 64, 8, 1, 1, "one_hot"),  # every pair to one expert
    (3001, 64, 256, 6, 32, "random"),
    (64, 132, 8, 2, 1, "routed_f32"),
    (5000, 64, 64, 8, 4, "routed"),  # 40000 pairs: past the single-workgroup limit, count + place launches
    (4096, 64, 8, 8, 1, "one_hot"),  # all 32768 pairs in one segment (count + place launches)
    (512, 64, 8, 8, 1, "one_hot"),  # 4096 pairs in one segment: the single-workgroup maximum
    (16384, 64, 64, 8, 8, "routed"),  # 131072 pairs: 128 blocks of 1024 (four 64-pair steps per wave)
    (65536, 64, 64, 8, 8, "random"),  # 524288 pairs: blocks of 4096, two batches of 64-pair steps per wave
    (70001, 64, 256, 3, 32, "random"),  # 210003 pairs, 256 experts: the last block is partial
    (65536, 64, 8, 8, 1, "one_hot"),  # 524288 pairs in one segment
]


@pytest.mark.parametrize("n,H,E,K,ep,kind", PERMUTE_CASES)
def test_permute(dev, n, H, E, K, ep, kind):
    rng = np.random.default_rng(n * 7 + E)
    if kind == "routed" or kind == "routed_f32":
        _, e_top, _ = _ids_from_random_logits(n, E, K, seed=n)
    elif kind == "skewed":
        _, e_top, _ = _ids_from_random_logits(n, E, K, seed=n, bias=zipf_bias(E))
    elif kind == "random":
        e_top = rng.integers(0, E, size=(n, K)).astype(np.int32)
    else:
        e_top = np.full((n, K), 3, dtype=np.int32)
    dtype = "f32" if kind == "routed_f32" else "bf16"
    if dtype == "bf16":
        xb, xf = random_bf16_matrix(rng, (n, H))
    else:
        xf = rng.standard_normal((n, H)).astype(np.float32)
        xb = xf
    x = dev_tensor(xb, dtype, dev)
    out = moe.moe_permute(torch.from_numpy(e_top).to(dev), x, E, ep=ep)
    torch.cuda.synchronize()
    counts = oracle.expert_counts(e_top, E)
    offsets = oracle.offsets_from_counts(counts)
    perm, inv = oracle.permutation(e_top, E)
    assert (out["counts"].cpu().numpy() == counts).all()
    assert (out["offsets"].cpu().numpy() == offsets).all()
    assert (out["splits"].cpu().numpy() == om.splits_by_rank(e_top, E, ep)).all()
    assert (out["perm"].cpu().numpy() == perm).all()
    assert (out["inv"].cpu().numpy() == inv).all()
    xp = out["x_perm"].cpu()
    xp = xp.view(torch.int16).numpy() if dtype == "bf16" else xp.numpy()
    ref = np.asarray(xb)[perm // K]
    assert (xp.view(ref.dtype) == ref).all()


def test_permute_empty_and_metadata_only(dev):
    E, K = 8, 2
    ids = torch.zeros((0, K), dtype=torch.int32, device=dev)
    out = moe.moe_permute(ids, None, E, ep=2)
    torch.cuda.synchronize()
    assert (out["counts"].cpu() == 0).all() and (out["offsets"].cpu() == 0).all() and (out["splits"].cpu() == 0).all()
    _, e_top, _ = _ids_from_random_logits(100, E, K, seed=1)
    out = moe.moe_permute(torch.from_numpy(e_top).to(dev), None, E)
    torch.cuda.synchronize()
    perm, _ = oracle.permutation(e_top, E)
    assert (out["perm"].cpu().numpy() == perm).all()


# ---------------------------------------------------------------------------
# moe_grouped_swiglu
# ---------------------------------------------------------------------------


def _segments(kind, rows, E, rng):
    if kind == "random":
        cuts = np.sort(rng.integers(0, rows + 1, size=E - 1))
        counts = np.diff(np.concatenate([[0], cuts, [rows]]))
    elif kind == "edge":  # empty, single-row, tile+1, and the rest
        counts = np.zeros(E, dtype=np.int64)
        counts[1] = 1
        counts[2] = 129
        counts[3] = rows - 130
    elif kind == "hot":  # one expert takes everything, in the middle
        counts = np.zeros(E, dtype=np.int64)
        counts[E // 2] = rows
    else:
        raise ValueError(kind)
    return counts.astype(np.int64)


GROUPED_CASES = [
    # rows, E, H, I, dtype, kind
    (300, 8, 128, 64, "bf16", "random"),
    (1000, 4, 256, 128, "bf16", "edge"),
    (777, 6, 192, 192, "bf16", "hot"),  # H % 128 == 64: masked output columns
    (2500, 16, 512, 256, "bf16", "random"),
    (130, 5, 64, 64, "f32", "edge"),
    (300, 8, 128, 64, "f32", "random"),
    (76800, 256, 128, 64, "bf16", "random"),  # E at its maximum, 2 row tiles per expert: >1 tile per workgroup
    (700, 4, 64, 128, "bf16", "random"),  # 256-row tiles with a single 64-deep k-step in GEMM1
]


@pytest.mark.parametrize("rows,E,H,I,dtype,kind", GROUPED_CASES)
def test_grouped_swiglu(dev, rows, E, H, I, dtype, kind):  # noqa: E741
    rng = np.random.default_rng(rows + H)
    counts = _segments(kind, rows, E, rng)
    offsets = oracle.offsets_from_counts(counts)
    w = make_layer(1, H, I, E, 1, dtype=dtype, seed=rows)
    if dtype == "bf16":
        xb, xf = random_bf16_matrix(rng, (rows, H))
    else:
        xf = rng.standard_normal((rows, H)).astype(np.float32)
        xb = xf
    t = layer_tensors(w, dev)
    Y = moe.moe_grouped_swiglu(dev_tensor(xb, dtype, dev), torch.from_numpy(offsets.astype(np.int32)).to(dev), t["W13"], t["W2"])
    torch.cuda.synchronize()
    ref = om.grouped_swiglu(xf, offsets, w.W13_f32, w.W2_f32)
    assert_close(to_f64(Y), ref, dtype, f"grouped rows={rows} E={E} {kind}")


@pytest.mark.parametrize("n,H,I,E,K,kind", [(300, 128, 64, 8, 2, "routed"), (1000, 256, 192, 16, 4, "skewed"), (4096, 2048, 1024, 64, 8, "routed")])
def test_expert_gemm_halves_and_gather(dev, n, H, I, E, K, kind):  # noqa: E741
    """GEMM1 (+SwiGLU) alone, GEMM1 with the gather fused, and GEMM2 alone."""
    w = make_layer(n, H, I, E, K, seed=n + I)
    bias = zipf_bias(E) if kind == "skewed" else None
    _, e_top, _ = _ids_from_random_logits(n, E, K, seed=n, bias=bias)
    counts = oracle.expert_counts(e_top, E)
    offsets = oracle.offsets_from_counts(counts)
    perm, _ = oracle.permutation(e_top, E)
    t = layer_tensors(w, dev)
    off_d = torch.from_numpy(offsets.astype(np.int32)).to(dev)
    perm_d = torch.from_numpy(perm.astype(np.int32)).to(dev)
    xp = t["x"][perm_d.long() // K].contiguous()
    h1 = moe.moe_expert_w13_swiglu(xp, off_d, t["W13"])
    h2 = moe.moe_expert_w13_swiglu_gather(t["x"], perm_d, K, off_d, t["W13"])
    torch.cuda.synchronize()
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))  # same kernel arithmetic, same bits
    ref_h = om.grouped_gate_up(w.x_f32[perm // K], offsets, w.W13_f32)
    assert_close(to_f64(h1), ref_h, "bf16", f"gate_up n={n} E={E}", intermediate=True)
    # GEMM2 alone, on an independent seeded h of the same scale as SwiGLU outputs.
    hb, hf = random_bf16_matrix(np.random.default_rng(n), (n * K, I), std=0.3)
    Y = moe.moe_expert_w2(dev_tensor(hb, "bf16", dev), off_d, t["W2"])
    torch.cuda.synchronize()
    assert_close(to_f64(Y), om.grouped_down(hf, offsets, w.W2_f32), "bf16", f"down n={n} E={E}")


def test_grouped_swiglu_leaves_rows_past_offsets(dev):
    rows, E, H, I = 200, 4, 64, 64  # noqa: E741
    counts = np.array([50, 0, 70, 30])  # offsets[E] = 150 < rows
    offsets = oracle.offsets_from_counts(counts)
    w = make_layer(1, H, I, E, 1, seed=3)
    rng = np.random.default_rng(0)
    xb, xf = random_bf16_matrix(rng, (rows, H))
    t = layer_tensors(w, dev)
    Y = torch.full((rows, H), 7.0, dtype=torch.bfloat16, device=dev)
    moe.moe_grouped_swiglu(dev_tensor(xb, "bf16", dev), torch.from_numpy(offsets.astype(np.int32)).to(dev), t["W13"], t["W2"], Y_perm=Y)
    torch.cuda.synchronize()
    assert (Y[150:].float().cpu() == 7.0).all()
    ref = om.grouped_swiglu(xf[:150], offsets, w.W13_f32, w.W2_f32)
    assert_close(to_f64(Y[:150]), ref, "bf16", "grouped partial")


# ---------------------------------------------------------------------------
# moe_expert_w2_scatter and moe_sum_slots (GEMM2 with the weighted
# un-permutation in its epilogue, then the contiguous slot sum)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("n,H,I,E,K,dtype", [(300, 128, 64, 8, 2, "bf16"), (4096, 2048, 1024, 64, 8, "bf16"), (32, 2048, 1024, 64, 8, "bf16"), (100, 64, 64, 8, 2, "f32"), (513, 192, 128, 16, 4, "bf16")])
def test_w2_scatter(dev, n, H, I, E, K, dtype):  # noqa: E741
    w = make_layer(n, H, I, E, K, dtype=dtype, seed=n + 2 * I)
    _, e_top, w_top = _ids_from_random_logits(n, E, K, seed=n + 1)
    counts = oracle.expert_counts(e_top, E)
    offsets = oracle.offsets_from_counts(counts)
    perm, inv = oracle.permutation(e_top, E)
    rng = np.random.default_rng(n + 3)
    if dtype == "bf16":
        hb, hf = random_bf16_matrix(rng, (n * K, I), std=0.3)
    else:
        hf = (0.3 * rng.standard_normal((n * K, I))).astype(np.float32)
        hb = hf
    t = layer_tensors(w, dev)
    w32 = w_top.astype(np.float32)
    Yt = moe.moe_expert_w2_scatter(dev_tensor(hb, dtype, dev), torch.from_numpy(offsets.astype(np.int32)).to(dev),
                                   torch.from_numpy(perm.astype(np.int32)).to(dev), torch.from_numpy(w32).to(dev),
                                   t["W2"])
    torch.cuda.synchronize()
    Yp = om.grouped_down(hf, offsets, w.W2_f32)
    ref = oracle.weighted_rows_token_order(Yp, inv, w32, n, K)
    assert_close(to_f64(Yt), ref, dtype, f"w2 scatter n={n} E={E} K={K}")


@pytest.mark.parametrize("n,H,K,dtype", [(300, 128, 2, "bf16"), (4096, 2048, 8, "bf16"), (64, 132, 3, "f32"), (50, 256, 16, "bf16"), (7, 64, 1, "bf16")])
def test_sum_slots(dev, n, H, K, dtype):
    rng = np.random.default_rng(n + K)
    if dtype == "bf16":
        yb, yf = random_bf16_matrix(rng, (n * K, H))
    else:
        yf = rng.standard_normal((n * K, H)).astype(np.float32)
        yb = yf
    y = moe.moe_sum_slots(dev_tensor(yb, dtype, dev), n, K)
    torch.cuda.synchronize()
    ref = oracle.combine_slot_order(yf, np.arange(n * K), None, n, K)
    # Unweighted sums of K unit-variance rows reach |y| ~ 4 sqrt(K): the bf16
    # rounding of the output is relative, so only the relative bounds apply.
    assert_close(to_f64(y), ref, dtype, f"slot sum n={n} K={K}", intermediate=True)
    if K == 1 and dtype == "bf16":  # one slot: an exact copy
        assert (y.cpu().view(torch.int16).numpy().view(np.uint16) == yb).all()


# ---------------------------------------------------------------------------
# moe_unpermute_combine
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("n,H,E,K,dtype,weighted", [(300, 128, 8, 2, "bf16", True), (4096, 2048, 64, 8, "bf16", True), (129, 64, 4, 1, "bf16", False), (64, 132, 8, 2, "f32", True), (50, 256, 16, 16, "bf16", True)])
def test_combine(dev, n, H, E, K, dtype, weighted):
    _, e_top, w_top = _ids_from_random_logits(n, E, K, seed=n + K)
    perm, inv = oracle.permutation(e_top, E)
    rng = np.random.default_rng(5)
    if dtype == "bf16":
        yb, yf = random_bf16_matrix(rng, (n * K, H))
    else:
        yf = rng.standard_normal((n * K, H)).astype(np.float32)
        yb = yf
    w32 = w_top.astype(np.float32)
    wt = torch.from_numpy(w32).to(dev) if weighted else None
    y = moe.moe_unpermute_combine(dev_tensor(yb, dtype, dev), torch.from_numpy(inv.astype(np.int32)).to(dev), wt, n, K)
    torch.cuda.synchronize()
    ref = oracle.combine_slot_order(yf, inv, w32 if weighted else None, n, K)
    assert_close(to_f64(y), ref, dtype, f"combine n={n} K={K}")
    if not weighted and K == 1 and dtype == "bf16":  # a plain un-permute is an exact copy
        assert (y.cpu().view(torch.int16).numpy().view(np.uint16) == yb[inv]).all()


# ---------------------------------------------------------------------------
# moe_forward (whole layer)
# ---------------------------------------------------------------------------


def _check_logits(got_logits, ref_fp64, what):
    """Device router logits against the oracle's fp64 product (step 1): the same
    -inf entries, and relative Frobenius <= 1e-5 and max-abs <= 1e-4 on the rest."""
    got = got_logits.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_fp64)
    assert (np.isfinite(got) == fin).all() and (got[~fin] == ref_fp64[~fin]).all()
    ma, rf = errors(got[fin], ref_fp64[fin])
    print(f"[{what} logits] max_abs={ma:.2e} rel_frob={rf:.2e}", flush=True)
    assert rf <= 1e-5 and ma <= 1e-4


def _check_dispatch(dev, ids, counts, ref, E, what):
    """Steps 3-5 of every row, bit-exact: ids and counts from the layer call, and
    offsets, splits, perm and inv from the permute kernel the layer runs, on the
    layer's own ids."""
    ids_h = ids.cpu().numpy()
    assert (ids_h == ref["e_top"]).all(), f"{what}: expert ids differ"
    assert (counts.cpu().numpy() == ref["counts"]).all(), f"{what}: counts differ"
    meta = moe.moe_permute(ids, None, E)
    torch.cuda.synchronize()
    for k in ("offsets", "perm", "inv"):
        assert (meta[k].cpu().numpy() == ref[k]).all(), f"{what}: {k} differ"
    assert (meta["splits"].cpu().numpy() == ref["splits"]).all()


def _forward_parity(dev, w, what):
    """The whole layer on every row. Both sides route from the same fp32 logits:
    the device's, which are first held to the oracle's fp64 router product. Then
    routing and dispatch are compared bit-exact and y within the layer's bounds,
    near-ties of the top-K boundary included."""
    t = layer_tensors(w, dev)
    y, logits, ids, wts, counts = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"], routing_out=True)
    torch.cuda.synchronize()
    _check_logits(logits, oracle.router_logits(w.x_f32, w.W_gate_f32, w.bias), what)
    L = logits.cpu().numpy()
    ref = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, w.K, w.renorm, bias=w.bias,
                         routing_logits_f32=L)
    near = int((oracle.topk_margin(L, w.K) <= 1e-4).sum())
    print(f"[{what}] rows at a top-K near-tie (margin <= 1e-4), all compared: {near} of {w.n}", flush=True)
    _check_dispatch(dev, ids, counts, ref, w.E, what)
    np.testing.assert_allclose(wts.cpu().numpy(), ref["w_top"], atol=1e-6, rtol=0)
    assert_close(to_f64(y), ref["y"], w.dtype, what)
    return y


@pytest.mark.parametrize("name", ["tiny_f32", "decode_bf16", "olmoe_bf16", "olmoe_skewed_bf16"])
def test_forward_configs(dev, name):
    w = make_config(name)
    y = _forward_parity(dev, w, name)
    # Deterministic: a second call gives the same bits.
    t = layer_tensors(w, dev)
    y2 = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"])
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y, y2.view(torch.int16) if y2.dtype == torch.bfloat16 else y2)


@pytest.mark.parametrize("n,H,I,E,K,dtype,renorm", [(1, 64, 64, 8, 2, "bf16", False), (257, 128, 64, 1, 1, "bf16", False), (300, 128, 128, 8, 8, "bf16", True), (100, 64, 64, 16, 1, "f32", False), (45, 256, 192, 32, 4, "bf16", True), (300, 128, 64, 256, 64, "bf16", True), (4500, 128, 64, 64, 8, "bf16", False)])
def test_forward_small_shapes(dev, n, H, I, E, K, dtype, renorm):  # noqa: E741
    w = make_layer(n, H, I, E, K, dtype=dtype, renorm=renorm, seed=n + H + I)
    _forward_parity(dev, w, f"forward n={n} E={E} K={K}")


@pytest.mark.parametrize("n,H,I,E,K", [(256, 7168, 2048, 8, 2), (100, 4096, 1536, 16, 4)])
def test_forward_wide_layer(dev, n, H, I, E, K):  # noqa: E741
    """A wide layer (up to H = 7168, I = 2048): GEMM1 runs 112 k-steps of 64 and 16 column blocks, GEMM2 28
    column blocks, the router 112 slices of W_gate; every row against the oracle. Weights ~ N(0, 0.01^2), so
    that y stays about as large as at the OLMoE shape and the absolute bound keeps its meaning there."""
    w = make_layer(n, H, I, E, K, seed=H + I, w_std=0.01)
    _forward_parity(dev, w, f"wide layer H={H} I={I}")


def test_forward_large_batch_sampled(dev):
    """The OLMoE layer on 16384 tokens (131072 expert rows, about 20 GEMM tiles per CU): every token's
    routing and dispatch is checked bit-exact (the oracle routes from the device's fp32 logits, which are
    held to the fp64 router product first), and the outputs of 512 sampled tokens against the oracle run
    on those tokens alone (the layer treats each token independently)."""
    w = make_config("olmoe_bf16")
    n = 16384
    rng = np.random.default_rng(16384)
    xb, xf = random_bf16_matrix(rng, (n, w.H))
    t = layer_tensors(w, dev)
    x = dev_tensor(xb, "bf16", dev)
    y, logits, ids, wts, counts = moe.moe_forward(x, t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, routing_out=True)
    torch.cuda.synchronize()
    what = f"forward n={n}"
    _check_logits(logits, oracle.router_logits(xf, w.W_gate_f32, None), what)
    L = logits.cpu().numpy()
    e_ref, w_ref, _ = oracle.route_from_logits(L, w.K, w.renorm)
    counts_ref = oracle.expert_counts(e_ref, w.E)
    perm_ref, inv_ref = oracle.permutation(e_ref, w.E)
    ref_all = dict(e_top=e_ref, counts=counts_ref, offsets=oracle.offsets_from_counts(counts_ref),
                   splits=oracle.splits_by_rank(e_ref, w.E, 1), perm=perm_ref, inv=inv_ref)
    print(f"[{what}] rows at a top-K near-tie, all compared: {int((oracle.topk_margin(L, w.K) <= 1e-4).sum())}",
          flush=True)
    _check_dispatch(dev, ids, counts, ref_all, w.E, what)
    np.testing.assert_allclose(wts.cpu().numpy(), w_ref, atol=1e-6, rtol=0)
    sample = np.sort(rng.choice(n, size=512, replace=False))
    ref = oracle.forward(xf[sample], w.W_gate_f32, w.W13_f32, w.W2_f32, w.K, w.renorm, routing_logits_f32=L[sample])
    assert (ref["e_top"] == e_ref[sample]).all()
    assert_close(to_f64(y)[sample], ref["y"], "bf16", f"{what}, 512 sampled tokens")


@pytest.mark.parametrize("name", ["decode_bf16", "olmoe_bf16"])
def test_forward_timed_matches_forward_and_brackets_gemm1(dev, name):
    """moe_forward_timed gives moe_forward's bits; its two events bracket GEMM1 inside the call (a positive
    span shorter than the whole call); an event torch has not created yet is refused."""
    w = make_config(name)
    t = layer_tensors(w, dev)
    y = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"])
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    g1.record()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    y2 = moe.moe_forward_timed(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, g0, g1, bias=t["bias"])
    end.record()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    span, whole = g0.elapsed_time(g1), start.elapsed_time(end)
    print(f"[{name}] GEMM1 {span * 1e3:.1f} us of {whole * 1e3:.1f} us", flush=True)
    assert 0 < span < whole
    with pytest.raises(moe.MoEError):
        moe.moe_forward_timed(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm,
                              torch.cuda.Event(enable_timing=True), None, bias=t["bias"])


def test_forward_side_stream_internal_workspace(dev):
    """moe_forward on a side stream with the binding allocating the workspace and outputs: those blocks
    belong to the side stream, so work on the main stream that allocates and overwrites memory right
    after the call cannot receive them while the side stream's kernels still use them."""
    w = make_config("olmoe_bf16")
    t = layer_tensors(w, dev)
    ref = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    for _ in range(3):
        y = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, stream=side)
        nbytes = moe.moe_forward_workspace_size(w.n, w.H, w.I, w.E, w.K, torch.bfloat16)
        junk = torch.empty(nbytes, dtype=torch.uint8, device=dev)  # main stream
        junk.fill_(0x7F)
        del junk
        torch.cuda.current_stream(dev).wait_stream(side)
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
        y.record_stream(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()


def test_forward_zero_tokens(dev):
    w = make_layer(4, 64, 64, 8, 2, seed=0)
    t = layer_tensors(w, dev)
    x0 = t["x"][:0]
    y, logits, ids, wts, counts = moe.moe_forward(x0, t["W_gate"], t["W13"], t["W2"], 2, False, routing_out=True)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and (counts.cpu() == 0).all()


# ---------------------------------------------------------------------------
# One GPU's expert-parallel share (pre-received rows, K = 1, unit weights)
# ---------------------------------------------------------------------------


def _ep_share_run(dev, ep, mb, t13, t2, stream=None):
    x = dev_tensor(mb.x_bits(), "bf16", dev)
    eid = torch.from_numpy(mb.eid.reshape(-1, 1)).to(dev)
    meta = moe.moe_permute(eid, x, ep.E_local, stream=stream)
    Y = moe.moe_grouped_swiglu(meta["x_perm"], meta["offsets"], t13, t2, stream=stream)
    out = moe.moe_unpermute_combine(Y, meta["inv"], None, ep.R, 1, stream=stream)
    return meta, out


def test_ep_share_full(dev):
    ep = make_config("ep_share_bf16")
    t13 = dev_tensor(ep.bits("W13"), "bf16", dev)
    t2 = dev_tensor(ep.bits("W2"), "bf16", dev)
    for mb in ep.micro_batches:
        meta, out = _ep_share_run(dev, ep, mb, t13, t2)
        torch.cuda.synchronize()
        ref = om.ep_share_forward(mb.x_f32, mb.eid, ep.W13_f32, ep.W2_f32)
        assert (meta["counts"].cpu().numpy() == mb.counts).all()
        assert (meta["perm"].cpu().numpy() == ref["perm"]).all()
        assert_close(to_f64(out), ref["out"], "bf16", f"ep share seed={mb.seed}")


def test_ep_share_two_streams_match_serial(dev):
    """The two-stream schedule gives bitwise the same outputs as one stream, twice in a row."""
    from routing_token_permute_amd import ep_share as eps

    ep = make_config("ep_share_bf16")
    t13 = dev_tensor(ep.bits("W13"), "bf16", dev)
    t2 = dev_tensor(ep.bits("W2"), "bf16", dev)

    def mbs():
        return [eps.prepare(eps.MicroBatch(dev_tensor(m.x_bits(), "bf16", dev),
                                           torch.from_numpy(m.eid.reshape(-1, 1)).to(dev)), ep.E_local, ep.I)
                for m in ep.micro_batches]

    serial = mbs()
    eps.run_serial(serial[0], serial[1], t13, t2, ep.E_local, torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    two = mbs()
    compute, comm = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    for _ in range(2):
        for mb in two:
            mb.out.zero_()
        torch.cuda.synchronize()
        eps.run_two_streams(two[0], two[1], t13, t2, ep.E_local, compute, comm)
        torch.cuda.synchronize()
        for s_mb, t_mb in zip(serial, two):
            assert torch.equal(s_mb.out.view(torch.int16), t_mb.out.view(torch.int16))
            assert torch.equal(s_mb.meta["perm"], t_mb.meta["perm"])


def test_ep_share_fused_matches_serial(dev):
    """The fused schedule (metadata-only permute, gather-fused GEMM1, GEMM2 storing rows at their arrival
    positions with unit weights) gives bitwise the serial schedule's outputs, twice in a row, on the plain and
    on the packed weights."""
    from routing_token_permute_amd import ep_share as eps

    ep = make_config("ep_share_bf16")
    t13 = dev_tensor(ep.bits("W13"), "bf16", dev)
    t2 = dev_tensor(ep.bits("W2"), "bf16", dev)
    mbs = [eps.prepare(eps.MicroBatch(dev_tensor(m.x_bits(), "bf16", dev),
                                      torch.from_numpy(m.eid.reshape(-1, 1)).to(dev)), ep.E_local, ep.I)
           for m in ep.micro_batches]
    s0 = torch.cuda.current_stream(dev)
    eps.run_serial(mbs[0], mbs[1], t13, t2, ep.E_local, s0)
    packed = (moe.moe_pack_w13(t13), moe.moe_pack_w2(t2))
    for pk in (None, packed, None, packed):  # plain and packed weights, each twice
        for mb in mbs:
            mb.out_fused.zero_()
        eps.run_fused(mbs[0], mbs[1], t13, t2, ep.E_local, s0, packed=pk)
        torch.cuda.synchronize()
        for mb in mbs:
            assert torch.equal(mb.out.view(torch.int16), mb.out_fused.view(torch.int16))


def test_ep_share_cu_masked_streams_match_serial(dev):
    """The two-stream schedule on CU-masked streams (16 units for permute/unpermute, the rest for the GEMMs)
    gives bitwise the outputs of the serial run; the GEMM sizes its grid by its stream's mask."""
    from routing_token_permute_amd import ep_share as eps

    ep = make_config("ep_share_bf16")
    t13 = dev_tensor(ep.bits("W13"), "bf16", dev)
    t2 = dev_tensor(ep.bits("W2"), "bf16", dev)

    def mbs():
        return [eps.prepare(eps.MicroBatch(dev_tensor(m.x_bits(), "bf16", dev),
                                           torch.from_numpy(m.eid.reshape(-1, 1)).to(dev)), ep.E_local, ep.I)
                for m in ep.micro_batches]

    serial = mbs()
    eps.run_serial(serial[0], serial[1], t13, t2, ep.E_local, torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    ms = eps.MaskedStreams(16, dev)
    try:
        assert ms.n_compute == torch.cuda.get_device_properties(dev).multi_processor_count - 16
        for _ in range(2):
            over = mbs()
            eps.run_two_streams(over[0], over[1], t13, t2, ep.E_local, ms.compute, ms.comm)
            torch.cuda.synchronize()
            for s_, o_ in zip(serial, over):
                assert torch.equal(s_.out.view(torch.int16), o_.out.view(torch.int16))
    finally:
        torch.cuda.synchronize()
        ms.close()
