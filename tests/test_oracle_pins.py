"""Pins for the fp64 CPU oracle: what the pages and the mathematics fix.

Each test ties one oracle function to something other than itself: the
worked moe_align_block_size example printed on the vLLM MoE page, a
separately written brute-force form, a closed form, an invariant, or a
special case that reduces to a textbook computation. None of these tests
touches the GPU.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from oracle import moe_oracle as om
from workloads import make_config, make_layer, zipf_bias

# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------


def _adversarial_logits(rng, n, E):
    """Random fp32 logits with planted ties, equal rows, -inf entries and signed zeros."""
    L = rng.standard_normal((n, E)).astype(np.float32)
    L[0, :] = 0.25  # all equal
    L[1, : E // 2] = L[1, E // 2 :]  # every value duplicated
    L[2, :] = -np.inf
    L[2, E - 1] = 1.0
    L[2, 0] = 0.5  # only a few finite
    L[3, :] = np.where(np.arange(E) % 2 == 0, np.float32(0.0), np.float32(-0.0))
    L[4, :] = np.round(L[4, :] * 2) / 2  # coarse grid: many ties
    L[5, ::3] = -np.inf
    return L


# ---------------------------------------------------------------------------
# The printed worked example
# ---------------------------------------------------------------------------


def test_worked_example_moe_align_block_size(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "moe_align_block_size_example.json")))
    e_top = np.array(ex["topk_ids_as_printed"]) - ex["id_base"]
    E, K, BM = ex["E"], ex["K"], ex["BLOCK_SIZE_M"]
    counts = oracle.expert_counts(e_top, E)
    assert counts.tolist() == [ex["hits_per_expert"]] * E
    perm, inv = oracle.permutation(e_top, E)
    offsets = oracle.offsets_from_counts(counts)
    # Rebuild the page's padded layout from (perm, offsets): each expert's
    # segment padded to a multiple of BLOCK_SIZE_M, one expert id per block.
    padded, block_expert = [], []
    for e in range(E):
        seg = perm[offsets[e] : offsets[e + 1]].tolist()
        nblk = -(-len(seg) // BM)
        padded += seg + ["PAD"] * (nblk * BM - len(seg))
        block_expert += [e] * nblk
    assert padded == ex["sorted_token_ids_as_printed"]
    assert block_expert == ex["expert_ids_as_printed"]
    assert len(padded) == ex["num_tokens_post_padded"]
    assert (perm[inv] == np.arange(E * 3)).all()


# ---------------------------------------------------------------------------
# Router: softmax and top-K
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("E,K", [(8, 2), (8, 8), (64, 8), (5, 1), (64, 64), (3, 2)])
def test_topk_matches_bruteforce_on_ties(E, K):
    rng = np.random.default_rng(E * 100 + K)
    L = _adversarial_logits(rng, 40, E) if E >= 6 else rng.standard_normal((40, E)).astype(np.float32)
    e_top, w_top, p = oracle.route_from_logits(L, K, renorm=False)
    for i, row in enumerate(L.tolist()):
        a = brute.topk_argmax_passes(row, K)
        b = brute.topk_full_sort(row, K)
        assert e_top[i].tolist() == a == b, (i, row)
        pb = brute.softmax_row(row)
        np.testing.assert_allclose(p[i], pb, rtol=1e-13, atol=1e-300)


def test_topk_invariants_and_renorm():
    rng = np.random.default_rng(7)
    L = _adversarial_logits(rng, 200, 16)
    K = 4
    e_top, w_top, p = oracle.route_from_logits(L, K, renorm=False)
    for i in range(L.shape[0]):
        sel = set(e_top[i].tolist())
        assert len(sel) == K
        unsel = [e for e in range(16) if e not in sel]
        assert min(L[i, e_top[i]]) >= max(L[i, unsel])
        assert (np.diff(w_top[i]) <= 0).all()  # non-increasing by slot
        assert (w_top[i] >= 0).all()
        # ties among selected: ascending expert index within equal logits
        for k in range(K - 1):
            if L[i, e_top[i, k]] == L[i, e_top[i, k + 1]]:
                assert e_top[i, k] < e_top[i, k + 1]
    e2, w2, _ = oracle.route_from_logits(L, K, renorm=True)
    assert (e2 == e_top).all()
    np.testing.assert_allclose(w2.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(w2, w_top / w_top.sum(axis=1, keepdims=True), rtol=1e-15)


def test_softmax_closed_forms():
    # Two experts: p0 = 1 / (1 + exp(l1 - l0)) (the logistic function).
    L = np.array([[0.3, -1.2], [5.0, 5.0], [-40.0, 2.0]], dtype=np.float32)
    _, _, p = oracle.route_from_logits(L, 1, renorm=False)
    l64 = L.astype(np.float64)
    np.testing.assert_allclose(p[:, 0], 1.0 / (1.0 + np.exp(l64[:, 1] - l64[:, 0])), rtol=1e-14)
    # Shift invariance, rows sum to one, -inf gives probability 0.
    rng = np.random.default_rng(3)
    L = rng.standard_normal((20, 9)).astype(np.float32)
    L[:, 4] = -np.inf
    _, _, p1 = oracle.route_from_logits(L, 3, renorm=False)
    _, _, p2 = oracle.route_from_logits(L + np.float32(8.0), 3, renorm=False)
    np.testing.assert_allclose(p1.sum(axis=1), 1.0, atol=1e-14)
    assert (p1[:, 4] == 0).all()
    np.testing.assert_allclose(p1, p2, atol=1e-6)  # fp32 shift rounds the inputs slightly


def test_topk_e_equals_k_renorm_is_full_softmax():
    rng = np.random.default_rng(11)
    L = rng.standard_normal((10, 6)).astype(np.float32)
    e_top, w_top, p = oracle.route_from_logits(L, 6, renorm=True)
    for i in range(10):
        np.testing.assert_allclose(w_top[i], p[i, e_top[i]], rtol=1e-14)


def test_router_logits_small_closed_form():
    x = np.array([[1.0, 2.0], [0.5, -1.0]])
    W = np.array([[1.0, 0.0, 2.0], [0.0, 1.0, -1.0]])
    b = np.array([0.0, 1.0, -np.inf], dtype=np.float32)
    L = oracle.router_logits(x, W, b)
    assert L[0].tolist()[:2] == [1.0, 3.0] and L[1].tolist()[:2] == [0.5, 0.0]
    assert np.isneginf(L[:, 2]).all()


# ---------------------------------------------------------------------------
# Counts, offsets, splits, permutation
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("n,E,K,ep", [(37, 8, 2, 4), (64, 8, 8, 1), (300, 64, 8, 8), (1, 4, 4, 2), (0, 8, 2, 2)])
def test_dispatch_metadata_invariants(n, E, K, ep):
    rng = np.random.default_rng(n + E + K)
    L = rng.standard_normal((n, E)).astype(np.float32)
    e_top, _, _ = oracle.route_from_logits(L, K, renorm=False) if n else (np.zeros((0, K), np.int32), None, None)
    counts = oracle.expert_counts(e_top, E)
    offsets = oracle.offsets_from_counts(counts)
    splits = oracle.splits_by_rank(e_top, E, ep)
    assert counts.sum() == n * K and (counts >= 0).all() and (counts <= n).all()
    assert offsets[0] == 0 and offsets[-1] == n * K and (np.diff(offsets) == counts).all()
    assert (splits == oracle.splits_from_offsets(offsets, ep)).all() and splits.sum() == n * K
    perm, inv = oracle.permutation(e_top, E)
    assert sorted(perm.tolist()) == list(range(n * K))  # bijection
    assert (perm[inv] == np.arange(n * K)).all() and (inv[perm] == np.arange(n * K)).all()
    flat = e_top.reshape(-1)
    for e in range(E):
        seg = perm[offsets[e] : offsets[e + 1]]
        assert (flat[seg] == e).all()
        assert (np.diff(seg) > 0).all()
    # An independently written stable sort by expert gives the same order.
    assert (np.argsort(flat, kind="stable") == perm).all()
    if n * K <= 2400:
        pb, ib = brute.permutation_triple_loop(e_top.tolist(), E)
        assert perm.tolist() == pb and inv.tolist() == ib


def test_splits_reject_bad_ep():
    with pytest.raises(ValueError):
        oracle.splits_by_rank(np.zeros((3, 2), np.int32), 8, 3)


# ---------------------------------------------------------------------------
# Experts and the whole layer
# ---------------------------------------------------------------------------


def _tiny(n=9, H=16, I=8, E=4, K=2, renorm=False, seed=5, dtype="f32"):  # noqa: E741
    return make_layer(n, H, I, E, K, dtype=dtype, renorm=renorm, seed=seed, w_std=0.3)


@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("E,K", [(4, 2), (4, 1), (4, 4), (6, 3)])
def test_layer_matches_per_token_and_dense_bruteforce(E, K, renorm):
    w = _tiny(E=E, K=K, renorm=renorm, seed=E * 10 + K)
    out = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, K, renorm, keep_permuted=True)
    e_b, w_b = brute.route(out["logits_f32"], K, renorm)
    assert out["e_top"].tolist() == e_b
    np.testing.assert_allclose(out["w_top"], np.array(w_b), rtol=1e-13)
    y_tok = brute.layer_per_token(w.x_f32, e_b, w_b, w.W13_f32, w.W2_f32)
    y_dense = brute.layer_dense(w.x_f32, e_b, w_b, w.W13_f32, w.W2_f32)
    np.testing.assert_allclose(out["y"], y_tok, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["y"], y_dense, rtol=1e-12, atol=1e-14)
    # The slot-order combine of the expert-major outputs is the same layer.
    y_c = oracle.combine_slot_order(out["Y_perm"], out["inv"], out["w_top"], w.n, K)
    np.testing.assert_allclose(out["y"], y_c, rtol=1e-12, atol=1e-14)


def test_single_expert_is_plain_swiglu_ffn():
    """E = 1, K = 1: the layer is one dense SwiGLU FFN; gate = first I columns."""
    w = _tiny(E=1, K=1)
    out = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, 1, False)
    x = w.x_f32.astype(np.float64)
    W_gate_proj = w.W13_f32[0][:, : w.I].astype(np.float64)
    W_up_proj = w.W13_f32[0][:, w.I :].astype(np.float64)
    g = np.einsum("nh,hi->ni", x, W_gate_proj)
    u = np.einsum("nh,hi->ni", x, W_up_proj)
    sig = np.array([[1.0 / (1.0 + math.exp(-v)) for v in row] for row in g])
    ref = np.einsum("ni,ih->nh", g * sig * u, w.W2_f32[0].astype(np.float64))
    assert (out["w_top"] == 1.0).all()
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-14)


def test_identical_experts_with_renorm_give_the_ffn():
    """All experts equal and weights renormalised: y = FFN(x) whatever the routing."""
    w = _tiny(E=5, K=3, renorm=True)
    W13 = np.repeat(w.W13_f32[:1], 5, axis=0)
    W2 = np.repeat(w.W2_f32[:1], 5, axis=0)
    out = oracle.forward(w.x_f32, w.W_gate_f32, W13, W2, 3, True)
    ref = np.stack([brute.ffn_token(w.x_f32[i], W13[0], W2[0]) for i in range(w.n)])
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-14)


def test_k_equals_e_with_renorm_is_dense_softmax_mixture():
    w = _tiny(E=4, K=4, renorm=True)
    out = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, 4, True)
    L = out["logits_f32"].astype(np.float64)
    p = np.exp(L - L.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = np.zeros_like(out["y"])
    for i in range(w.n):
        for e in range(4):
            ref[i] += p[i, e] * brute.ffn_token(w.x_f32[i], w.W13_f32[e], w.W2_f32[e])
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-14)


def test_linearity_in_w2():
    w = _tiny(E=4, K=2)
    out0 = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, np.zeros_like(w.W2_f32), 2, False)
    assert (out0["y"] == 0).all()
    a = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, 2, False)["y"]
    b = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, 2.5 * w.W2_f32.astype(np.float64), 2, False)["y"]
    np.testing.assert_allclose(b, 2.5 * a, rtol=1e-13, atol=1e-15)


def test_silu_identities():
    # silu(z) - silu(-z) = z, silu(0) = 0, and silu(z) ~ z for large z.
    X = np.array([[1.0]])
    for z in [-3.0, -0.5, 0.0, 0.7, 4.0]:
        W13 = np.array([[z, 1.0]])  # gate column = z, up column = 1
        W2 = np.array([[1.0]])
        fz = oracle.expert_ffn(X, W13, W2)[0, 0]
        fm = oracle.expert_ffn(X, np.array([[-z, 1.0]]), W2)[0, 0]
        assert abs((fz - fm) - z) < 1e-15
    big = oracle.expert_ffn(X, np.array([[40.0, 1.0]]), np.array([[1.0]]))[0, 0]
    assert abs(big - 40.0) < 1e-12
    # gate is the first half: gate = -3, up = 2 gives silu(-3) * 2, not silu(2) * (-3)
    v = oracle.expert_ffn(X, np.array([[-3.0, 2.0]]), np.array([[1.0]]))[0, 0]
    assert abs(v - (-3.0 / (1 + math.exp(3.0)) * 2.0)) < 1e-15


def test_grouped_gate_up_and_down_match_row_by_row_bruteforce():
    """Per-segment steps 8 and 9 against per-row loops, with an empty segment."""
    rng = np.random.default_rng(21)
    E, H, I, rows = 4, 12, 6, 17  # noqa: E741
    counts = np.array([5, 0, 9, 3])
    offsets = oracle.offsets_from_counts(counts)
    x = rng.standard_normal((rows, H))
    W13 = rng.standard_normal((E, H, 2 * I)) * 0.3
    W2 = rng.standard_normal((E, I, H)) * 0.3
    h = om.grouped_gate_up(x, offsets, W13)
    y = om.grouped_down(h, offsets, W2)
    for e in range(E):
        for r in range(offsets[e], offsets[e + 1]):
            np.testing.assert_allclose(h[r], brute.gate_up_token(x[r], W13[e]), rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(y[r], brute.down_token(h[r], W2[e]), rtol=1e-13, atol=1e-15)
    assert (h[offsets[-1]:] == 0).all() and (y[offsets[-1]:] == 0).all()


def test_grouped_swiglu_matches_layer_segments():
    w = _tiny(E=4, K=2)
    out = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, 2, False, keep_permuted=True)
    xp = w.x_f32[out["perm"] // 2]
    Y = om.grouped_swiglu(xp, out["offsets"], w.W13_f32, w.W2_f32)
    np.testing.assert_allclose(Y, out["Y_perm"], rtol=1e-14, atol=1e-16)


# ---------------------------------------------------------------------------
# The named workloads: properties the configs promise
# ---------------------------------------------------------------------------


def test_zipf_bias_recipe():
    b = zipf_bias(64)
    q = np.arange(1, 65, dtype=np.float64) ** -1.2
    q /= q.sum()
    finite = np.isfinite(b)
    assert (~finite).sum() == 8 and np.isneginf(b[7::8]).all()
    np.testing.assert_allclose(b[finite], (3 * np.log(q))[finite], rtol=1e-6)
    assert (np.diff(b[finite]) < 0).all()  # rank 1 is the most favoured


@pytest.mark.slow
def test_skewed_config_routing_properties():
    w = make_config("olmoe_skewed_bf16")
    L = oracle.round_to_f32(oracle.router_logits(w.x_f32, w.W_gate_f32, w.bias))
    e_top, _, _ = oracle.route_from_logits(L, w.K, renorm=False)
    counts = oracle.expert_counts(e_top, w.E)
    assert (counts[7::8] == 0).all()
    cv = counts.std() / counts.mean()
    assert cv > 1.0, cv
    assert counts.max() == w.n  # a hot expert takes every token


def test_tiny_config_routing_is_renormalised():
    w = make_config("tiny_f32")
    out = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, w.K, w.renorm)
    np.testing.assert_allclose(out["w_top"].sum(1), 1.0, atol=1e-12)
    assert out["counts"].sum() == w.n * w.K


def test_ep_share_oracle_small():
    from workloads.gen import make_ep_share

    ep = make_ep_share(R=96, H=32, I=16, E_local=4, S=3, alpha=0.5, w_std=0.2)
    mb = ep.micro_batches[0]
    out = om.ep_share_forward(mb.x_f32, mb.eid, ep.W13_f32, ep.W2_f32)
    # counts agree with the generator's own multinomial draw
    assert (out["counts"] == mb.counts).all()
    assert (out["counts"] == mb.source_counts.sum(0)).all()
    # every row goes through its own expert, in arrival order
    for r in range(ep.R):
        ref = brute.ffn_token(mb.x_f32[r], ep.W13_f32[mb.eid[r]], ep.W2_f32[mb.eid[r]])
        np.testing.assert_allclose(out["out"][r], ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Planted mistakes: the pins above must notice plausible slips in the oracle
# ---------------------------------------------------------------------------


def _pins_pass(fn, *a):
    try:
        fn(*a)
        return True
    except AssertionError:
        return False


def test_planted_mistakes_are_caught(monkeypatch, golden_dir):
    # 1. Ties to the highest expert index.
    orig_route = om.route_from_logits

    def route_ties_high(L, K, renorm, keep_fp64=False):
        L = np.asarray(L, np.float32)
        E = L.shape[1]
        e, w, p = orig_route(L[:, ::-1], K, renorm)
        return (E - 1 - e).astype(np.int32), w, p[:, ::-1]

    monkeypatch.setattr(oracle, "route_from_logits", route_ties_high)
    assert not _pins_pass(test_topk_matches_bruteforce_on_ties, 8, 2)
    monkeypatch.undo()

    # 2. Gate and up halves swapped.
    def ffn_swapped(X, W13, W2):
        W13 = np.asarray(W13, np.float64)
        I = W13.shape[1] // 2  # noqa: E741
        return orig_ffn(X, np.concatenate([W13[:, I:], W13[:, :I]], axis=1), W2)

    orig_ffn = om.expert_ffn
    monkeypatch.setattr(om, "expert_ffn", ffn_swapped)
    assert not _pins_pass(test_single_expert_is_plain_swiglu_ffn)
    monkeypatch.undo()

    # 3. Segments in descending token order (an unstable permutation).
    orig_perm = om.permutation

    def perm_reversed(e_top, E):
        perm, _ = orig_perm(e_top, E)
        counts = oracle.expert_counts(e_top, E)
        offs = oracle.offsets_from_counts(counts)
        perm = np.concatenate([perm[offs[e] : offs[e + 1]][::-1] for e in range(E)])
        inv = np.empty_like(perm)
        inv[perm] = np.arange(perm.size)
        return perm, inv

    monkeypatch.setattr(oracle, "permutation", perm_reversed)
    assert not _pins_pass(test_worked_example_moe_align_block_size, golden_dir)
    monkeypatch.undo()

    # 4. Weights taken from the logits instead of the softmax.
    def route_no_softmax(L, K, renorm, keep_fp64=False):
        e, w, p = orig_route(L, K, renorm, keep_fp64)
        return e, np.take_along_axis(np.asarray(L, np.float64), e.astype(np.int64), 1), p

    monkeypatch.setattr(om, "route_from_logits", route_no_softmax)
    assert not _pins_pass(test_layer_matches_per_token_and_dense_bruteforce, 4, 2, False)
    monkeypatch.undo()


def test_weighted_rows_token_order_sums_to_the_combine():
    """[Fusion] §4.2.5's fused second layer only moves Algorithm 2 step 11's summands: each token's K weighted
    rows, summed, are the slot-order combine; row i*K+k is slot k of token i (its expert row times its weight)."""
    n, E, K, H = 37, 6, 3, 5
    rng = np.random.default_rng(11)
    L = rng.standard_normal((n, E)).astype(np.float32)
    e_top, w_top, _ = oracle.route_from_logits(L, K, renorm=False)
    perm, inv = oracle.permutation(e_top, E)
    Y = rng.standard_normal((n * K, H))
    Z = oracle.weighted_rows_token_order(Y, inv, w_top, n, K)
    ref = oracle.combine_slot_order(Y, inv, w_top, n, K)
    np.testing.assert_allclose(Z.reshape(n, K, H).sum(axis=1), ref, rtol=1e-13, atol=1e-13)
    for i, k in [(0, 0), (5, 2), (n - 1, 1)]:
        p = inv[i * K + k]
        assert perm[p] == i * K + k
        np.testing.assert_allclose(Z[i * K + k], w_top[i, k] * Y[p], rtol=0, atol=0)


# ---------------------------------------------------------------------------
# Backward: the gradient of the layer, pinned by finite differences and by
# the dispatch/combine duality
# ---------------------------------------------------------------------------


def _grad_problem(n=7, H=6, I=4, E=5, K=2, seed=3, bias=True):  # noqa: E741
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, H))
    W_gate = rng.standard_normal((H, E))
    b = rng.standard_normal(E) if bias else None
    W13 = rng.standard_normal((E, H, 2 * I)) * 0.5
    W2 = rng.standard_normal((E, I, H)) * 0.5
    dy = rng.standard_normal((n, H))
    return x, W_gate, b, W13, W2, dy


def _fd_check(x, W_gate, b, W13, W2, dy, K, renorm, seed=0, eps=1e-6, tol=2e-7):
    """Central differences of L = <dy, y> along a random direction per input,
    against <gradient, direction>; the top-K selection must not move."""
    g = oracle.backward(x, W_gate, W13, W2, K, renorm, dy, bias=b, fp64_routing=True)
    e_ref = g["fwd"]["e_top"]
    params = dict(x=x, W_gate=W_gate, W13=W13, W2=W2)
    grads = dict(x=g["dx"], W_gate=g["dW_gate"], W13=g["dW13"], W2=g["dW2"])
    if b is not None:
        params["bias"], grads["bias"] = b, g["dbias"]
    rng = np.random.default_rng(seed)
    for name, val in params.items():
        V = rng.standard_normal(np.shape(val))

        def loss(sign):
            p = dict(params)
            p[name] = val + sign * eps * V
            f = oracle.forward(p["x"], p["W_gate"], p["W13"], p["W2"], K, renorm, bias=p.get("bias"), fp64_routing=True)
            assert (f["e_top"] == e_ref).all(), "the step moved the top-K selection"
            return float(np.sum(dy * f["y"]))

        fd = (loss(+1) - loss(-1)) / (2 * eps)
        an = float(np.sum(grads[name] * V))
        assert abs(fd - an) <= tol * (abs(an) + np.sqrt(np.sum(grads[name] ** 2)) * np.sqrt(V.size)), (name, fd, an)


@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("E,K", [(5, 2), (4, 1), (6, 6), (3, 3)])
def test_backward_matches_finite_differences(E, K, renorm):
    """Every gradient (x, W_gate, bias, W13, W2) of the fp64 layer agrees with central differences."""
    _fd_check(*_grad_problem(E=E, K=K, seed=E * 10 + K), K, renorm)


def test_backward_finite_differences_per_element():
    """Single-element differences for a few entries of each input (no averaging over a direction)."""
    x, W_gate, b, W13, W2, dy = _grad_problem(n=5, H=4, I=3, E=4, K=2, seed=9)
    g = oracle.backward(x, W_gate, W13, W2, 2, True, dy, bias=b, fp64_routing=True)
    eps = 1e-6

    def L(**kw):
        p = dict(x=x, W_gate=W_gate, W13=W13, W2=W2, bias=b)
        p.update(kw)
        f = oracle.forward(p["x"], p["W_gate"], p["W13"], p["W2"], 2, True, bias=p["bias"], fp64_routing=True)
        return float(np.sum(dy * f["y"]))

    for name, val, gr in [("x", x, g["dx"]), ("W_gate", W_gate, g["dW_gate"]), ("W13", W13, g["dW13"]),
                          ("W2", W2, g["dW2"]), ("bias", b, g["dbias"])]:
        flat = np.asarray(val).reshape(-1)
        for j in [0, flat.size // 3, flat.size - 1]:
            d = np.zeros_like(flat)
            d[j] = eps
            fd = (L(**{name: val + d.reshape(val.shape)}) - L(**{name: val - d.reshape(val.shape)})) / (2 * eps)
            assert abs(fd - gr.reshape(-1)[j]) <= 1e-7 * (1 + abs(fd)), (name, j, fd, gr.reshape(-1)[j])


def test_combine_and_dispatch_backward_are_adjoints():
    """[Fusion] §6.2.4 and [goin] §2.3 (d): the backward of a combine is a dispatch and the backward of a
    dispatch is a combine. For fixed weights both maps are linear, so each gradient map is the adjoint:
    <combine(Y), dy> = <Y, combine_backward(dy)>, <gather(x), dX> = <x, dispatch_backward(dX)>; and dw is
    the derivative of <combine(Y), dy> in w, which is linear too."""
    rng = np.random.default_rng(4)
    n, E, K, H = 23, 7, 3, 5
    L = rng.standard_normal((n, E)).astype(np.float32)
    e_top, w_top, _ = oracle.route_from_logits(L, K, renorm=False)
    perm, inv = oracle.permutation(e_top, E)
    Y = rng.standard_normal((n * K, H))
    dy = rng.standard_normal((n, H))
    dY, dw = oracle.combine_backward(dy, Y, inv, w_top, n, K)
    lhs = np.sum(oracle.combine_slot_order(Y, inv, w_top, n, K) * dy)
    assert abs(lhs - np.sum(Y * dY)) <= 1e-12 * (1 + abs(lhs))
    assert abs(lhs - np.sum(w_top * dw)) <= 1e-12 * (1 + abs(lhs))
    x = rng.standard_normal((n, H))
    dX = rng.standard_normal((n * K, H))
    lhs = np.sum(x[perm // K] * dX)
    assert abs(lhs - np.sum(x * oracle.dispatch_backward(dX, inv, n, K))) <= 1e-12 * (1 + abs(lhs))


def test_swiglu_backward_closed_forms():
    """At g = 0: SiLU'(0) = 1/2 and SiLU(0) = 0, so dg = dh·u/2 and du = 0; for large g, SiLU'(g) -> 1 and
    SiLU(g) -> g; for very negative g both go to 0."""
    dh = np.array([[2.0, -3.0, 1.0]])
    gu = np.array([[0.0, 40.0, -40.0, 5.0, 7.0, 11.0]])
    d = oracle.swiglu_backward(dh, gu)
    np.testing.assert_allclose(d[0, :3], [2.0 * 5.0 * 0.5, -3.0 * 7.0 * 1.0, 0.0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(d[0, 3:], [0.0, -3.0 * 40.0, 0.0], rtol=1e-12, atol=1e-12)


def test_router_backward_single_expert_and_dense_cases():
    """E = K = 1: the softmax of one logit is constant, so the router gradient vanishes. K = E with
    renormalisation: the weights are the full softmax, and dlogits is the softmax Jacobian applied to dw."""
    rng = np.random.default_rng(2)
    n, E = 6, 1
    r = oracle.router_backward(rng.standard_normal((n, E)), np.zeros((n, 1), np.int32), rng.standard_normal((n, 1)),
                               1, False, keep_fp64=True)
    assert np.abs(r["dlogits"]).max() == 0.0
    E = 4
    Lg = rng.standard_normal((n, E))
    e_top, _, p = oracle.route_from_logits(Lg, E, True, keep_fp64=True)
    dw = rng.standard_normal((n, E))
    r = oracle.router_backward(Lg, e_top, dw, E, True, keep_fp64=True)
    dp = np.zeros((n, E))
    np.put_along_axis(dp, e_top.astype(np.int64), dw, axis=1)
    for i in range(n):
        J = np.diag(p[i]) - np.outer(p[i], p[i])  # Jacobian of softmax (symmetric)
        np.testing.assert_allclose(r["dlogits"][i], J @ dp[i], rtol=1e-12, atol=1e-14)


def test_planted_backward_mistakes_are_caught(monkeypatch):
    prob = _grad_problem(E=5, K=2, seed=52)
    _fd_check(*prob, 2, True)

    def check():
        _fd_check(*prob, 2, True)

    # 1. SiLU derivative without its g·(1 - s) term.
    def swiglu_short(dh, gu):
        I = gu.shape[1] // 2  # noqa: E741
        g, u = gu[:, :I], gu[:, I:]
        s = 1 / (1 + np.exp(-g))
        return np.concatenate([dh * u * s, dh * g * s], axis=1)

    monkeypatch.setattr(om, "swiglu_backward", swiglu_short)
    assert not _pins_pass(check)
    monkeypatch.undo()

    # 2. Softmax backward without the <p, dp> term.
    orig_rb = om.router_backward

    def router_no_centering(Lg, e_top, dw, K, renorm, x=None, W_gate=None, keep_fp64=False):
        r = orig_rb(Lg, e_top, dw, K, renorm, x=x, W_gate=W_gate, keep_fp64=keep_fp64)
        _, _, p = oracle.route_from_logits(Lg, K, renorm, keep_fp64=keep_fp64)
        dp = np.zeros_like(p)
        np.put_along_axis(dp, np.asarray(e_top, np.int64), dw, axis=1)
        r["dlogits"] = p * dp
        r["dx"] = r["dlogits"] @ np.asarray(W_gate).T
        r["dW_gate"] = np.asarray(x).T @ r["dlogits"]
        r["dbias"] = r["dlogits"].sum(0)
        return r

    monkeypatch.setattr(om, "router_backward", router_no_centering)
    assert not _pins_pass(check)
    monkeypatch.undo()

    # 3. Renormalisation ignored in the backward.
    def router_no_renorm(Lg, e_top, dw, K, renorm, x=None, W_gate=None, keep_fp64=False):
        return orig_rb(Lg, e_top, dw, K, False, x=x, W_gate=W_gate, keep_fp64=keep_fp64)

    monkeypatch.setattr(om, "router_backward", router_no_renorm)
    assert not _pins_pass(check)
    monkeypatch.undo()

    # 4. Weight gradient with the operands the wrong way round (dout^T · in, transposed back).
    orig_wg = om.grouped_weight_grad

    def wg_swapped(inp, dout, offsets):
        inp = np.asarray(inp, np.float64)
        return orig_wg(inp[:, ::-1], dout, offsets)

    monkeypatch.setattr(om, "grouped_weight_grad", wg_swapped)
    assert not _pins_pass(check)
    monkeypatch.undo()

    # 5. Combine backward that forgets the routing weight.
    orig_cb = om.combine_backward

    def cb_unweighted(dy, Y, inv, w, n, K):
        return orig_cb(dy, Y, inv, np.ones_like(np.asarray(w, np.float64)), n, K)

    monkeypatch.setattr(om, "combine_backward", cb_unweighted)
    assert not _pins_pass(check)
    monkeypatch.undo()


# ---------------------------------------------------------------------------
# FP8 E4M3 weights: the format's definition and the column quantizer
# ---------------------------------------------------------------------------


def test_e4m3_table_landmarks():
    """Values fixed by the format: 1.0 = 0x38, the largest finite 448 = 0x7E, the smallest normal 2^-6 = 0x08,
    the smallest subnormal 2^-9 = 0x01, zero and minus zero, NaN at 0x7F/0xFF, and 127 distinct non-negative
    finite values in increasing code order."""
    t = oracle.fp8.e4m3_decode_table()
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0x08] == 2.0**-6 and t[0x01] == 2.0**-9
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0xB8] == -1.0 and t[0xFE] == -448.0
    assert t[0x3C] == 1.5 and t[0x40] == 2.0 and t[0x07] == 7 * 2.0**-9
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0) and len(np.unique(pos)) == 127
    np.testing.assert_array_equal(t[0x80:0xFF], -t[0x00:0x7F])


def test_e4m3_encode_round_trip_ties_and_saturation():
    f = oracle.fp8
    t = f.e4m3_decode_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)])
    np.testing.assert_array_equal(f.e4m3_encode(t[codes]), codes.astype(np.uint8))  # exact values map to themselves
    # Midpoints between neighbours go to the even code; just off the midpoint, to the nearer one.
    for c in range(0, 0x7E):
        a, b = t[c], t[c + 1]
        mid = (a + b) / 2
        even = c if c % 2 == 0 else c + 1
        assert f.e4m3_encode(np.array([mid]))[0] == even
        assert f.e4m3_encode(np.array([np.nextafter(mid, -np.inf)]))[0] == c
        assert f.e4m3_encode(np.array([np.nextafter(mid, np.inf)]))[0] == c + 1
        assert f.e4m3_encode(np.array([-mid]))[0] == (even | 0x80 if even else 0)
    # Saturation beyond the largest finite value; tiny values round to zero.
    np.testing.assert_array_equal(f.e4m3_encode(np.array([448.0, 464.0, 1e6, -1e6])), [0x7E, 0x7E, 0x7E, 0xFE])
    assert f.e4m3_encode(np.array([2.0**-11]))[0] == 0  # a quarter of the smallest subnormal


def test_e4m3_encode_error_bound_and_monotone():
    """|x - decode(encode(x))| is at most half the gap to the neighbouring value (the definition of nearest),
    and encoding is monotone."""
    f = oracle.fp8
    rng = np.random.default_rng(8)
    x = np.sort(np.concatenate([rng.uniform(-448, 448, 4000), rng.normal(0, 1e-2, 4000), rng.normal(0, 3, 4000)]))
    c = f.e4m3_encode(x)
    v = f.e4m3_decode(c)
    pos = f.e4m3_decode_table()[:0x7F]
    gaps = np.diff(pos)
    # gap at |x|: the spacing of the interval containing |x|
    idx = np.clip(np.searchsorted(pos, np.abs(x), side="right") - 1, 0, len(gaps) - 1)
    assert np.all(np.abs(x - v) <= gaps[idx] / 2 + 1e-300)
    assert np.all(np.diff(v) >= 0)


def test_quantize_columns_scales_and_exact_grid():
    """Each column's largest magnitude maps to 448 (code 0x7E) and the scales are amax / 448 in fp32; a column
    that already lies on the FP8 grid times a power of two is reproduced exactly; a zero column gets scale 1."""
    f = oracle.fp8
    rng = np.random.default_rng(3)
    W = rng.standard_normal((2, 40, 24)).astype(np.float32) * np.float32(0.02)
    W[1, :, 5] = 0.0
    t = f.e4m3_decode_table()
    grid = t[rng.integers(0, 0x7F, 40)] * 2.0**-12  # FP8 values times 2^-12, exact in fp32
    grid[0] = 448 * 2.0**-12  # make the column's amax a grid value so its scale is exactly 2^-12
    W[0, :, 3] = grid.astype(np.float32)
    codes, s = f.quantize_columns(W)
    assert codes.shape == (2, 24, 40) and codes.dtype == np.uint8 and s.dtype == np.float32
    amax = np.abs(W).max(axis=1)
    exp_s = np.where(amax > 0, amax / np.float32(448), np.float32(1))
    np.testing.assert_array_equal(s, exp_s)
    for e in range(2):
        for n in range(24):
            if amax[e, n] > 0:
                k = np.argmax(np.abs(W[e, :, n]))
                assert codes[e, n, k] & 0x7F == 0x7E
    assert s[1, 5] == 1.0 and (codes[1, 5] == 0).all()
    Wd = f.dequantize_columns(codes, s)
    np.testing.assert_array_equal(Wd[0, :, 3], grid)
    # Relative error per column bounded by the format's half-ulp at the top of the range (2^-4 of amax).
    assert np.all(np.abs(Wd - W) <= amax[:, None, :] * 2.0**-4 * 1.0000001)


def test_forward_fp8_is_the_layer_on_dequantized_weights():
    """With weights already on the scaled FP8 grid the FP8 layer equals the plain layer on those weights, and
    for random weights it stays within the quantisation error of the bf16 layer."""
    f = oracle.fp8
    w = make_layer(20, 32, 16, 4, 2, dtype="f32", seed=6)
    c13, s13 = f.quantize_columns(w.W13_f32)
    c2, s2 = f.quantize_columns(w.W2_f32)
    got = f.forward_fp8(w.x_f32, w.W_gate_f32, c13, s13, c2, s2, w.K, w.renorm)
    W13d, W2d = f.dequantize_columns(c13, s13), f.dequantize_columns(c2, s2)
    ref = oracle.forward(w.x_f32, w.W_gate_f32, W13d, W2d, w.K, w.renorm)
    np.testing.assert_allclose(got["y"], ref["y"], rtol=0, atol=0)
    c13b, s13b = f.quantize_columns(W13d.astype(np.float32))  # quantizing grid values again changes nothing
    np.testing.assert_array_equal(c13b, c13)
    np.testing.assert_array_equal(s13b, s13)
    plain = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, w.K, w.renorm)
    rel = np.linalg.norm(got["y"] - plain["y"]) / np.linalg.norm(plain["y"])
    assert 1e-3 < rel < 0.1


def test_planted_fp8_mistakes_are_caught(monkeypatch):
    f = oracle.fp8
    orig_encode = f.e4m3_encode

    # 1. Ties rounded away from zero instead of to even.
    def encode_ties_away(x):
        x = np.asarray(x, dtype=np.float64)
        c = orig_encode(x).astype(np.int64)
        v = f.e4m3_decode(c)
        nxt = f.e4m3_decode(np.minimum((c & 0x7F) + 1, 0x7E) | (c & 0x80))
        tie = np.abs(np.abs(x) - (np.abs(v) + np.abs(nxt)) / 2) == 0
        return np.where(tie & (np.abs(x) > np.abs(v)), (c & 0x7F) + 1 | (c & 0x80), c).astype(np.uint8)

    monkeypatch.setattr(f, "e4m3_encode", encode_ties_away)
    assert not _pins_pass(test_e4m3_encode_round_trip_ties_and_saturation)
    monkeypatch.undo()

    # 2. Exponent bias 8 in the decode table.
    orig_table = f.e4m3_decode_table

    def table_bias8():
        return orig_table() / 2.0

    monkeypatch.setattr(f, "e4m3_decode_table", table_bias8)
    assert not _pins_pass(test_e4m3_table_landmarks)
    monkeypatch.undo()

    # 3. Scales per input row instead of per output column.
    def quantize_rows(W):
        W32 = np.asarray(W, dtype=np.float32)
        amax = np.max(np.abs(W32), axis=2)
        scale = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
        codes = orig_encode((W32 / scale[:, :, None]).astype(np.float32))
        return np.ascontiguousarray(np.transpose(codes, (0, 2, 1))), scale

    monkeypatch.setattr(f, "quantize_columns", quantize_rows)
    assert not _pins_pass(test_quantize_columns_scales_and_exact_grid)
    monkeypatch.undo()


def test_e4m3_encode_matches_nearest_search():
    """The exponent/mantissa encoder equals the nearest-value search on every code, every midpoint and its two
    neighbours, and random values across the whole range (both signs)."""
    f = oracle.fp8
    t = f.e4m3_decode_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    pts = np.concatenate([t, mids, np.nextafter(mids, -np.inf), np.nextafter(mids, np.inf), [500.0, 1e-12, 0.0]])
    rng = np.random.default_rng(21)
    pts = np.concatenate([pts, rng.uniform(0, 460, 2000), np.abs(rng.normal(0, 0.01, 2000)),
                          2.0 ** rng.uniform(-12, 9, 2000)])
    pts = np.concatenate([pts, -pts]).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(f.e4m3_encode(pts), brute.e4m3_encode_by_search(pts))


# ---------------------------------------------------------------------------
# FP8 activations: per-token scales and the padded FP8 receive buffer
# ---------------------------------------------------------------------------


def test_quantize_rows_per_token_scale_exact_grid_and_search():
    """Per-token FP8: a row on the scaled E4M3 grid with amax 448 * 2^j quantizes exactly (scale 2^j, codes round
    trip); a zero row gets scale 1 and code 0; codes equal the nearest-value search of fp32 x / s; quantizing the
    rows equals quantizing the columns of the transpose; the error stays within half a code gap at the top of the
    range (2^-4 of the row's amax)."""
    f = oracle.fp8
    t = f.e4m3_decode_table()[:0x7F]
    rng = np.random.default_rng(31)
    exact = rng.choice(np.concatenate([t, -t]), size=(6, 40))
    exact[:, 0] = 448.0
    exact *= 2.0 ** np.arange(-3, 3)[:, None]
    codes, s = f.quantize_rows(exact.astype(np.float32))
    np.testing.assert_array_equal(s, (2.0 ** np.arange(-3, 3)).astype(np.float32))
    np.testing.assert_array_equal(f.dequantize_rows(codes, s), exact)
    z_codes, z_s = f.quantize_rows(np.zeros((2, 8), np.float32))
    assert (z_codes == 0).all() and (z_s == 1.0).all()
    X = (rng.standard_normal((30, 64)) * rng.uniform(0.01, 5, (30, 1))).astype(np.float32)
    codes, s = f.quantize_rows(X)
    amax = np.max(np.abs(X), axis=1)
    assert (s == (amax / np.float32(448)).astype(np.float32)).all()
    q = (X / s[:, None]).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(codes, brute.e4m3_encode_by_search(q))
    c_cols, s_cols = f.quantize_columns(X.T[None])  # columns of X^T are the rows of X
    np.testing.assert_array_equal(c_cols[0], codes)
    np.testing.assert_array_equal(s_cols[0], s)
    assert np.all(np.abs(f.dequantize_rows(codes, s) - X) <= amax[:, None] * 2.0**-4 * 1.0000001)


def test_padded_offsets_token_groups():
    """Groups of 16 rows: the worked case counts (3, 0, 16, 17, 1) -> starts (0, 16, 16, 32, 64, 80); every group
    is a multiple of 16, holds its rows, and pads fewer than 16; an empty expert takes no rows."""
    f = oracle.fp8
    np.testing.assert_array_equal(f.padded_offsets([3, 0, 16, 17, 1]), [0, 16, 16, 32, 64, 80])
    rng = np.random.default_rng(5)
    c = rng.integers(0, 70, size=40)
    c[::7] = 0
    P = f.padded_offsets(c)
    g = np.diff(P)
    assert P[0] == 0 and (g % 16 == 0).all() and (g >= c).all() and (g - c < 16).all() and (g[c == 0] == 0).all()


def test_dispatch_fp8_receive_buffer():
    """The FP8 receive buffer: each (token, slot) pair appears once, at its expert's padded group in ascending
    flat order (the unpadded permutation shifted by the group starts); its row holds the token's codes and
    scale; padding rows hold code 0, scale 0 and perm -1; inv and perm are inverse on the real rows."""
    f = oracle.fp8
    w = make_layer(70, 32, 16, 8, 3, dtype="bf16", seed=9)
    L = oracle.round_to_f32(oracle.router_logits(w.x_f32, w.W_gate_f32))
    e_top, _, _ = oracle.route_from_logits(L, w.K, False)
    d = f.dispatch_fp8(w.x_f32, e_top, w.E)
    codes_tok, s_tok = f.quantize_rows(w.x_f32)
    perm, _ = oracle.permutation(e_top, w.E)
    offs = oracle.offsets_from_counts(oracle.expert_counts(e_top, w.E))
    P = d["offsets"]
    assert d["codes"].shape == (P[-1], w.H)
    real = d["perm"] >= 0
    assert real.sum() == w.n * w.K
    for e in range(w.E):
        seg = perm[offs[e] : offs[e + 1]]
        np.testing.assert_array_equal(d["perm"][P[e] : P[e] + seg.size], seg)
        assert (d["perm"][P[e] + seg.size : P[e + 1]] == -1).all()
    np.testing.assert_array_equal(d["perm"][d["inv"]], np.arange(w.n * w.K))
    np.testing.assert_array_equal(d["codes"][real], codes_tok[d["perm"][real] // w.K])
    np.testing.assert_array_equal(d["scales"][real], s_tok[d["perm"][real] // w.K])
    assert (d["codes"][~real] == 0).all() and (d["scales"][~real] == 0).all()


def test_forward_fp8a_exact_activations_and_error():
    """With activations already on each row's scaled FP8 grid, the FP8-activation layer equals the FP8-weight
    layer (no activation quantization error); for random activations it stays within the quantization error."""
    f = oracle.fp8
    w = make_layer(24, 32, 16, 4, 2, dtype="f32", seed=12)
    c13, s13 = f.quantize_columns(w.W13_f32)
    c2, s2 = f.quantize_columns(w.W2_f32)
    t = f.e4m3_decode_table()[:0x7F]
    rng = np.random.default_rng(4)
    xg = rng.choice(np.concatenate([t, -t]), size=(w.n, w.H))
    xg[:, 0] = 448.0
    xg = (xg * 2.0**-9).astype(np.float32)  # scale 2^-9 per row, exact
    a = f.forward_fp8a(xg, w.W_gate_f32, c13, s13, c2, s2, w.K, w.renorm, fp8_h=False)
    b = f.forward_fp8(xg, w.W_gate_f32, c13, s13, c2, s2, w.K, w.renorm)
    np.testing.assert_allclose(a["y"], b["y"], rtol=0, atol=1e-15)
    a = f.forward_fp8a(w.x_f32, w.W_gate_f32, c13, s13, c2, s2, w.K, w.renorm, fp8_h=False)
    b = f.forward_fp8(w.x_f32, w.W_gate_f32, c13, s13, c2, s2, w.K, w.renorm)
    assert (a["e_top"] == b["e_top"]).all()  # routing stays on the unquantized activations
    rel = np.linalg.norm(a["y"] - b["y"]) / np.linalg.norm(b["y"])
    assert 1e-4 < rel < 0.1


def _fp8_h_identity_layer(n=40, I=48, seed=31):
    """E = K = 1 with renormalisation (y = Y exactly) and W2 = (448 * 2^-10) * identity (I = H), whose column
    codes are exactly 448 with scale 2^-10, so y = 0.4375 * (h as the layer quantizes it), exactly in fp64."""
    f = oracle.fp8
    rng = np.random.default_rng(seed)
    H = I
    x = rng.standard_normal((n, H)).astype(np.float32)
    W_gate = rng.standard_normal((H, 1)).astype(np.float32)
    W13 = (0.2 * rng.standard_normal((1, H, 2 * I))).astype(np.float32)
    W2 = (np.eye(I, dtype=np.float32) * np.float32(448 * 2.0**-10))[None]
    c13, s13 = f.quantize_columns(W13)
    c2, s2 = f.quantize_columns(W2)
    assert (s2 == np.float32(2.0**-10)).all() and (f.dequantize_columns(c2, s2) == W2).all()
    q = f.forward_fp8a(x, W_gate, c13, s13, c2, s2, 1, True)["y"] / 0.4375
    h = f.forward_fp8a(x, W_gate, c13, s13, c2, s2, 1, True, fp8_h=False)["y"] / 0.4375
    return q, h


def test_fp8a_intermediate_rows_on_their_scaled_grid():
    """The FP8 h of the layer: every row of the quantized h lies on the E4M3 grid scaled by its own row's
    amax / 448 (the largest element maps to 448), and each element is the nearest grid value of h (within
    half a gap: 2^-4 of its magnitude for normal values, 2^-10 of the row scale below 2^-6)."""
    q, h = _fp8_h_identity_layer()
    grid = oracle.fp8.e4m3_decode_table()[:0x7F]
    grid = np.concatenate([grid, -grid])
    for i in range(q.shape[0]):
        amax = np.max(np.abs(q[i]))
        assert amax > 0
        s = amax / 448.0
        v = q[i] / s
        assert np.isin(v, grid).all(), f"row {i} is not on its own scaled E4M3 grid"
        # half an E4M3 gap of the bf16 value, plus the bf16 rounding itself (2^-9 relative)
        tol = (np.maximum(2.0**-4 * np.abs(h[i]) * (1 + 2.0**-8), 2.0**-10 * s) + 2.0**-9 * np.abs(h[i])) * (1 + 1e-9)
        assert (np.abs(q[i] - h[i]) <= tol).all()
    assert np.abs(q - h).max() > 0  # the quantization happened


def test_round_to_bf16_matches_the_format():
    """round_to_bf16: representable values unchanged, midpoints to the even significand, and equal to torch's
    fp32 -> bfloat16 conversion (round to nearest even) on random fp32 values of every magnitude."""
    import torch

    f = oracle.fp8
    for v in [1.0, -2.5, 0.0, 3.0 * 2.0**-20, 65280.0]:
        assert f.round_to_bf16(v) == v
    assert f.round_to_bf16(1.0 + 2.0**-8) == 1.0  # halfway between 1 and 1 + 2^-7: even
    assert f.round_to_bf16(1.0 + 3 * 2.0**-8) == 1.0 + 2.0**-6
    assert f.round_to_bf16(1.0 + 2.0**-8 + 2.0**-30) == 1.0 + 2.0**-7
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert (f.round_to_bf16(x) == ref).all()


def test_planted_fp8_activation_mistakes_are_caught(monkeypatch):
    f = oracle.fp8
    orig_q, orig_pad, orig_disp = f.quantize_rows, f.padded_offsets, f.dispatch_fp8

    # 1. One scale for the whole matrix instead of one per token.
    def quantize_global(X):
        X32 = np.asarray(X, dtype=np.float32)
        s = np.float32(np.max(np.abs(X32)) / np.float32(448))
        return f.e4m3_encode((X32 / s).astype(np.float32)), np.full(X32.shape[0], s, np.float32)

    monkeypatch.setattr(f, "quantize_rows", quantize_global)
    assert not _pins_pass(test_quantize_rows_per_token_scale_exact_grid_and_search)
    monkeypatch.undo()

    # 1b. h quantized with one scale per column instead of one per row, and h not quantized at all.
    def round_cols(X):
        X32 = np.asarray(X, dtype=np.float32)
        s = np.max(np.abs(X32), axis=0) / np.float32(448)
        s = np.where(s > 0, s, np.float32(1)).astype(np.float32)
        return f.e4m3_decode(f.e4m3_encode((X32 / s[None, :]).astype(np.float32))) * s[None, :].astype(np.float64)

    monkeypatch.setattr(f, "fp8_round_rows", round_cols)
    assert not _pins_pass(test_fp8a_intermediate_rows_on_their_scaled_grid)
    monkeypatch.setattr(f, "fp8_round_rows", lambda X: np.asarray(X, dtype=np.float64))
    assert not _pins_pass(test_fp8a_intermediate_rows_on_their_scaled_grid)
    monkeypatch.undo()

    # 2. Groups padded to 8 rows.
    monkeypatch.setattr(f, "padded_offsets", lambda c, group=8: orig_pad(c, 8))
    assert not _pins_pass(test_padded_offsets_token_groups)
    monkeypatch.undo()

    # 3. Padding rows given scale 1.
    def dispatch_pad_scale_one(x, e_top, E, group=16):
        d = orig_disp(x, e_top, E, group)
        d["scales"] = np.where(d["perm"] < 0, np.float32(1), d["scales"]).astype(np.float32)
        return d

    monkeypatch.setattr(f, "dispatch_fp8", dispatch_pad_scale_one)
    assert not _pins_pass(test_dispatch_fp8_receive_buffer)
    monkeypatch.undo()
    assert f.quantize_rows is orig_q
