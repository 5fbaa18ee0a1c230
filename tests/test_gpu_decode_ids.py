"""The decode-sized GEMM1 that places the routing ids itself
(moe_expert_w13_swiglu_from_ids, and its FP8 x FP8 form
moe_expert_w13_swiglu_from_ids_fp8a), and the layers that run it in place of
the permute launch (moe_forward and moe_forward_fp8a at n <= 32).

Its metadata (counts, offsets, splits, perm, inv) must equal the oracle's
expert-major placement bit for bit; h must equal, bit for bit, what
moe_permute + moe_expert_w13_swiglu_gather give on the same ids (the same
tile arithmetic), and stay within the bf16 bounds of the oracle's gate/up
product. The layer must give the same bits as the staged calls.
"""

import numpy as np
import pytest
import torch

import oracle
import routing_token_permute_amd as moe
from gpu_util import assert_close, dev_tensor, layer_tensors, require_gpu, to_f64
from oracle import moe_oracle as om
from workloads import make_layer, zipf_bias

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _ids(n, E, K, kind, seed):
    """Routing ids from seeded random logits (K distinct experts per token); "skewed" adds the Zipf
    bias so that hot experts take up to n rows; "invalid" then puts ids outside [0, E) in some slots."""
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((n, E)).astype(np.float32)
    if kind == "skewed":
        L = L + zipf_bias(E)
    e_top, _, _ = oracle.route_from_logits(L, K, renorm=False)
    e_top = e_top.astype(np.int64)
    if kind == "invalid":
        flat = e_top.reshape(-1)
        flat[::5] = -1
        flat[3::7] = E
    return e_top


def _placement(e_top, E, ep):
    """Expected metadata: the oracle's on all-valid ids; with ids outside [0, E), the same placement of
    the valid pairs (the others are neither counted nor placed)."""
    flat = e_top.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    if valid.all():
        counts = oracle.expert_counts(e_top, E)
        perm, inv = oracle.permutation(e_top, E)
        splits = oracle.splits_by_rank(e_top, E, ep)
    else:
        counts = np.bincount(flat[valid], minlength=E)
        perm = np.flatnonzero(valid)[np.argsort(flat[valid], kind="stable")]
        inv = np.full(flat.size, -1, dtype=np.int64)
        inv[perm] = np.arange(perm.size)
        El = E // ep
        splits = np.array([counts[j * El:(j + 1) * El].sum() for j in range(ep)])
    return dict(counts=counts, offsets=oracle.offsets_from_counts(counts), splits=splits, perm=perm, inv=inv,
                valid=valid)


CASES = [
    # n, H, I, E, K, ep, kind
    (1, 128, 128, 8, 2, 1, "routed"),
    (5, 256, 128, 16, 4, 2, "routed"),
    (17, 128, 256, 64, 8, 4, "routed"),
    (32, 2048, 1024, 64, 8, 1, "routed"),  # the OLMoE decode batch
    (32, 256, 128, 64, 8, 1, "skewed"),  # hot experts with all 32 rows
    (32, 128, 128, 256, 32, 8, "routed"),  # 1024 pairs over 256 experts
    (31, 128, 128, 128, 33, 1, "routed"),  # 1023 pairs
    (32, 128, 128, 64, 1, 1, "routed"),
    (24, 128, 128, 64, 8, 1, "invalid"),
    (5, 128, 128, 1, 1, 1, "routed"),  # one expert: every pair in one tile
    (7, 64, 64, 2, 2, 2, "routed"),  # every token picks both experts; a single 64-deep k-step
    (32, 128, 192, 4, 4, 1, "routed"),  # K = E: all 32 tokens in every expert; a masked column tail
]


@pytest.mark.parametrize("n,H,I,E,K,ep,kind", CASES)
def test_w13_from_ids(dev, n, H, I, E, K, ep, kind):  # noqa: E741
    what = f"w13_from_ids n={n} E={E} K={K} ep={ep} {kind}"
    print(f"[{what}]", flush=True)
    e_top = _ids(n, E, K, kind, seed=n * 131 + E)
    ref = _placement(e_top, E, ep)
    w = make_layer(n, H, I, E, K, seed=n + H + E)
    t = layer_tensors(w, dev)
    ids_d = torch.from_numpy(e_top.astype(np.int32)).to(dev)
    h, meta = moe.moe_expert_w13_swiglu_from_ids(t["x"], ids_d, t["W13"], ep)
    torch.cuda.synchronize()
    for k in ("counts", "offsets", "splits", "perm"):
        got = meta[k].cpu().numpy()
        exp = ref[k] if k != "perm" else ref["perm"]
        m = int(ref["offsets"][-1]) if k == "perm" else got.size
        assert (got[:m] == exp[:m]).all(), f"{what}: {k} differ"
    inv = meta["inv"].cpu().numpy()
    assert (inv[ref["valid"]] == ref["inv"][ref["valid"]]).all(), f"{what}: inv differs"
    rows = int(ref["offsets"][-1])
    # The same h as the permute + gathered GEMM1 on the oracle's placement, bit for bit.
    off_d = torch.from_numpy(ref["offsets"].astype(np.int32)).to(dev)
    perm_full = np.zeros(n * K, dtype=np.int32)
    perm_full[:rows] = ref["perm"][:rows]
    h2 = moe.moe_expert_w13_swiglu_gather(t["x"], torch.from_numpy(perm_full).to(dev), K, off_d, t["W13"])
    torch.cuda.synchronize()
    assert torch.equal(h[:rows].view(torch.int16), h2[:rows].view(torch.int16)), f"{what}: h differs"
    ref_h = om.grouped_gate_up(w.x_f32[ref["perm"][:rows] // K], ref["offsets"], w.W13_f32)
    assert_close(to_f64(h[:rows]), ref_h, "bf16", what, intermediate=True)


def test_w13_from_ids_zero_tokens(dev):
    w = make_layer(1, 128, 128, 16, 2, seed=3)
    t = layer_tensors(w, dev)
    x0 = t["x"][:0]
    meta = {k: torch.full(s, 7, dtype=torch.int32, device=dev)
            for k, s in (("counts", (16,)), ("offsets", (17,)), ("splits", (2,)), ("perm", (0,)), ("inv", (0,)))}
    h, meta = moe.moe_expert_w13_swiglu_from_ids(x0, torch.zeros((0, 2), dtype=torch.int32, device=dev), t["W13"], 2,
                                                 out=meta)
    torch.cuda.synchronize()
    assert h.shape == (0, 128)
    for k in ("counts", "offsets", "splits"):
        assert (meta[k].cpu() == 0).all()


@pytest.mark.parametrize("n,H,I,E,K,renorm,bias", [(1, 128, 128, 8, 2, False, None), (7, 256, 128, 64, 8, True, None),
                                                  (32, 2048, 1024, 64, 8, False, "zipf"),
                                                  (32, 128, 128, 256, 32, True, None)])
def test_forward_decode_matches_staged_calls(dev, n, H, I, E, K, renorm, bias):  # noqa: E741
    """moe_forward at n <= 32 (GEMM1 places the ids itself) gives the bits of the staged calls:
    moe_route, moe_permute, moe_expert_w13_swiglu_gather, moe_expert_w2, moe_unpermute_combine."""
    what = f"forward from ids n={n} E={E} K={K}"
    print(f"[{what}]", flush=True)
    w = make_layer(n, H, I, E, K, dtype="bf16", renorm=renorm, seed=n * 7 + E)
    t = layer_tensors(w, dev)
    b = torch.from_numpy(zipf_bias(E).astype(np.float32)).to(dev) if bias == "zipf" else None
    y, logits, ids, wts, counts = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], K, renorm, bias=b,
                                                  routing_out=True)
    _, ids2, wts2 = moe.moe_route(t["x"], t["W_gate"], b, K, renorm)
    meta = moe.moe_permute(ids2, None, E)
    h = moe.moe_expert_w13_swiglu_gather(t["x"], meta["perm"], K, meta["offsets"], t["W13"])
    Y = moe.moe_expert_w2(h, meta["offsets"], t["W2"])
    y2 = moe.moe_unpermute_combine(Y, meta["inv"], wts2, n, K)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(counts, meta["counts"])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"{what}: y differs from the staged calls"
    L = logits.cpu().numpy()
    ref = oracle.forward(w.x_f32, w.W_gate_f32, w.W13_f32, w.W2_f32, K, renorm,
                         bias=None if b is None else b.cpu().numpy(), routing_logits_f32=L)
    assert (ids.cpu().numpy() == ref["e_top"]).all()
    assert_close(to_f64(y), ref["y"], "bf16", what)


FP8_CASES = [
    # n, H, I, E, K, ep, kind
    (1, 128, 128, 8, 2, 1, "routed"),
    (17, 256, 128, 64, 8, 4, "routed"),
    (32, 2048, 1024, 64, 8, 1, "routed"),  # the OLMoE decode batch
    (32, 128, 128, 256, 32, 8, "routed"),  # 1024 pairs over 256 experts
    (24, 128, 128, 64, 8, 1, "invalid"),
    (5, 128, 128, 1, 1, 1, "routed"),
    (32, 128, 256, 4, 4, 2, "routed"),  # K = E: all 32 tokens in every expert
]


@pytest.mark.parametrize("n,H,I,E,K,ep,kind", FP8_CASES)
def test_w13_from_ids_fp8a(dev, n, H, I, E, K, ep, kind):  # noqa: E741
    """The FP8 x FP8 GEMM1 from the ids: metadata bit-exact against the oracle's placement, h bit for bit
    the in-place FP8 GEMM1's on that placement, and within the bf16 bounds of the oracle's product of the
    dequantized token rows and weight columns."""
    from oracle import fp8 as of8

    what = f"w13_from_ids_fp8a n={n} E={E} K={K} ep={ep} {kind}"
    print(f"[{what}]", flush=True)
    e_top = _ids(n, E, K, kind, seed=n * 137 + E)
    ref = _placement(e_top, E, ep)
    w = make_layer(n, H, I, E, K, seed=n + 3 * H + E)
    t = layer_tensors(w, dev)
    q13, s13 = moe.moe_quantize_fp8(t["W13"])
    codes_tok, s_tok = moe.moe_quantize_rows_fp8(t["x"])
    ids_d = torch.from_numpy(e_top.astype(np.int32)).to(dev)
    h, meta = moe.moe_expert_w13_swiglu_from_ids_fp8a(codes_tok, s_tok, ids_d, q13, s13, ep)
    torch.cuda.synchronize()
    rows = int(ref["offsets"][-1])
    for k in ("counts", "offsets", "splits"):
        assert (meta[k].cpu().numpy() == ref[k]).all(), f"{what}: {k} differ"
    assert (meta["perm"].cpu().numpy()[:rows] == ref["perm"][:rows]).all(), f"{what}: perm differs"
    assert (meta["inv"].cpu().numpy()[ref["valid"]] == ref["inv"][ref["valid"]]).all(), f"{what}: inv differs"
    perm_full = np.zeros(n * K, dtype=np.int32)
    perm_full[:rows] = ref["perm"][:rows]
    h2 = moe.moe_expert_w13_swiglu_gather_fp8a(codes_tok, s_tok, torch.from_numpy(perm_full).to(dev), K,
                                              torch.from_numpy(ref["offsets"].astype(np.int32)).to(dev), q13, s13)
    torch.cuda.synchronize()
    assert torch.equal(h[:rows].view(torch.int16), h2[:rows].view(torch.int16)), f"{what}: h differs"
    ct, st = of8.quantize_rows(w.x_f32)
    c13, r13 = of8.quantize_columns(w.W13_f32)
    ref_h = om.grouped_gate_up(of8.dequantize_rows(ct, st)[ref["perm"][:rows] // K], ref["offsets"],
                               of8.dequantize_columns(c13, r13))
    assert_close(to_f64(h[:rows]), ref_h, "bf16", what, intermediate=True)


@pytest.mark.parametrize("n,H,I,E,K,renorm", [(7, 256, 128, 64, 8, True), (32, 2048, 1024, 64, 8, False)])
def test_forward_fp8a_decode_matches_staged_calls(dev, n, H, I, E, K, renorm):  # noqa: E741
    """moe_forward_fp8a at n <= 32 (the FP8 GEMM1 places the ids itself) gives the bits of the staged
    calls: route, permute, token quantization, in-place FP8 GEMM1, h quantization, FP8 GEMM2, combine."""
    what = f"forward fp8a from ids n={n} E={E} K={K}"
    print(f"[{what}]", flush=True)
    w = make_layer(n, H, I, E, K, dtype="bf16", renorm=renorm, seed=n * 11 + E)
    t = layer_tensors(w, dev)
    q13, s13 = moe.moe_quantize_fp8(t["W13"])
    q2, s2 = moe.moe_quantize_fp8(t["W2"])
    y, logits, ids, wts, counts = moe.moe_forward_fp8a(t["x"], t["W_gate"], q13, s13, q2, s2, K, renorm,
                                                       routing_out=True)
    _, ids2, wts2 = moe.moe_route(t["x"], t["W_gate"], None, K, renorm)
    meta = moe.moe_permute(ids2, None, E)
    codes_tok, s_tok = moe.moe_quantize_rows_fp8(t["x"])
    h = moe.moe_expert_w13_swiglu_gather_fp8a(codes_tok, s_tok, meta["perm"], K, meta["offsets"], q13, s13)
    hq, hs = moe.moe_quantize_rows_fp8(h)
    Y = moe.moe_expert_w2_fp8a(hq, hs, meta["offsets"], q2, s2)
    y2 = moe.moe_unpermute_combine(Y, meta["inv"], wts2, n, K)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(counts, meta["counts"])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"{what}: y differs from the staged calls"


W8_CASES = [
    # n, H, I, E, K, ep, kind
    (3, 128, 128, 8, 2, 1, "routed"),
    (32, 2048, 1024, 64, 8, 1, "routed"),  # the OLMoE decode batch
    (32, 128, 128, 256, 32, 4, "routed"),  # 1024 pairs over 256 experts
    (24, 128, 192, 64, 8, 1, "invalid"),  # a masked column tail
]


@pytest.mark.parametrize("n,H,I,E,K,ep,kind", W8_CASES)
def test_w13_from_ids_fp8_weights(dev, n, H, I, E, K, ep, kind):  # noqa: E741
    """GEMM1 with FP8 weights from the ids: metadata bit-exact against the oracle's placement, h bit for bit
    the gathered FP8-weight GEMM1's on that placement, and within the bf16 bounds of the oracle's product
    with the dequantized weight columns."""
    from oracle import fp8 as of8

    what = f"w13_from_ids_fp8 n={n} E={E} K={K} ep={ep} {kind}"
    print(f"[{what}]", flush=True)
    e_top = _ids(n, E, K, kind, seed=n * 139 + E)
    ref = _placement(e_top, E, ep)
    w = make_layer(n, H, I, E, K, seed=n + 5 * H + E)
    t = layer_tensors(w, dev)
    q13, s13 = moe.moe_quantize_fp8(t["W13"])
    ids_d = torch.from_numpy(e_top.astype(np.int32)).to(dev)
    h, meta = moe.moe_expert_w13_swiglu_from_ids_fp8(t["x"], ids_d, q13, s13, ep)
    torch.cuda.synchronize()
    rows = int(ref["offsets"][-1])
    for k in ("counts", "offsets", "splits"):
        assert (meta[k].cpu().numpy() == ref[k]).all(), f"{what}: {k} differ"
    assert (meta["perm"].cpu().numpy()[:rows] == ref["perm"][:rows]).all(), f"{what}: perm differs"
    assert (meta["inv"].cpu().numpy()[ref["valid"]] == ref["inv"][ref["valid"]]).all(), f"{what}: inv differs"
    perm_full = np.zeros(n * K, dtype=np.int32)
    perm_full[:rows] = ref["perm"][:rows]
    h2 = moe.moe_expert_w13_swiglu_gather_fp8(t["x"], torch.from_numpy(perm_full).to(dev), K,
                                             torch.from_numpy(ref["offsets"].astype(np.int32)).to(dev), q13, s13)
    torch.cuda.synchronize()
    assert torch.equal(h[:rows].view(torch.int16), h2[:rows].view(torch.int16)), f"{what}: h differs"
    c13, r13 = of8.quantize_columns(w.W13_f32)
    ref_h = om.grouped_gate_up(w.x_f32[ref["perm"][:rows] // K], ref["offsets"], of8.dequantize_columns(c13, r13))
    assert_close(to_f64(h[:rows]), ref_h, "bf16", what, intermediate=True)


@pytest.mark.parametrize("n,H,I,E,K,renorm", [(9, 256, 128, 16, 4, True), (32, 2048, 1024, 64, 8, False)])
def test_forward_fp8_decode_matches_staged_calls(dev, n, H, I, E, K, renorm):  # noqa: E741
    """moe_forward_fp8 at n <= 32 (the FP8-weight GEMM1 places the ids itself) gives the bits of the staged
    calls: route, permute, gathered FP8-weight GEMM1, FP8-weight GEMM2, combine."""
    what = f"forward fp8 from ids n={n} E={E} K={K}"
    print(f"[{what}]", flush=True)
    w = make_layer(n, H, I, E, K, dtype="bf16", renorm=renorm, seed=n * 13 + E)
    t = layer_tensors(w, dev)
    q13, s13 = moe.moe_quantize_fp8(t["W13"])
    q2, s2 = moe.moe_quantize_fp8(t["W2"])
    y, logits, ids, wts, counts = moe.moe_forward_fp8(t["x"], t["W_gate"], q13, s13, q2, s2, K, renorm,
                                                      routing_out=True)
    _, ids2, wts2 = moe.moe_route(t["x"], t["W_gate"], None, K, renorm)
    meta = moe.moe_permute(ids2, None, E)
    h = moe.moe_expert_w13_swiglu_gather_fp8(t["x"], meta["perm"], K, meta["offsets"], q13, s13)
    Y = moe.moe_expert_w2_fp8(h, meta["offsets"], q2, s2)
    y2 = moe.moe_unpermute_combine(Y, meta["inv"], wts2, n, K)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(counts, meta["counts"])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"{what}: y differs from the staged calls"
