"""Packed expert weights (moe_pack_w13, moe_pack_w2) and the layer over them
(moe_forward_packed).

The pack is a pure rearrangement of the weights' bits: its output must equal,
bit for bit, the layout written out below from its definition (per expert and
32 rows of K, one unit of 256 columns x 32 k-values per 256-column output
block, each column's four 16-byte k-chunks at slot chunk ^ ((column / 2) % 4);
GEMM1's blocks 128 gate columns then the matching 128 up columns; zeros past
the matrix). The layer over packed weights runs the same tile arithmetic in the
same order as moe_forward, so every output must equal moe_forward's bit for
bit (moe_forward itself is held to the oracle elsewhere).
"""

import numpy as np
import pytest
import torch

import routing_token_permute_amd as moe
from gpu_util import layer_tensors, require_gpu
from workloads import make_config, make_layer, zipf_bias

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _block_columns(N, half):
    """Source column of each (block, packed column); -1 past the matrix."""
    if half:
        NB = -(-half // 128)
        cols = np.full((NB, 256), -1, dtype=np.int64)
        for nb in range(NB):
            j = nb * 128 + np.arange(128)
            ok = j < half
            cols[nb, :128][ok] = j[ok]
            cols[nb, 128:][ok] = half + j[ok]
    else:
        NB = -(-N // 256)
        c = np.arange(NB * 256).reshape(NB, 256)
        cols = np.where(c < N, c, -1)
    return cols


def _pack_reference(W, half):
    """The packed layout, written out: W (E, Kdim, N) uint16 bits."""
    E, Kdim, N = W.shape
    cols = _block_columns(N, half)
    NB = cols.shape[0]
    out = np.zeros((E, Kdim // 32, NB, 256, 32), dtype=np.uint16)
    chunks = W.reshape(E, Kdim // 32, 4, 8, N)  # (e, unit, chunk q, value, column)
    for nb in range(NB):
        for c in range(256):
            col = cols[nb, c]
            if col < 0:
                continue
            for q in range(4):
                slot = q ^ ((c >> 1) & 3)
                out[:, :, nb, c, 8 * slot:8 * slot + 8] = chunks[:, :, q, :, col]
    return out


def _bits(rng, shape, dev):
    a = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    return a, torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)


@pytest.mark.parametrize("E,H,I", [(3, 128, 192), (2, 320, 64), (5, 64, 128), (8, 2048, 1024)])
def test_pack_layout(dev, E, H, I):  # noqa: E741
    """Any 16-bit patterns (NaN and infinity codes included) land at the documented places, bit for bit."""
    rng = np.random.default_rng(E * 1000 + H + I)
    w13, W13 = _bits(rng, (E, H, 2 * I), dev)
    w2, W2 = _bits(rng, (E, I, H), dev)
    p13 = moe.moe_pack_w13(W13)
    p2 = moe.moe_pack_w2(W2)
    torch.cuda.synchronize()
    got13 = p13.view(torch.int16).cpu().numpy().view(np.uint16)
    got2 = p2.view(torch.int16).cpu().numpy().view(np.uint16)
    assert (got13 == _pack_reference(w13, I)).all()
    assert (got2 == _pack_reference(w2, 0)).all()


def _forward_both(dev, w):
    t = layer_tensors(w, dev)
    W13p, W2p = moe.moe_pack_w13(t["W13"]), moe.moe_pack_w2(t["W2"])
    plain = moe.moe_forward(t["x"], t["W_gate"], t["W13"], t["W2"], w.K, w.renorm, bias=t["bias"], routing_out=True)
    packed = moe.moe_forward_packed(t["x"], t["W_gate"], W13p, W2p, w.K, w.renorm, bias=t["bias"],
                                    routing_out=True)
    torch.cuda.synchronize()
    return plain, packed


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


@pytest.mark.parametrize("name", ["olmoe_bf16", "olmoe_skewed_bf16", "decode_bf16"])
def test_forward_packed_matches_forward(dev, name):
    """The OLMoE layer (256-row tiles), its skewed form (empty and hot experts) and the decode batch (GEMM1
    from the routing ids, 32-row tiles): y, logits, ids, weights and counts bit for bit."""
    plain, packed = _forward_both(dev, make_config(name))
    for what, a, b in zip(("y", "logits", "topk_ids", "topk_w", "counts"), plain, packed):
        assert _same(a, b), f"{name}: {what} differ"


@pytest.mark.parametrize("n,H,I,E,K,skewed", [
    (300, 128, 192, 8, 2, False),   # I = 192: GEMM1's second column block half empty
    (45, 256, 192, 32, 4, True),
    (700, 320, 128, 16, 4, False),  # H = 320: five 64-deep GEMM1 k-steps, GEMM2's second block ragged
    (1, 64, 64, 8, 2, False),
    (2000, 64, 64, 64, 8, True),    # 32-row and 256-row tiles side by side
    (256, 7168, 2048, 8, 2, False),  # wide: 224 K-units per expert for GEMM1, 28 column blocks for GEMM2
])
def test_forward_packed_ragged_shapes(dev, n, H, I, E, K, skewed):  # noqa: E741
    w = make_layer(n, H, I, E, K, seed=n + H + I + E, bias=zipf_bias(E) if skewed else None)
    plain, packed = _forward_both(dev, w)
    for what, a, b in zip(("y", "logits", "topk_ids", "topk_w", "counts"), plain, packed):
        assert _same(a, b), f"n={n} H={H} I={I} E={E} K={K}: {what} differ"


def test_forward_packed_events_and_zero_tokens(dev):
    """The optional events bracket GEMM1 (positive elapsed time within the layer's); n = 0 writes zero
    counts and nothing else."""
    w = make_config("olmoe_bf16")
    t = layer_tensors(w, dev)
    W13p, W2p = moe.moe_pack_w13(t["W13"]), moe.moe_pack_w2(t["W2"])
    b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.record()
    e.record()
    s0.record()
    moe.moe_forward_packed(t["x"], t["W_gate"], W13p, W2p, w.K, w.renorm, gemm1_begin=b, gemm1_end=e)
    s1.record()
    torch.cuda.synchronize()
    g1, whole = b.elapsed_time(e), s0.elapsed_time(s1)
    assert 0 < g1 < whole
    y, logits, ids, wts, counts = moe.moe_forward_packed(t["x"][:0], t["W_gate"], W13p, W2p, w.K, w.renorm,
                                                         routing_out=True)
    torch.cuda.synchronize()
    assert y.shape == (0, w.H) and (counts.cpu() == 0).all()


@pytest.mark.parametrize("n,H,I,E,K", [(4096, 2048, 1024, 64, 8), (300, 128, 192, 8, 2), (700, 320, 128, 16, 4)])
def test_staged_packed_gemms_match_plain(dev, n, H, I, E, K):  # noqa: E741
    """The gathered GEMM1 and GEMM2 over packed weights give the plain-layout calls' h and Y_perm bit for bit."""
    w = make_layer(n, H, I, E, K, seed=3 * n + E)
    t = layer_tensors(w, dev)
    logits, ids, wts = moe.moe_route(t["x"], t["W_gate"], None, K, False)
    meta = moe.moe_permute(ids, None, E)
    W13p, W2p = moe.moe_pack_w13(t["W13"]), moe.moe_pack_w2(t["W2"])
    h = moe.moe_expert_w13_swiglu_gather(t["x"], meta["perm"], K, meta["offsets"], t["W13"])
    hp = moe.moe_expert_w13_swiglu_gather_packed(t["x"], meta["perm"], K, meta["offsets"], W13p, I)
    Y = moe.moe_expert_w2(h, meta["offsets"], t["W2"])
    Yp = moe.moe_expert_w2_packed(h, meta["offsets"], W2p, H)
    torch.cuda.synchronize()
    assert _same(h, hp) and _same(Y, Yp)


@pytest.mark.parametrize("n,E,K", [(32, 64, 8), (7, 16, 4), (1, 8, 1)])
def test_from_ids_packed_matches_plain(dev, n, E, K):
    """The decode GEMM1 that places the ids itself, over packed weights: h and all metadata bit for bit."""
    w = make_layer(n, 256, 192, E, K, seed=n + E + K)
    t = layer_tensors(w, dev)
    _, ids, _ = moe.moe_route(t["x"], t["W_gate"], None, K, False)
    W13p = moe.moe_pack_w13(t["W13"])
    h, meta = moe.moe_expert_w13_swiglu_from_ids(t["x"], ids, t["W13"])
    hp, metap = moe.moe_expert_w13_swiglu_from_ids_packed(t["x"], ids, W13p, w.I)
    torch.cuda.synchronize()
    assert _same(h, hp)
    for k in ("counts", "offsets", "splits", "perm", "inv"):
        assert torch.equal(meta[k], metap[k]), k
