"""The expert GEMMs write their tiles and nothing else.

The epilogue stores every tile through a buffer resource that spans only the
tile's rows; lanes without a valid output (rows past a short tile, columns past
a masked tail, 16-row slices a tile does not fill) carry an out-of-range offset
that the hardware drops. Here each output is a view into a larger buffer with
guard rows on both sides, all pre-filled with a sentinel bit pattern: the guard
rows must keep the sentinel, and the view must hold bitwise what a call into a
fresh buffer returns (no row left unwritten, none written twice with different
values). Routing comes from the oracle's permutation of seeded top-K ids, so
some experts are empty and most end in a short tile.
"""

import numpy as np
import pytest
import torch

import oracle
import routing_token_permute_amd as moe
from gpu_util import dev_tensor, layer_tensors, require_gpu
from workloads import make_layer, random_bf16_matrix

pytestmark = pytest.mark.gpu

GUARD = 40  # rows of sentinel before and after each output view
SENTINEL = -12345  # int16 bit pattern of a bf16 NaN-free value never produced here


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _guarded(rows, cols, dev):
    buf = torch.full((rows + 2 * GUARD, cols), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    return buf, buf[GUARD:GUARD + rows]


def _check_guards(buf, rows, what):
    bits = buf.view(torch.int16)
    assert bool((bits[:GUARD] == SENTINEL).all()), f"{what}: a store landed before the output"
    assert bool((bits[GUARD + rows:] == SENTINEL).all()), f"{what}: a store landed after the output"


def _routing(n, E, K, seed):
    """Seeded top-K ids with a skew (a quarter of the experts never chosen)."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((n, E)).astype(np.float32)
    logits[:, : E // 4] -= 1e4
    e_top = np.argsort(-logits, axis=1, kind="stable")[:, :K].astype(np.int64)
    counts = oracle.expert_counts(e_top, E)
    return oracle.offsets_from_counts(counts), oracle.permutation(e_top, E)[0]


# n, H, I, E, K: the 32-row tile configuration (rows / E <= 64) and the 256-row
# one, each with I and H that leave a masked column tail (I % 128 = 64 for
# GEMM1, H % 256 = 192 for GEMM2).
# The last two have more tiles than an MI355X has compute units (256), so
# workgroups go on to further tiles and their first k-steps wait behind the
# previous tile's counted stores.
CASES = [(100, 192, 192, 16, 4), (700, 448, 192, 8, 2), (1300, 192, 320, 12, 3),
         (512, 704, 320, 64, 8), (2048, 704, 320, 64, 8)]


@pytest.mark.parametrize("n,H,I,E,K", CASES)
def test_expert_gemm_stores_stay_in_their_rows(dev, n, H, I, E, K):  # noqa: E741
    w = make_layer(n, H, I, E, K, seed=n + H + I)
    t = layer_tensors(w, dev)
    offsets, perm = _routing(n, E, K, seed=n)
    off_d = torch.from_numpy(offsets.astype(np.int32)).to(dev)
    perm_d = torch.from_numpy(perm.astype(np.int32)).to(dev)
    rows = n * K

    h_ref = moe.moe_expert_w13_swiglu_gather(t["x"], perm_d, K, off_d, t["W13"])
    buf_h, h = _guarded(rows, I, dev)
    moe.moe_expert_w13_swiglu_gather(t["x"], perm_d, K, off_d, t["W13"], h=h)

    h_tr_ref, gu_ref = moe.moe_expert_w13_swiglu_gather_train(t["x"], perm_d, K, off_d, t["W13"])
    buf_h2, h2 = _guarded(rows, I, dev)
    buf_gu, gu = _guarded(rows, 2 * I, dev)
    moe.moe_expert_w13_swiglu_gather_train(t["x"], perm_d, K, off_d, t["W13"], h=h2, gate_up=gu)

    hb, _ = random_bf16_matrix(np.random.default_rng(n + 1), (rows, I), std=0.3)
    h_in = dev_tensor(hb, "bf16", dev)
    Y_ref = moe.moe_expert_w2(h_in, off_d, t["W2"])
    buf_Y, Y = _guarded(rows, H, dev)
    moe.moe_expert_w2(h_in, off_d, t["W2"], Y_perm=Y)
    torch.cuda.synchronize()

    for buf, view, ref, what in ((buf_h, h, h_ref, "GEMM1 h"), (buf_h2, h2, h_tr_ref, "GEMM1 (train) h"),
                                 (buf_gu, gu, gu_ref, "GEMM1 (train) gate_up"), (buf_Y, Y, Y_ref, "GEMM2 Y_perm")):
        _check_guards(buf, view.shape[0], what)
        assert torch.equal(view.view(torch.int16), ref.view(torch.int16)), f"{what}: differs from a fresh buffer"
        assert not bool((view.view(torch.int16) == SENTINEL).all(dim=1).any()), f"{what}: a row was left unwritten"
