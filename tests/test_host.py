"""Host-side checks of the C-ABI library: it loads, exports every function
include/moe.h declares, and rejects bad arguments before touching the GPU.
No call here reaches a kernel launch."""

import ctypes
import os
import re

import pytest

import routing_token_permute_amd as moe
from routing_token_permute_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

EINVAL, EUNSUP, EWS = 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from routing_token_permute_amd import build

        build.build()
    return moe.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for fn in ("moe_route", "moe_permute", "moe_grouped_swiglu", "moe_unpermute_combine", "moe_forward"):
        assert fn in names


def test_library_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert names
    for name in names:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks {name}"


def test_status_strings(lib):
    for code in range(5):
        s = moe.status_string(code)
        assert s.startswith("MOE_")
    assert "unknown" in moe.status_string(99)
    assert lib.moe_version() >= 100


def test_workspace_sizes(lib):
    a = lib.moe_forward_workspace_size(4096, 2048, 1024, 64, 8, 1)
    b = lib.moe_forward_workspace_size(32, 2048, 1024, 64, 8, 1)
    assert a > b > 0
    # h and Y_perm dominate: nK * (H + I) * 2 bytes (GEMM1 gathers x itself)
    assert a >= 4096 * 8 * (2048 + 1024) * 2
    assert lib.moe_permute_workspace_size(4096, 64, 8) >= 16 * 64 * 4
    assert lib.moe_grouped_swiglu_workspace_size(32768, 1024, 1) >= 32768 * 1024 * 2
    assert lib.moe_forward_workspace_size(-1, 2048, 1024, 64, 8, 1) == 0


P = ctypes.c_void_p(16)  # a non-null dummy; validation rejects before it is used


def test_route_rejects_bad_arguments(lib):
    s = None
    # K > E
    assert lib.moe_route(P, P, None, 8, 64, 4, 5, 0, 1, P, P, P, s) == EINVAL
    # E too large
    assert lib.moe_route(P, P, None, 8, 64, 257, 2, 0, 1, P, P, P, s) == EINVAL
    # bf16 hidden size not a multiple of 64
    assert lib.moe_route(P, P, None, 8, 96, 8, 2, 0, 1, P, P, P, s) == EINVAL
    # null outputs
    assert lib.moe_route(P, P, None, 8, 64, 8, 2, 0, 1, None, P, P, s) == EINVAL
    # unknown dtype
    assert lib.moe_route(P, P, None, 8, 64, 8, 2, 0, 7, P, P, P, s) == EUNSUP
    # negative n
    assert lib.moe_route(P, P, None, -1, 64, 8, 2, 0, 1, P, P, P, s) == EINVAL


def test_permute_rejects_bad_arguments(lib):
    s = None
    ws_ok = lib.moe_permute_workspace_size(100, 8, 2)
    # ep does not divide E
    assert lib.moe_permute(P, None, 100, 64, 8, 2, 3, 1, P, P, P, P, P, None, P, ws_ok, s) == EINVAL
    # workspace too small
    assert lib.moe_permute(P, None, 100, 64, 8, 2, 1, 1, P, P, P, P, P, None, P, 0, s) == EWS
    # x given without x_perm
    assert lib.moe_permute(P, P, 100, 64, 8, 2, 1, 1, P, P, P, P, P, None, P, ws_ok, s) == EINVAL
    # null counts
    assert lib.moe_permute(P, None, 100, 64, 8, 2, 1, 1, None, P, P, P, P, None, P, ws_ok, s) == EINVAL


def test_grouped_and_combine_reject_bad_arguments(lib):
    s = None
    # I not a multiple of 64 for bf16
    assert lib.moe_grouped_swiglu(P, P, 10, P, P, 4, 64, 48, 1, P, P, 1 << 20, s) == EINVAL
    # workspace too small
    assert lib.moe_grouped_swiglu(P, P, 10, P, P, 4, 64, 64, 1, P, P, 16, s) == EWS
    # K too large
    assert lib.moe_unpermute_combine(P, P, None, 10, 64, 65, 1, P, s) == EINVAL
    # fp32 H not a multiple of 4
    assert lib.moe_unpermute_combine(P, P, None, 10, 66, 2, 0, P, s) == EINVAL


def test_forward_rejects_bad_arguments(lib):
    s = None
    ws = lib.moe_forward_workspace_size(16, 64, 64, 8, 2, 1)
    args = [P, P, None, P, P, 16, 64, 64, 8, 2, 0, 1, P, None, None, None, None, P, ws, s]
    bad = list(args)
    bad[18] = ws - 1
    assert lib.moe_forward(*bad) == EWS
    bad = list(args)
    bad[0] = None
    assert lib.moe_forward(*bad) == EINVAL
    bad = list(args)
    bad[9] = 0  # K = 0
    assert lib.moe_forward(*bad) == EINVAL
    for i in (6, 7):  # H, then I, above 2^20 (the GEMM epilogues' 32-bit tile offsets)
        bad = list(args)
        bad[i] = (1 << 20) + 64
        assert lib.moe_forward(*bad) == EINVAL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(moe.MoEError):
        _lib.load_library(str(tmp_path / "missing.so"))


def test_oracle_is_not_imported_by_the_product():
    pkg = os.path.join(ROOT, "routing_token_permute_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in text.replace("the oracle", ""), f


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with status 2 and says why, before touching a device."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_scatter_and_slot_sum_reject_bad_arguments(lib):
    s = None
    # null perm / weights with rows > 0
    assert lib.moe_expert_w2_scatter(P, P, 8, None, P, P, 4, 64, 64, 1, P, s) == EINVAL
    assert lib.moe_expert_w2_scatter(P, P, 8, P, None, P, 4, 64, 64, 1, P, s) == EINVAL
    # bf16 sizes not multiples of 64
    assert lib.moe_expert_w2_scatter(P, P, 8, P, P, P, 4, 96, 64, 1, P, s) == EINVAL
    # unknown dtype
    assert lib.moe_expert_w2_scatter(P, P, 8, P, P, P, 4, 64, 64, 9, P, s) == EUNSUP
    # slot sum: K out of range, null output, bad hidden size
    assert lib.moe_sum_slots(P, 8, 64, 0, 1, P, s) == EINVAL
    assert lib.moe_sum_slots(P, 8, 64, 65, 1, P, s) == EINVAL
    assert lib.moe_sum_slots(P, 8, 64, 2, 1, None, s) == EINVAL
    assert lib.moe_sum_slots(P, 8, 96, 2, 1, P, s) == EINVAL
    assert lib.moe_sum_slots(P, 0, 64, 2, 1, None, s) == 0  # n == 0 is a no-op


def test_backward_calls_reject_bad_arguments(lib):
    s = None
    # combine backward: K out of range, null dw, bad hidden size, unknown dtype
    assert lib.moe_combine_backward(P, P, P, P, 8, 64, 65, 1, P, P, s) == EINVAL
    assert lib.moe_combine_backward(P, P, P, P, 8, 64, 2, 1, P, None, s) == EINVAL
    assert lib.moe_combine_backward(P, P, P, P, 8, 96, 2, 1, P, P, s) == EINVAL
    assert lib.moe_combine_backward(P, P, P, P, 8, 64, 2, 9, P, P, s) == EUNSUP
    assert lib.moe_combine_backward(None, None, None, None, 0, 64, 2, 1, None, None, s) == 0
    # GEMM2 backward without the saved pre-activations; bad I
    assert lib.moe_expert_w2_backward(P, P, 8, P, None, 4, 64, 64, 1, P, s) == EINVAL
    assert lib.moe_expert_w2_backward(P, P, 8, P, P, 4, 64, 48, 1, P, s) == EINVAL
    assert lib.moe_expert_w13_backward(P, P, 8, P, 4, 64, 64, 1, None, s) == EINVAL
    assert lib.moe_expert_w13_backward(P, P, 8, P, 300, 64, 64, 1, P, s) == EINVAL  # E > 256
    # weight gradient: null output, bad M, null inputs with rows > 0
    assert lib.moe_expert_weight_grad(P, P, P, 8, 4, 64, 64, 1, None, s) == EINVAL
    assert lib.moe_expert_weight_grad(P, P, P, 8, 4, 65, 64, 1, P, s) == EINVAL
    assert lib.moe_expert_weight_grad(None, P, P, 8, 4, 64, 64, 1, P, s) == EINVAL
    # dispatch backward
    assert lib.moe_dispatch_backward(P, P, None, 8, 64, 0, 1, P, s) == EINVAL
    assert lib.moe_dispatch_backward(P, None, None, 8, 64, 2, 1, P, s) == EINVAL
    # route backward: K > E, missing workspace for the weight gradients, missing W_gate for dx
    rws = lib.moe_route_backward_workspace_size(16, 64, 8)
    assert rws >= (64 + 1) * 8 * 4  # one token chunk of partial dW_gate and dbias
    assert lib.moe_route_backward(P, P, P, P, P, P, 16, 64, 8, 9, 0, 1, P, P, P, P, P, rws, s) == EINVAL
    assert lib.moe_route_backward(P, P, P, P, P, P, 16, 64, 8, 2, 0, 1, P, P, P, P, None, 0, s) == EWS
    assert lib.moe_route_backward(P, None, P, P, P, P, 16, 64, 8, 2, 0, 1, P, P, None, None, None, 0, s) == EINVAL
    # whole backward: small workspace, missing gradient output
    ws = lib.moe_backward_workspace_size(16, 64, 64, 8, 2, 1)
    assert ws >= 16 * 2 * (64 + 128) * 2
    args = [P, P, P, P, P, 16, 64, 64, 8, 2, 0, 1] + [P] * 9 + [P, P, P, P, P] + [P, ws, s]
    bad = list(args)
    bad[-2] = ws - 1
    assert lib.moe_backward(*bad) == EWS
    bad = list(args)
    bad[24] = None  # dW13
    assert lib.moe_backward(*bad) == EINVAL
    # training forward: null saved buffer
    fws = lib.moe_forward_train_workspace_size(16, 8, 2)
    fargs = [P, P, None, P, P, 16, 64, 64, 8, 2, 0, 1, P] + [P] * 9 + [P, fws, s]
    bad = list(fargs)
    bad[20] = None  # gate_up
    assert lib.moe_forward_train(*bad) == EINVAL
    bad = list(fargs)
    bad[-2] = 0
    assert lib.moe_forward_train(*bad) == EWS


def test_comm_cu_bits_balanced_across_xcds():
    """The communication stream's CUs are spread evenly over the 8 XCDs under both ways of numbering CUs in a
    mask (XCD by XCD, or round-robin), and the sizes outside the supported range are refused."""
    import collections

    from routing_token_permute_amd.ep_share import comm_cu_bits

    for n in (8, 16, 24, 32, 64, 128):
        b = comm_cu_bits(n)
        assert len(b) == n == len(set(b)) and all(0 <= x < 256 for x in b)
        assert sorted(collections.Counter(x // 32 for x in b).values()) == [n // 8] * 8
        assert sorted(collections.Counter(x % 8 for x in b).values()) == [n // 8] * 8
    for bad in (0, 7, 12, 136):
        with pytest.raises(ValueError):
            comm_cu_bits(bad)


def test_misaligned_pointers_are_rejected(lib):
    """Row matrices, weights and workspaces must be 16-byte aligned, per-pair arrays 4-byte aligned
    (the kernels' vector loads, LDS DMA and buffer stores): an offset pointer gives MOE_EINVAL before
    any launch."""
    s = None
    A = ctypes.c_void_p(0x10000)       # 16-byte aligned
    M8 = ctypes.c_void_p(0x10008)      # 8-byte aligned only
    M2 = ctypes.c_void_p(0x10002)      # 2-byte aligned only
    ws = lib.moe_forward_workspace_size(16, 64, 64, 8, 2, 1)
    args = [A, A, None, A, A, 16, 64, 64, 8, 2, 0, 1, A, None, None, None, None, A, ws, s]
    for i in (0, 1, 3, 4, 12, 17):  # x, W_gate, W13, W2, y, ws
        bad = list(args)
        bad[i] = M8
        assert lib.moe_forward(*bad) == EINVAL, i
    for i in (13, 14, 15, 16):  # logits, ids, weights, counts: 4-byte arrays
        bad = list(args)
        bad[i] = M2
        assert lib.moe_forward(*bad) == EINVAL, i
    # route, combine, the expert GEMMs and the backward pieces
    assert lib.moe_route(M8, A, None, 8, 64, 8, 2, 0, 1, A, A, A, s) == EINVAL
    assert lib.moe_route(A, A, None, 8, 64, 8, 2, 0, 1, A, M2, A, s) == EINVAL
    assert lib.moe_unpermute_combine(M8, A, None, 10, 64, 2, 1, A, s) == EINVAL
    assert lib.moe_unpermute_combine(A, A, None, 10, 64, 2, 1, M8, s) == EINVAL
    assert lib.moe_expert_w2(A, A, 8, M8, 4, 64, 64, 1, A, s) == EINVAL
    assert lib.moe_expert_w13_swiglu_gather(A, M2, 4, 2, A, A, 4, 64, 64, 1, A, s) == EINVAL
    assert lib.moe_dispatch_backward(A, A, M8, 8, 64, 2, 1, A, s) == EINVAL
    pws = lib.moe_permute_workspace_size(100, 8, 2)
    assert lib.moe_permute(A, None, 100, 64, 8, 2, 1, 1, A, A, A, A, A, None, M8, pws, s) == EINVAL


def test_zero_tokens_needs_no_workspace(lib):
    """n == 0 is a no-op for the layer call (nothing to write without counts_out), workspace or not."""
    assert lib.moe_forward(None, None, None, None, None, 0, 64, 64, 8, 2, 0, 1, None, None, None, None, None,
                           None, 0, None) == 0
    assert lib.moe_workspace_size(16, 64, 64, 8, 2, 1) == lib.moe_forward_workspace_size(16, 64, 64, 8, 2, 1)


def test_persistent_forward_rejects_bad_arguments(lib):
    """moe_forward_persistent: bf16 only, a warm-up of at least one row tile, a ring either off (0) or
    larger than the warm-up, and a workspace of the stated size, all checked before any launch."""
    s = None
    ws = lib.moe_forward_persistent_workspace_size(16, 64, 64, 8, 2, 0)
    assert ws > 0
    # a ring pool bounds h: at the OLMoE shape 8 queues x 8 slots x 256 rows x I is below n*K rows x I
    assert (lib.moe_forward_persistent_workspace_size(4096, 2048, 1024, 64, 8, 8)
            < lib.moe_forward_persistent_workspace_size(4096, 2048, 1024, 64, 8, 0))
    assert lib.moe_forward_persistent_workspace_size(16, 64, 64, 8, 2, -1) == 0
    args = [P, P, None, P, P, 16, 64, 64, 8, 2, 0, 1, 4, 0, P, None, None, None, None, P, ws, s]
    bad = list(args)
    bad[11] = 0  # fp32
    assert lib.moe_forward_persistent(*bad) == EUNSUP
    bad = list(args)
    bad[12] = 0  # no warm-up
    assert lib.moe_forward_persistent(*bad) == EINVAL
    bad = list(args)
    bad[13] = 4  # ring not larger than the warm-up
    assert lib.moe_forward_persistent(*bad) == EINVAL
    bad = list(args)
    bad[20] = ws - 1
    assert lib.moe_forward_persistent(*bad) == EWS
    # the packed form: the same checks (no dtype argument: bf16)
    pargs = [P, P, None, P, P, 16, 64, 64, 8, 2, 0, 4, 0, P, None, None, None, None, P, ws, s]
    for i, v, code in ((11, 0, EINVAL), (12, 4, EINVAL), (19, ws - 1, EWS), (3, None, EINVAL),
                       (4, ctypes.c_void_p(0x10008), EINVAL)):
        bad = list(pargs)
        bad[i] = v
        assert lib.moe_forward_persistent_packed(*bad) == code, i


def test_w13_from_ids_rejects_unserved_shapes(lib):
    """moe_expert_w13_swiglu_from_ids serves bf16 decode batches only (n <= 32, n*K <= 1024, E <= 256);
    every other shape, dtype or argument error is refused before any launch."""
    s = None
    # x, ids, n, K, W13, E, H, I, ep, dt, h, counts, offsets, splits, perm, inv, stream
    args = [P, P, 32, 8, P, 64, 128, 128, 1, 1, P, P, P, P, P, P, s]
    for i, v, code in ((9, 0, EUNSUP),      # fp32
                       (2, 33, EUNSUP),     # more tokens than one row tile holds
                       (3, 33, EUNSUP),     # 32 x 33 pairs > 1024
                       (8, 3, EINVAL),      # ep does not divide E
                       (6, 100, EINVAL),    # H not a multiple of the tile width
                       (2, -1, EINVAL),
                       (10, None, EINVAL),  # no h
                       (14, None, EINVAL)):  # no perm
        bad = list(args)
        bad[i] = v
        assert lib.moe_expert_w13_swiglu_from_ids(*bad) == code, (i, v)


def test_w13_from_ids_fp8a_rejects_unserved_shapes(lib):
    """The FP8 form serves the same decode shapes (n <= 32, n*K <= 1024, E <= 256, H and I multiples of
    128) and refuses the rest before any launch."""
    s = None
    # codes, s_tok, ids, n, K, W13q, s13, E, H, I, ep, h, counts, offsets, splits, perm, inv, stream
    args = [P, P, P, 32, 8, P, P, 64, 128, 128, 1, P, P, P, P, P, P, s]
    for i, v, code in ((3, 33, EUNSUP), (4, 33, EUNSUP), (8, 192, EINVAL), (9, 64, EINVAL), (10, 3, EINVAL),
                       (11, None, EINVAL), (16, None, EINVAL)):
        bad = list(args)
        bad[i] = v
        assert lib.moe_expert_w13_swiglu_from_ids_fp8a(*bad) == code, (i, v)


def test_w13_from_ids_fp8_weights_rejects_unserved_shapes(lib):
    """The FP8-weight form serves the same decode shapes and refuses the rest before any launch."""
    s = None
    # x, ids, n, K, W13q, s13, E, H, I, ep, h, counts, offsets, splits, perm, inv, stream
    args = [P, P, 32, 8, P, P, 64, 128, 128, 1, P, P, P, P, P, P, s]
    for i, v, code in ((2, 33, EUNSUP), (3, 33, EUNSUP), (7, 100, EINVAL), (9, 3, EINVAL), (10, None, EINVAL),
                       (15, None, EINVAL)):
        bad = list(args)
        bad[i] = v
        assert lib.moe_expert_w13_swiglu_from_ids_fp8(*bad) == code, (i, v)


def test_packed_weights_reject_bad_arguments(lib):
    """Packed sizes follow the documented layout and are 0 outside the bf16 GEMMs' range; the pack calls and
    moe_forward_packed refuse bad shapes, null and misaligned pointers, and a short workspace, before any
    HIP call."""
    s = None
    assert lib.moe_packed_w13_bytes(64, 2048, 1024) == 64 * 8 * 256 * 2048 * 2
    assert lib.moe_packed_w2_bytes(64, 2048, 1024) == 64 * 8 * 256 * 1024 * 2
    assert lib.moe_packed_w13_bytes(3, 128, 192) == 3 * 2 * 256 * 128 * 2  # I = 192: two 128-column blocks
    assert lib.moe_packed_w2_bytes(3, 320, 64) == 3 * 2 * 256 * 64 * 2  # H = 320: two 256-column blocks
    for E, H, I in ((0, 64, 64), (257, 64, 64), (8, 96, 64), (8, 64, 32), (8, 0, 64)):
        assert lib.moe_packed_w13_bytes(E, H, I) == 0 and lib.moe_packed_w2_bytes(E, H, I) == 0
        assert lib.moe_pack_w13(P, E, H, I, P, s) == EINVAL
        assert lib.moe_pack_w2(P, E, H, I, P, s) == EINVAL
    assert lib.moe_pack_w13(None, 8, 64, 64, P, s) == EINVAL
    assert lib.moe_pack_w2(P, 8, 64, 64, None, s) == EINVAL
    M8 = ctypes.c_void_p(0x10008)  # 8-byte aligned only
    assert lib.moe_pack_w13(M8, 8, 64, 64, P, s) == EINVAL
    assert lib.moe_pack_w2(P, 8, 64, 64, M8, s) == EINVAL
    ws = lib.moe_forward_workspace_size(16, 64, 64, 8, 2, 1)
    args = [P, P, None, P, P, 16, 64, 64, 8, 2, 0, P, None, None, None, None, P, ws, None, None, s]
    bad = list(args)
    bad[17] = ws - 1
    assert lib.moe_forward_packed(*bad) == EWS
    for i in (0, 1, 3, 4, 11):  # x, W_gate, W13p, W2p, y
        bad = list(args)
        bad[i] = None
        assert lib.moe_forward_packed(*bad) == EINVAL
    bad = list(args)
    bad[3] = M8
    assert lib.moe_forward_packed(*bad) == EINVAL
    bad = list(args)
    bad[9] = 9  # K > E
    assert lib.moe_forward_packed(*bad) == EINVAL
