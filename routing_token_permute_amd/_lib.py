"""ctypes binding of libmoe.so: the C ABI declared in include/moe.h.

This module only marshals arguments: it checks tensor shapes, dtypes and
devices, allocates outputs and workspaces with torch (device memory and
streams are torch's job here), and passes raw device pointers and the current
HIP stream to the library. Every step of the layer runs in the library's HIP
kernels. If the library is missing or cannot be loaded, every call raises.
"""

from __future__ import annotations

import ctypes
import functools
import inspect
import os
from typing import Optional

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmoe.so")

MOE_F32 = 0
MOE_BF16 = 1

_VP = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

# (name, restype, argtypes) for every exported function of include/moe.h.
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_version": (_I, []),
    "moe_device_info": (_I, [_VP, _VP, _VP, _VP]),
    "moe_route": (_I, [_VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP]),
    "moe_permute_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_permute": (_I, [_VP, _VP, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "moe_grouped_swiglu_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_grouped_swiglu": (_I, [_VP, _VP, _I, _VP, _VP, _I, _I, _I, _I, _VP, _VP, _SZ, _VP]),
    "moe_expert_w13_swiglu": (_I, [_VP, _VP, _I, _VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_expert_w13_swiglu_gather": (_I, [_VP, _VP, _I, _I, _VP, _VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_expert_w13_swiglu_from_ids_fp8a": (_I, [_VP, _VP, _VP, _I, _I, _VP, _VP, _I, _I, _I, _I, _VP, _VP, _VP, _VP,
                                                 _VP, _VP, _VP]),
    "moe_expert_w13_swiglu_from_ids_fp8": (_I, [_VP, _VP, _I, _I, _VP, _VP, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP,
                                                _VP, _VP]),
    "moe_expert_w13_swiglu_from_ids": (_I, [_VP, _VP, _I, _I, _VP, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP,
                                            _VP]),
    "moe_expert_w2": (_I, [_VP, _VP, _I, _VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_expert_w2_scatter": (_I, [_VP, _VP, _I, _VP, _VP, _VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_sum_slots": (_I, [_VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_unpermute_combine": (_I, [_VP, _VP, _VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_forward_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_forward_noalloc_max_bytes": (_SZ, []),
    "moe_forward_persistent_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_forward_persistent": (
        _I,
        [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    ),
    "moe_forward_noalloc": (
        _I,
        [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP],
    ),
    "moe_forward": (
        _I,
        [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    ),
    "moe_forward_timed": (
        _I,
        [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP, _VP, _VP],
    ),
    "moe_expert_w13_swiglu_gather_packed": (_I, [_VP, _VP, _I, _I, _VP, _VP, _I, _I, _I, _VP, _VP]),
    "moe_expert_w13_swiglu_from_ids_packed": (
        _I, [_VP, _VP, _I, _I, _VP, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "moe_expert_w2_packed": (_I, [_VP, _VP, _I, _VP, _I, _I, _I, _VP, _VP]),
    "moe_expert_w2_scatter_packed": (_I, [_VP, _VP, _I, _VP, _VP, _VP, _I, _I, _I, _VP, _VP]),
    "moe_forward_persistent_packed": (
        _I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "moe_packed_w13_bytes": (_SZ, [_I, _I, _I]),
    "moe_packed_w2_bytes": (_SZ, [_I, _I, _I]),
    "moe_pack_w13": (_I, [_VP, _I, _I, _I, _VP, _VP]),
    "moe_pack_w2": (_I, [_VP, _I, _I, _I, _VP, _VP]),
    "moe_forward_packed": (
        _I,
        [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP, _VP, _VP],
    ),
    "moe_expert_w13_swiglu_gather_train": (_I, [_VP, _VP, _I, _I, _VP, _VP, _I, _I, _I, _I, _VP, _VP, _VP]),
    "moe_forward_train_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_forward_train": (
        _I,
        [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
         _VP, _SZ, _VP],
    ),
    "moe_combine_backward": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _I, _VP, _VP, _VP]),
    "moe_expert_w2_backward": (_I, [_VP, _VP, _I, _VP, _VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_expert_w13_backward": (_I, [_VP, _VP, _I, _VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_expert_weight_grad": (_I, [_VP, _VP, _VP, _I, _I, _I, _I, _I, _VP, _VP]),
    "moe_expert_weight_grad_gather": (_I, [_VP, _VP, _I, _I, _VP, _VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_dispatch_backward": (_I, [_VP, _VP, _VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_route_backward_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_route_backward": (
        _I,
        [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    ),
    "moe_quantize_fp8": (_I, [_VP, _I, _I, _I, _I, _VP, _VP, _VP]),
    "moe_expert_w13_swiglu_gather_fp8": (_I, [_VP, _VP, _I, _I, _VP, _VP, _VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_expert_w2_fp8": (_I, [_VP, _VP, _I, _VP, _VP, _I, _I, _I, _I, _VP, _VP]),
    "moe_forward_fp8": (
        _I,
        [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    ),
    "moe_quantize_rows_fp8": (_I, [_VP, _I, _I, _I, _VP, _VP, _VP]),
    "moe_fp8_padded_rows": (_SZ, [_I, _I, _I]),
    "moe_dispatch_fp8": (_I, [_VP, _VP, _VP, _I, _I, _I, _VP, _VP, _I, _VP, _VP, _VP, _VP, _VP, _VP]),
    "moe_expert_w13_swiglu_fp8a": (_I, [_VP, _VP, _VP, _I, _VP, _VP, _I, _I, _I, _VP, _VP]),
    "moe_expert_w2_fp8a": (_I, [_VP, _VP, _VP, _I, _VP, _VP, _I, _I, _I, _VP, _VP]),
    "moe_expert_w13_swiglu_gather_fp8a": (_I, [_VP, _VP, _VP, _I, _I, _VP, _VP, _VP, _I, _I, _I, _VP, _VP]),
    "moe_forward_fp8a_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "moe_forward_fp8a": (
        _I,
        [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    ),
    "moe_backward_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_backward": (
        _I,
        [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
         _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    ),
}

_lib: Optional[ctypes.CDLL] = None


class MoEError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so once and attach the C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise MoEError(
            f"{path} is not built; build it with `python -m routing_token_permute_amd.build` "
            "(there is no fallback implementation)"
        )
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().moe_status_string(code).decode()


def device_info() -> dict:
    """Compute units, peak shader clock and memory clock/bus of the current device."""
    lib = load_library()
    vals = [ctypes.c_int(0) for _ in range(4)]
    _check(lib.moe_device_info(*[ctypes.byref(v) for v in vals]), "moe_device_info")
    return dict(compute_units=vals[0].value, sclk_khz=vals[1].value, mem_clk_khz=vals[2].value,
                mem_bus_bits=vals[3].value)


def _check(code: int, what: str):
    if code != 0:
        raise MoEError(f"{what}: {status_string(code)}")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise MoEError(f"unsupported dtype {t.dtype}; expected torch.bfloat16 or torch.float32")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_stream(fn):
    """Run a binding with `stream` (when given) as torch's current stream, so
    that every output and workspace it allocates belongs to that stream's pool:
    torch's caching allocator then never hands such a block to work on another
    stream while the library's kernels may still use it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        s = sig.bind(*args, **kwargs).arguments.get("stream")
        if s is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(s):
            return fn(*args, **kwargs)

    return wrapper


def _stream(device: torch.device, stream: Optional[torch.cuda.Stream]):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, shape, dtype=None, device=None):
    if not t.is_cuda:
        raise MoEError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise MoEError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise MoEError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise MoEError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise MoEError(f"{name} is on {t.device}, expected {device}")


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if ws is None:
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    if ws.dtype != torch.uint8 or ws.numel() < nbytes or not ws.is_cuda:
        raise MoEError(f"workspace must be a uint8 GPU tensor of at least {nbytes} bytes")
    return ws


# ---------------------------------------------------------------------------
# The five entry points of include/moe.h
# ---------------------------------------------------------------------------


@_on_stream
def moe_route(x, W_gate, bias, K: int, renorm: bool, logits=None, topk_ids=None, topk_w=None, stream=None, E=None):
    """Router GEMM + softmax + top-K. With x None, `logits` (n, E) fp32 is the input.

    Returns (logits, topk_ids, topk_w).
    """
    lib = load_library()
    if x is not None:
        n, H = x.shape
        E = W_gate.shape[1]
        dev = x.device
        _need(x, "x", (n, H))
        _need(W_gate, "W_gate", (H, E), x.dtype, dev)
        dt = _dt(x)
        if logits is None:
            logits = _empty((n, E), torch.float32, dev)
    else:
        if logits is None:
            raise MoEError("logits are required when x is None")
        n, E = logits.shape
        H = 0
        dev = logits.device
        dt = MOE_F32
    _need(logits, "logits", (n, E), torch.float32, dev)
    if bias is not None:
        _need(bias, "bias", (E,), torch.float32, dev)
    topk_ids = _empty((n, K), torch.int32, dev) if topk_ids is None else topk_ids
    topk_w = _empty((n, K), torch.float32, dev) if topk_w is None else topk_w
    _need(topk_ids, "topk_ids", (n, K), torch.int32, dev)
    _need(topk_w, "topk_w", (n, K), torch.float32, dev)
    code = lib.moe_route(
        _ptr(x), _ptr(W_gate), _ptr(bias), n, H, E, K, int(bool(renorm)), dt,
        _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _stream(dev, stream),
    )
    _check(code, "moe_route")
    return logits, topk_ids, topk_w


@_on_stream
def moe_permute(topk_ids, x, E: int, ep: int = 1, out=None, ws=None, stream=None):
    """Counts, offsets, splits, perm, inv and (when x is given) x_perm.

    Returns a dict of tensors; `out` may supply any of them preallocated.
    """
    lib = load_library()
    n, K = topk_ids.shape
    dev = topk_ids.device
    _need(topk_ids, "topk_ids", (n, K), torch.int32)
    out = dict(out or {})
    H = 0
    dt = MOE_BF16
    if x is not None:
        H = x.shape[1]
        _need(x, "x", (n, H), None, dev)
        dt = _dt(x)
        out.setdefault("x_perm", _empty((n * K, H), x.dtype, dev))
        _need(out["x_perm"], "x_perm", (n * K, H), x.dtype, dev)
    out.setdefault("counts", _empty((E,), torch.int32, dev))
    out.setdefault("offsets", _empty((E + 1,), torch.int32, dev))
    out.setdefault("splits", _empty((ep,), torch.int32, dev))
    out.setdefault("perm", _empty((n * K,), torch.int32, dev))
    out.setdefault("inv", _empty((n * K,), torch.int32, dev))
    for name, shape in (("counts", (E,)), ("offsets", (E + 1,)), ("splits", (ep,)), ("perm", (n * K,)), ("inv", (n * K,))):
        _need(out[name], name, shape, torch.int32, dev)
    nbytes = lib.moe_permute_workspace_size(n, E, K)
    ws = _workspace(nbytes, dev, ws)
    code = lib.moe_permute(
        _ptr(topk_ids), _ptr(x), n, H, E, K, ep, dt,
        _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["splits"]), _ptr(out["perm"]), _ptr(out["inv"]),
        _ptr(out.get("x_perm")), _ptr(ws), ws.numel(), _stream(dev, stream),
    )
    _check(code, "moe_permute")
    return out


@_on_stream
def moe_grouped_swiglu(x_perm, offsets, W13, W2, Y_perm=None, ws=None, stream=None):
    """Per-expert SwiGLU FFN on expert-major rows. Returns Y_perm (rows, H)."""
    lib = load_library()
    rows, H = x_perm.shape
    E, H2, I2 = W13.shape
    I = I2 // 2  # noqa: E741
    dev = x_perm.device
    if H2 != H:
        raise MoEError(f"W13 is {tuple(W13.shape)}, expected (E, {H}, 2I)")
    _need(x_perm, "x_perm", (rows, H))
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(W13, "W13", (E, H, 2 * I), x_perm.dtype, dev)
    _need(W2, "W2", (E, I, H), x_perm.dtype, dev)
    Y_perm = _empty((rows, H), x_perm.dtype, dev) if Y_perm is None else Y_perm
    _need(Y_perm, "Y_perm", (rows, H), x_perm.dtype, dev)
    dt = _dt(x_perm)
    ws = _workspace(lib.moe_grouped_swiglu_workspace_size(rows, I, dt), dev, ws)
    code = lib.moe_grouped_swiglu(
        _ptr(x_perm), _ptr(offsets), rows, _ptr(W13), _ptr(W2), E, H, I, dt,
        _ptr(Y_perm), _ptr(ws), ws.numel(), _stream(dev, stream),
    )
    _check(code, "moe_grouped_swiglu")
    return Y_perm


@_on_stream
def moe_expert_w13_swiglu(x_perm, offsets, W13, h=None, stream=None):
    """Algorithm 2 step 8 on expert-major rows: h = SiLU(X W13[:, :I]) * (X W13[:, I:])."""
    lib = load_library()
    rows, H = x_perm.shape
    E, _, I2 = W13.shape
    I = I2 // 2  # noqa: E741
    dev = x_perm.device
    _need(x_perm, "x_perm", (rows, H))
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(W13, "W13", (E, H, 2 * I), x_perm.dtype, dev)
    h = _empty((rows, I), x_perm.dtype, dev) if h is None else h
    _need(h, "h", (rows, I), x_perm.dtype, dev)
    code = lib.moe_expert_w13_swiglu(
        _ptr(x_perm), _ptr(offsets), rows, _ptr(W13), E, H, I, _dt(x_perm), _ptr(h), _stream(dev, stream)
    )
    _check(code, "moe_expert_w13_swiglu")
    return h


@_on_stream
def moe_expert_w13_swiglu_gather(x, perm, K, offsets, W13, h=None, stream=None):
    """Algorithm 2 steps 7-8 fused: h rows for pairs perm[r], reading token rows x[perm[r] // K]."""
    lib = load_library()
    n, H = x.shape
    E, _, I2 = W13.shape
    I = I2 // 2  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H))
    _need(perm, "perm", (n * K,), torch.int32, dev)
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(W13, "W13", (E, H, 2 * I), x.dtype, dev)
    h = _empty((n * K, I), x.dtype, dev) if h is None else h
    _need(h, "h", (n * K, I), x.dtype, dev)
    code = lib.moe_expert_w13_swiglu_gather(
        _ptr(x), _ptr(perm), n, K, _ptr(offsets), _ptr(W13), E, H, I, _dt(x), _ptr(h), _stream(dev, stream)
    )
    _check(code, "moe_expert_w13_swiglu_gather")
    return h


@_on_stream
def moe_expert_w13_swiglu_from_ids(x, topk_ids, W13, ep: int = 1, h=None, out=None, stream=None):
    """Decode-sized GEMM1 straight from the routing ids: h (n*K, I) and the metadata dict of
    moe_permute (counts, offsets, splits, perm, inv) from one launch. Returns (h, meta)."""
    lib = load_library()
    n, H = x.shape
    K = topk_ids.shape[1]
    E, _, I2 = W13.shape
    I = I2 // 2  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H))
    _need(topk_ids, "topk_ids", (n, K), torch.int32, dev)
    _need(W13, "W13", (E, H, 2 * I), x.dtype, dev)
    h = _empty((n * K, I), x.dtype, dev) if h is None else h
    _need(h, "h", (n * K, I), x.dtype, dev)
    out = dict(out or {})
    for name, shape in (("counts", (E,)), ("offsets", (E + 1,)), ("splits", (ep,)), ("perm", (n * K,)),
                        ("inv", (n * K,))):
        out.setdefault(name, _empty(shape, torch.int32, dev))
        _need(out[name], name, shape, torch.int32, dev)
    code = lib.moe_expert_w13_swiglu_from_ids(
        _ptr(x), _ptr(topk_ids), n, K, _ptr(W13), E, H, I, ep, _dt(x), _ptr(h), _ptr(out["counts"]),
        _ptr(out["offsets"]), _ptr(out["splits"]), _ptr(out["perm"]), _ptr(out["inv"]), _stream(dev, stream),
    )
    _check(code, "moe_expert_w13_swiglu_from_ids")
    return h, out


@_on_stream
def moe_expert_w2(h, offsets, W2, Y_perm=None, stream=None):
    """Algorithm 2 step 9 on expert-major rows: Y_perm = h W2[e] per segment."""
    lib = load_library()
    rows, I = h.shape  # noqa: E741
    E, _, H = W2.shape
    dev = h.device
    _need(h, "h", (rows, I))
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(W2, "W2", (E, I, H), h.dtype, dev)
    Y_perm = _empty((rows, H), h.dtype, dev) if Y_perm is None else Y_perm
    _need(Y_perm, "Y_perm", (rows, H), h.dtype, dev)
    code = lib.moe_expert_w2(_ptr(h), _ptr(offsets), rows, _ptr(W2), E, H, I, _dt(h), _ptr(Y_perm), _stream(dev, stream))
    _check(code, "moe_expert_w2")
    return Y_perm


@_on_stream
def moe_expert_w2_scatter(h, offsets, perm, topk_w, W2, Y_tok=None, stream=None):
    """GEMM2 with the weight and un-permutation in its epilogue:
    Y_tok[perm[p]] = topk_w.flat[perm[p]] * (h[p] W2[e]). topk_w is (n, K) fp32."""
    lib = load_library()
    rows, I = h.shape  # noqa: E741
    E, _, H = W2.shape
    dev = h.device
    _need(h, "h", (rows, I))
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(perm, "perm", (rows,), torch.int32, dev)
    if topk_w.numel() != rows or topk_w.dtype != torch.float32 or not topk_w.is_contiguous() or topk_w.device != dev:
        raise MoEError(f"topk_w: expected {rows} contiguous fp32 values on {dev}")
    _need(W2, "W2", (E, I, H), h.dtype, dev)
    Y_tok = _empty((rows, H), h.dtype, dev) if Y_tok is None else Y_tok
    _need(Y_tok, "Y_tok", (rows, H), h.dtype, dev)
    code = lib.moe_expert_w2_scatter(_ptr(h), _ptr(offsets), rows, _ptr(perm), _ptr(topk_w), _ptr(W2), E, H, I,
                                     _dt(h), _ptr(Y_tok), _stream(dev, stream))
    _check(code, "moe_expert_w2_scatter")
    return Y_tok


@_on_stream
def moe_sum_slots(Y_tok, n: int, K: int, y=None, stream=None):
    """y[i] = sum_k Y_tok[i*K+k] in slot order (fp32 accumulation)."""
    lib = load_library()
    rows, H = Y_tok.shape
    dev = Y_tok.device
    _need(Y_tok, "Y_tok", (n * K, H))
    y = _empty((n, H), Y_tok.dtype, dev) if y is None else y
    _need(y, "y", (n, H), Y_tok.dtype, dev)
    code = lib.moe_sum_slots(_ptr(Y_tok), n, H, K, _dt(Y_tok), _ptr(y), _stream(dev, stream))
    _check(code, "moe_sum_slots")
    return y


@_on_stream
def moe_unpermute_combine(Y_perm, inv, topk_w, n: int, K: int, y=None, stream=None):
    """y[i] = sum_k w[i,k] Y_perm[inv[i*K+k]] (unit weights when topk_w is None)."""
    lib = load_library()
    rows, H = Y_perm.shape
    dev = Y_perm.device
    _need(Y_perm, "Y_perm", (n * K, H))
    _need(inv, "inv", (n * K,), torch.int32, dev)
    if topk_w is not None:
        _need(topk_w, "topk_w", (n, K), torch.float32, dev)
    y = _empty((n, H), Y_perm.dtype, dev) if y is None else y
    _need(y, "y", (n, H), Y_perm.dtype, dev)
    code = lib.moe_unpermute_combine(
        _ptr(Y_perm), _ptr(inv), _ptr(topk_w), n, H, K, _dt(Y_perm), _ptr(y), _stream(dev, stream)
    )
    _check(code, "moe_unpermute_combine")
    return y


@_on_stream
def moe_forward_workspace_size(n, H, I, E, K, dtype) -> int:  # noqa: E741
    return int(load_library().moe_forward_workspace_size(n, H, I, E, K, _dt(torch.empty(0, dtype=dtype))))


@_on_stream
def moe_forward(x, W_gate, W13, W2, K: int, renorm: bool, bias=None, y=None, ws=None, routing_out=False, stream=None):
    """Whole layer. Returns y, or (y, logits, topk_ids, topk_w, counts) with routing_out."""
    lib = load_library()
    n, H = x.shape
    E = W_gate.shape[1]
    I = W13.shape[2] // 2  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H))
    _need(W_gate, "W_gate", (H, E), x.dtype, dev)
    _need(W13, "W13", (E, H, 2 * I), x.dtype, dev)
    _need(W2, "W2", (E, I, H), x.dtype, dev)
    if bias is not None:
        _need(bias, "bias", (E,), torch.float32, dev)
    y = _empty((n, H), x.dtype, dev) if y is None else y
    _need(y, "y", (n, H), x.dtype, dev)
    dt = _dt(x)
    ws = _workspace(lib.moe_forward_workspace_size(n, H, I, E, K, dt), dev, ws)
    extra = [None] * 4
    if routing_out:
        extra = [
            _empty((n, E), torch.float32, dev),
            _empty((n, K), torch.int32, dev),
            _empty((n, K), torch.float32, dev),
            _empty((E,), torch.int32, dev),
        ]
    code = lib.moe_forward(
        _ptr(x), _ptr(W_gate), _ptr(bias), _ptr(W13), _ptr(W2), n, H, I, E, K, int(bool(renorm)), dt,
        _ptr(y), *[_ptr(t) for t in extra], _ptr(ws), ws.numel(), _stream(dev, stream),
    )
    _check(code, "moe_forward")
    return (y, *extra) if routing_out else y


@_on_stream
def moe_forward_timed(x, W_gate, W13, W2, K: int, renorm: bool, gemm1_begin, gemm1_end, bias=None, y=None, ws=None,
                      stream=None):
    """moe_forward that records two timing events on the stream right before and after the layer's GEMM1
    launch. Each event is a torch.cuda.Event (enable_timing=True, recorded once before so that it exists),
    a raw hipEvent_t handle (int), or None. Returns y."""
    lib = load_library()
    n, H = x.shape
    E = W_gate.shape[1]
    I = W13.shape[2] // 2  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H))
    _need(W_gate, "W_gate", (H, E), x.dtype, dev)
    _need(W13, "W13", (E, H, 2 * I), x.dtype, dev)
    _need(W2, "W2", (E, I, H), x.dtype, dev)
    if bias is not None:
        _need(bias, "bias", (E,), torch.float32, dev)
    y = _empty((n, H), x.dtype, dev) if y is None else y
    _need(y, "y", (n, H), x.dtype, dev)
    dt = _dt(x)
    ws = _workspace(lib.moe_forward_workspace_size(n, H, I, E, K, dt), dev, ws)
    handles = []
    for ev in (gemm1_begin, gemm1_end):
        h = ev if (ev is None or isinstance(ev, int)) else ev.cuda_event
        if ev is not None and not h:
            raise MoEError("record the event once before passing it (torch creates it on first record)")
        handles.append(h)
    code = lib.moe_forward_timed(
        _ptr(x), _ptr(W_gate), _ptr(bias), _ptr(W13), _ptr(W2), n, H, I, E, K, int(bool(renorm)), dt,
        _ptr(y), None, None, None, None, _ptr(ws), ws.numel(), handles[0], handles[1], _stream(dev, stream),
    )
    _check(code, "moe_forward_timed")
    return y


def _event_handles(events):
    handles = []
    for ev in events:
        h = ev if (ev is None or isinstance(ev, int)) else ev.cuda_event
        if ev is not None and not h:
            raise MoEError("record the event once before passing it (torch creates it on first record)")
        handles.append(h)
    return handles


@_on_stream
def moe_pack_w13(W13, stream=None):
    """W13 (E, H, 2I) bf16 in the GEMMs' packed form: a bf16 tensor of shape
    (E, H/32, ceil(I/128), 256, 32) (expert, 32-deep unit, column block, column, k
    as stored: the 16-byte k-chunks of column c sit at slot chunk ^ ((c/2) % 4))."""
    lib = load_library()
    E, H, I2 = W13.shape
    I = I2 // 2  # noqa: E741
    _need(W13, "W13", (E, H, 2 * I), torch.bfloat16)
    out = _empty((E, H // 32, -(-I // 128), 256, 32), torch.bfloat16, W13.device)
    if out.numel() * 2 != lib.moe_packed_w13_bytes(E, H, I):
        raise MoEError("moe_pack_w13: unsupported shape")
    _check(lib.moe_pack_w13(_ptr(W13), E, H, I, _ptr(out), _stream(W13.device, stream)), "moe_pack_w13")
    return out


@_on_stream
def moe_pack_w2(W2, stream=None):
    """W2 (E, I, H) bf16 in the packed form: (E, I/32, ceil(H/256), 256, 32)."""
    lib = load_library()
    E, I, H = W2.shape  # noqa: E741
    _need(W2, "W2", (E, I, H), torch.bfloat16)
    out = _empty((E, I // 32, -(-H // 256), 256, 32), torch.bfloat16, W2.device)
    if out.numel() * 2 != lib.moe_packed_w2_bytes(E, H, I):
        raise MoEError("moe_pack_w2: unsupported shape")
    _check(lib.moe_pack_w2(_ptr(W2), E, H, I, _ptr(out), _stream(W2.device, stream)), "moe_pack_w2")
    return out


def _packed_dims(W13p=None, W2p=None):
    """(E, H or I from the unit count, blocks) of a packed weight tensor."""
    t = W13p if W13p is not None else W2p
    if t.dim() != 5 or tuple(t.shape[3:]) != (256, 32) or t.dtype != torch.bfloat16:
        raise MoEError(f"packed weights must be bf16 of shape (E, K/32, blocks, 256, 32), got {tuple(t.shape)}")
    return t.shape[0], t.shape[1] * 32, t.shape[2]


@_on_stream
def moe_expert_w13_swiglu_gather_packed(x, perm, K, offsets, W13p, I, h=None, stream=None):  # noqa: E741
    """moe_expert_w13_swiglu_gather over W13 packed by moe_pack_w13 (bf16); I is the layer's
    intermediate size (the packed blocks round it up to 128)."""
    lib = load_library()
    n, H = x.shape
    E, Hp, NB = _packed_dims(W13p=W13p)
    dev = x.device
    if Hp != H or NB != -(-I // 128):
        raise MoEError("W13p does not match x and I")
    _need(x, "x", (n, H), torch.bfloat16)
    _need(perm, "perm", (n * K,), torch.int32, dev)
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    h = _empty((n * K, I), torch.bfloat16, dev) if h is None else h
    _need(h, "h", (n * K, I), torch.bfloat16, dev)
    code = lib.moe_expert_w13_swiglu_gather_packed(_ptr(x), _ptr(perm), n, K, _ptr(offsets), _ptr(W13p), E, H, I,
                                                   _ptr(h), _stream(dev, stream))
    _check(code, "moe_expert_w13_swiglu_gather_packed")
    return h


@_on_stream
def moe_expert_w13_swiglu_from_ids_packed(x, topk_ids, W13p, I, ep: int = 1, h=None, out=None,  # noqa: E741
                                          stream=None):
    """moe_expert_w13_swiglu_from_ids over W13 packed by moe_pack_w13 (bf16). Returns (h, meta)."""
    lib = load_library()
    n, H = x.shape
    K = topk_ids.shape[1]
    E, Hp, NB = _packed_dims(W13p=W13p)
    dev = x.device
    if Hp != H or NB != -(-I // 128):
        raise MoEError("W13p does not match x and I")
    _need(x, "x", (n, H), torch.bfloat16)
    _need(topk_ids, "topk_ids", (n, K), torch.int32, dev)
    h = _empty((n * K, I), torch.bfloat16, dev) if h is None else h
    _need(h, "h", (n * K, I), torch.bfloat16, dev)
    out = dict(out or {})
    for name, shape in (("counts", (E,)), ("offsets", (E + 1,)), ("splits", (ep,)), ("perm", (n * K,)),
                        ("inv", (n * K,))):
        out.setdefault(name, _empty(shape, torch.int32, dev))
        _need(out[name], name, shape, torch.int32, dev)
    code = lib.moe_expert_w13_swiglu_from_ids_packed(
        _ptr(x), _ptr(topk_ids), n, K, _ptr(W13p), E, H, I, ep, _ptr(h), _ptr(out["counts"]), _ptr(out["offsets"]),
        _ptr(out["splits"]), _ptr(out["perm"]), _ptr(out["inv"]), _stream(dev, stream),
    )
    _check(code, "moe_expert_w13_swiglu_from_ids_packed")
    return h, out


@_on_stream
def moe_expert_w2_packed(h, offsets, W2p, H, Y_perm=None, stream=None):
    """moe_expert_w2 over W2 packed by moe_pack_w2 (bf16); H is the layer's hidden size."""
    lib = load_library()
    rows, I = h.shape  # noqa: E741
    E, Ip, NB = _packed_dims(W2p=W2p)
    dev = h.device
    if Ip != I or NB != -(-H // 256):
        raise MoEError("W2p does not match h and H")
    _need(h, "h", (rows, I), torch.bfloat16)
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    Y_perm = _empty((rows, H), torch.bfloat16, dev) if Y_perm is None else Y_perm
    _need(Y_perm, "Y_perm", (rows, H), torch.bfloat16, dev)
    code = lib.moe_expert_w2_packed(_ptr(h), _ptr(offsets), rows, _ptr(W2p), E, H, I, _ptr(Y_perm),
                                    _stream(dev, stream))
    _check(code, "moe_expert_w2_packed")
    return Y_perm


@_on_stream
def moe_expert_w2_scatter_packed(h, offsets, perm, topk_w, W2p, H, Y_tok=None, stream=None):
    """moe_expert_w2_scatter over W2 packed by moe_pack_w2 (bf16); H is the layer's hidden size."""
    lib = load_library()
    rows, I = h.shape  # noqa: E741
    E, Ip, NB = _packed_dims(W2p=W2p)
    dev = h.device
    if Ip != I or NB != -(-H // 256):
        raise MoEError("W2p does not match h and H")
    _need(h, "h", (rows, I), torch.bfloat16)
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(perm, "perm", (rows,), torch.int32, dev)
    if topk_w.numel() != rows or topk_w.dtype != torch.float32 or not topk_w.is_contiguous() or topk_w.device != dev:
        raise MoEError(f"topk_w: expected {rows} contiguous fp32 values on {dev}")
    Y_tok = _empty((rows, H), torch.bfloat16, dev) if Y_tok is None else Y_tok
    _need(Y_tok, "Y_tok", (rows, H), torch.bfloat16, dev)
    code = lib.moe_expert_w2_scatter_packed(_ptr(h), _ptr(offsets), rows, _ptr(perm), _ptr(topk_w), _ptr(W2p), E, H,
                                            I, _ptr(Y_tok), _stream(dev, stream))
    _check(code, "moe_expert_w2_scatter_packed")
    return Y_tok


@_on_stream
def moe_forward_packed(x, W_gate, W13p, W2p, K: int, renorm: bool, bias=None, y=None, ws=None, routing_out=False,
                       gemm1_begin=None, gemm1_end=None, stream=None):
    """moe_forward (bf16) over weights packed by moe_pack_w13 / moe_pack_w2; the same results bit for
    bit. Returns y, or (y, logits, topk_ids, topk_w, counts) with routing_out. gemm1_begin / gemm1_end:
    optional timing events around GEMM1, as in moe_forward_timed."""
    lib = load_library()
    n, H = x.shape
    E = W_gate.shape[1]
    I = W2p.shape[1] * 32  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H), torch.bfloat16)
    _need(W_gate, "W_gate", (H, E), torch.bfloat16, dev)
    _need(W13p, "W13p", (E, H // 32, -(-I // 128), 256, 32), torch.bfloat16, dev)
    _need(W2p, "W2p", (E, I // 32, -(-H // 256), 256, 32), torch.bfloat16, dev)
    if bias is not None:
        _need(bias, "bias", (E,), torch.float32, dev)
    y = _empty((n, H), torch.bfloat16, dev) if y is None else y
    _need(y, "y", (n, H), torch.bfloat16, dev)
    ws = _workspace(lib.moe_forward_workspace_size(n, H, I, E, K, MOE_BF16), dev, ws)
    extra = [None] * 4
    if routing_out:
        extra = [_empty((n, E), torch.float32, dev), _empty((n, K), torch.int32, dev),
                 _empty((n, K), torch.float32, dev), _empty((E,), torch.int32, dev)]
    handles = _event_handles((gemm1_begin, gemm1_end))
    code = lib.moe_forward_packed(
        _ptr(x), _ptr(W_gate), _ptr(bias), _ptr(W13p), _ptr(W2p), n, H, I, E, K, int(bool(renorm)), _ptr(y),
        *[_ptr(t) for t in extra], _ptr(ws), ws.numel(), handles[0], handles[1], _stream(dev, stream),
    )
    _check(code, "moe_forward_packed")
    return (y, *extra) if routing_out else y


def moe_forward_persistent_workspace_size(n, H, I, E, K, pool_row_tiles=0) -> int:  # noqa: E741
    return int(load_library().moe_forward_persistent_workspace_size(n, H, I, E, K, pool_row_tiles))


@_on_stream
def moe_forward_persistent(x, W_gate, W13, W2, K: int, renorm: bool, bias=None, warmup_row_tiles=16,
                           pool_row_tiles=0, y=None, ws=None, routing_out=False, stream=None):
    """moe_forward with GEMM1 + SwiGLU and GEMM2 in one persistent kernel (bf16). Returns y, or
    (y, logits, topk_ids, topk_w, counts) with routing_out. The workspace's last int32 is the
    scheduler's flag word (nonzero if a bounded wait ran out)."""
    lib = load_library()
    n, H = x.shape
    E = W_gate.shape[1]
    I = W13.shape[2] // 2  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H), torch.bfloat16)
    _need(W_gate, "W_gate", (H, E), torch.bfloat16, dev)
    _need(W13, "W13", (E, H, 2 * I), torch.bfloat16, dev)
    _need(W2, "W2", (E, I, H), torch.bfloat16, dev)
    if bias is not None:
        _need(bias, "bias", (E,), torch.float32, dev)
    y = _empty((n, H), torch.bfloat16, dev) if y is None else y
    _need(y, "y", (n, H), torch.bfloat16, dev)
    ws = _workspace(lib.moe_forward_persistent_workspace_size(n, H, I, E, K, pool_row_tiles), dev, ws)
    extra = [None] * 4
    if routing_out:
        extra = [_empty((n, E), torch.float32, dev), _empty((n, K), torch.int32, dev),
                 _empty((n, K), torch.float32, dev), _empty((E,), torch.int32, dev)]
    code = lib.moe_forward_persistent(
        _ptr(x), _ptr(W_gate), _ptr(bias), _ptr(W13), _ptr(W2), n, H, I, E, K, int(bool(renorm)), MOE_BF16,
        int(warmup_row_tiles), int(pool_row_tiles), _ptr(y), *[_ptr(t) for t in extra], _ptr(ws), ws.numel(),
        _stream(dev, stream),
    )
    _check(code, "moe_forward_persistent")
    return (y, *extra) if routing_out else y


@_on_stream
def moe_forward_persistent_packed(x, W_gate, W13p, W2p, K: int, renorm: bool, bias=None, warmup_row_tiles=16,
                                  pool_row_tiles=0, y=None, ws=None, routing_out=False, stream=None):
    """moe_forward_persistent over weights packed by moe_pack_w13 / moe_pack_w2 (bf16); the same results
    bit for bit. Returns y, or (y, logits, topk_ids, topk_w, counts) with routing_out."""
    lib = load_library()
    n, H = x.shape
    E = W_gate.shape[1]
    I = W2p.shape[1] * 32  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H), torch.bfloat16)
    _need(W_gate, "W_gate", (H, E), torch.bfloat16, dev)
    _need(W13p, "W13p", (E, H // 32, -(-I // 128), 256, 32), torch.bfloat16, dev)
    _need(W2p, "W2p", (E, I // 32, -(-H // 256), 256, 32), torch.bfloat16, dev)
    if bias is not None:
        _need(bias, "bias", (E,), torch.float32, dev)
    y = _empty((n, H), torch.bfloat16, dev) if y is None else y
    _need(y, "y", (n, H), torch.bfloat16, dev)
    ws = _workspace(lib.moe_forward_persistent_workspace_size(n, H, I, E, K, pool_row_tiles), dev, ws)
    extra = [None] * 4
    if routing_out:
        extra = [_empty((n, E), torch.float32, dev), _empty((n, K), torch.int32, dev),
                 _empty((n, K), torch.float32, dev), _empty((E,), torch.int32, dev)]
    code = lib.moe_forward_persistent_packed(
        _ptr(x), _ptr(W_gate), _ptr(bias), _ptr(W13p), _ptr(W2p), n, H, I, E, K, int(bool(renorm)),
        int(warmup_row_tiles), int(pool_row_tiles), _ptr(y), *[_ptr(t) for t in extra], _ptr(ws), ws.numel(),
        _stream(dev, stream),
    )
    _check(code, "moe_forward_persistent_packed")
    return (y, *extra) if routing_out else y


@_on_stream
def moe_forward_noalloc(x, W_gate, W13, W2, K: int, renorm: bool, bias=None, y=None, routing_out=False, stream=None):
    """moe_forward on the library's fixed device scratch (no workspace argument; the library
    allocates nothing). Returns y, or (y, logits, topk_ids, topk_w, counts) with routing_out."""
    lib = load_library()
    n, H = x.shape
    E = W_gate.shape[1]
    I = W13.shape[2] // 2  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H))
    _need(W_gate, "W_gate", (H, E), x.dtype, dev)
    _need(W13, "W13", (E, H, 2 * I), x.dtype, dev)
    _need(W2, "W2", (E, I, H), x.dtype, dev)
    if bias is not None:
        _need(bias, "bias", (E,), torch.float32, dev)
    y = _empty((n, H), x.dtype, dev) if y is None else y
    _need(y, "y", (n, H), x.dtype, dev)
    extra = [None] * 4
    if routing_out:
        extra = [
            _empty((n, E), torch.float32, dev),
            _empty((n, K), torch.int32, dev),
            _empty((n, K), torch.float32, dev),
            _empty((E,), torch.int32, dev),
        ]
    code = lib.moe_forward_noalloc(
        _ptr(x), _ptr(W_gate), _ptr(bias), _ptr(W13), _ptr(W2), n, H, I, E, K, int(bool(renorm)), _dt(x),
        _ptr(y), *[_ptr(t) for t in extra], _stream(dev, stream),
    )
    _check(code, "moe_forward_noalloc")
    return (y, *extra) if routing_out else y


# ---------------------------------------------------------------------------
# Backward (training) entry points
# ---------------------------------------------------------------------------


@_on_stream
def moe_expert_w13_swiglu_gather_train(x, perm, K, offsets, W13, h=None, gate_up=None, stream=None):
    """moe_expert_w13_swiglu_gather that also writes the pre-activations [gate | up].

    Returns (h (n*K, I), gate_up (n*K, 2I))."""
    lib = load_library()
    n, H = x.shape
    E, _, I2 = W13.shape
    I = I2 // 2  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H))
    _need(perm, "perm", (n * K,), torch.int32, dev)
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(W13, "W13", (E, H, 2 * I), x.dtype, dev)
    h = _empty((n * K, I), x.dtype, dev) if h is None else h
    gate_up = _empty((n * K, 2 * I), x.dtype, dev) if gate_up is None else gate_up
    _need(h, "h", (n * K, I), x.dtype, dev)
    _need(gate_up, "gate_up", (n * K, 2 * I), x.dtype, dev)
    code = lib.moe_expert_w13_swiglu_gather_train(
        _ptr(x), _ptr(perm), n, K, _ptr(offsets), _ptr(W13), E, H, I, _dt(x), _ptr(h), _ptr(gate_up),
        _stream(dev, stream),
    )
    _check(code, "moe_expert_w13_swiglu_gather_train")
    return h, gate_up


@_on_stream
def moe_forward_train(x, W_gate, W13, W2, K: int, renorm: bool, bias=None, saved=None, y=None, ws=None, stream=None):
    """The layer's forward keeping what moe_backward reads.

    Returns (y, saved) where saved is a dict of logits, topk_ids, topk_w,
    offsets, perm, inv, gate_up, h, Y_perm (preallocated ones may be passed in
    `saved`)."""
    lib = load_library()
    n, H = x.shape
    E = W_gate.shape[1]
    I = W13.shape[2] // 2  # noqa: E741
    dev, dt_t = x.device, x.dtype
    _need(x, "x", (n, H))
    _need(W_gate, "W_gate", (H, E), dt_t, dev)
    _need(W13, "W13", (E, H, 2 * I), dt_t, dev)
    _need(W2, "W2", (E, I, H), dt_t, dev)
    if bias is not None:
        _need(bias, "bias", (E,), torch.float32, dev)
    shapes = dict(
        logits=((n, E), torch.float32), topk_ids=((n, K), torch.int32), topk_w=((n, K), torch.float32),
        offsets=((E + 1,), torch.int32), perm=((n * K,), torch.int32), inv=((n * K,), torch.int32),
        gate_up=((n * K, 2 * I), dt_t), h=((n * K, I), dt_t), Y_perm=((n * K, H), dt_t),
    )
    saved = dict(saved or {})
    for name, (shape, dtype) in shapes.items():
        saved.setdefault(name, _empty(shape, dtype, dev))
        _need(saved[name], name, shape, dtype, dev)
    y = _empty((n, H), dt_t, dev) if y is None else y
    _need(y, "y", (n, H), dt_t, dev)
    ws = _workspace(lib.moe_forward_train_workspace_size(n, E, K), dev, ws)
    code = lib.moe_forward_train(
        _ptr(x), _ptr(W_gate), _ptr(bias), _ptr(W13), _ptr(W2), n, H, I, E, K, int(bool(renorm)), _dt(x), _ptr(y),
        *[_ptr(saved[k]) for k in shapes], _ptr(ws), ws.numel(), _stream(dev, stream),
    )
    _check(code, "moe_forward_train")
    return y, saved


@_on_stream
def moe_combine_backward(dy, Y_perm, inv, topk_w, n: int, K: int, dY_perm=None, dw=None, stream=None):
    """dY_perm[inv[iK+k]] = w[i,k] dy[i] and dw[i,k] = <dy[i], Y_perm[inv[iK+k]]>. Returns (dY_perm, dw)."""
    lib = load_library()
    H = dy.shape[1]
    dev = dy.device
    _need(dy, "dy", (n, H))
    _need(Y_perm, "Y_perm", (n * K, H), dy.dtype, dev)
    _need(inv, "inv", (n * K,), torch.int32, dev)
    _need(topk_w, "topk_w", (n, K), torch.float32, dev)
    dY_perm = _empty((n * K, H), dy.dtype, dev) if dY_perm is None else dY_perm
    dw = _empty((n, K), torch.float32, dev) if dw is None else dw
    _need(dY_perm, "dY_perm", (n * K, H), dy.dtype, dev)
    _need(dw, "dw", (n, K), torch.float32, dev)
    code = lib.moe_combine_backward(_ptr(dy), _ptr(Y_perm), _ptr(inv), _ptr(topk_w), n, H, K, _dt(dy), _ptr(dY_perm),
                                    _ptr(dw), _stream(dev, stream))
    _check(code, "moe_combine_backward")
    return dY_perm, dw


@_on_stream
def moe_expert_w2_backward(dY_perm, offsets, W2, gate_up, dgate_up=None, stream=None):
    """dgate_up = SwiGLU'(gate_up) applied to dY_perm W2[e]^T per expert segment."""
    lib = load_library()
    rows, H = dY_perm.shape
    E, I, _ = W2.shape  # noqa: E741
    dev = dY_perm.device
    _need(dY_perm, "dY_perm", (rows, H))
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(W2, "W2", (E, I, H), dY_perm.dtype, dev)
    _need(gate_up, "gate_up", (rows, 2 * I), dY_perm.dtype, dev)
    dgate_up = _empty((rows, 2 * I), dY_perm.dtype, dev) if dgate_up is None else dgate_up
    _need(dgate_up, "dgate_up", (rows, 2 * I), dY_perm.dtype, dev)
    code = lib.moe_expert_w2_backward(_ptr(dY_perm), _ptr(offsets), rows, _ptr(W2), _ptr(gate_up), E, H, I,
                                      _dt(dY_perm), _ptr(dgate_up), _stream(dev, stream))
    _check(code, "moe_expert_w2_backward")
    return dgate_up


@_on_stream
def moe_expert_w13_backward(dgate_up, offsets, W13, dX_perm=None, stream=None):
    """dX_perm = dgate_up W13[e]^T per expert segment."""
    lib = load_library()
    rows, I2 = dgate_up.shape
    E, H, _ = W13.shape
    I = I2 // 2  # noqa: E741
    dev = dgate_up.device
    _need(dgate_up, "dgate_up", (rows, 2 * I))
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(W13, "W13", (E, H, 2 * I), dgate_up.dtype, dev)
    dX_perm = _empty((rows, H), dgate_up.dtype, dev) if dX_perm is None else dX_perm
    _need(dX_perm, "dX_perm", (rows, H), dgate_up.dtype, dev)
    code = lib.moe_expert_w13_backward(_ptr(dgate_up), _ptr(offsets), rows, _ptr(W13), E, H, I, _dt(dgate_up),
                                       _ptr(dX_perm), _stream(dev, stream))
    _check(code, "moe_expert_w13_backward")
    return dX_perm


@_on_stream
def moe_expert_weight_grad(a, b, offsets, dW=None, stream=None):
    """dW[e] = a[seg e]^T b[seg e] over each expert's rows. Returns dW (E, M, N)."""
    lib = load_library()
    rows, M = a.shape
    N = b.shape[1]
    E = offsets.shape[0] - 1
    dev = a.device
    _need(a, "a", (rows, M))
    _need(b, "b", (rows, N), a.dtype, dev)
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    dW = _empty((E, M, N), a.dtype, dev) if dW is None else dW
    _need(dW, "dW", (E, M, N), a.dtype, dev)
    code = lib.moe_expert_weight_grad(_ptr(a), _ptr(b), _ptr(offsets), rows, E, M, N, _dt(a), _ptr(dW),
                                      _stream(dev, stream))
    _check(code, "moe_expert_weight_grad")
    return dW


@_on_stream
def moe_expert_weight_grad_gather(x, perm, K: int, b, offsets, dW=None, stream=None):
    """dW[e] = sum over rows r of expert e of x[perm[r] // K]^T b[r]. Returns dW (E, M, N)."""
    lib = load_library()
    n, M = x.shape
    rows, N = b.shape
    E = offsets.shape[0] - 1
    dev = x.device
    _need(x, "x", (n, M))
    _need(perm, "perm", (n * K,), torch.int32, dev)
    _need(b, "b", (n * K, N), x.dtype, dev)
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    dW = _empty((E, M, N), x.dtype, dev) if dW is None else dW
    _need(dW, "dW", (E, M, N), x.dtype, dev)
    code = lib.moe_expert_weight_grad_gather(_ptr(x), _ptr(perm), n, K, _ptr(b), _ptr(offsets), E, M, N, _dt(x),
                                             _ptr(dW), _stream(dev, stream))
    _check(code, "moe_expert_weight_grad_gather")
    return dW


@_on_stream
def moe_dispatch_backward(dX_perm, inv, n: int, K: int, add=None, dx=None, stream=None):
    """dx[i] = add[i] + sum_k dX_perm[inv[iK+k]] (add: (n, H) fp32 or None)."""
    lib = load_library()
    H = dX_perm.shape[1]
    dev = dX_perm.device
    _need(dX_perm, "dX_perm", (n * K, H))
    _need(inv, "inv", (n * K,), torch.int32, dev)
    if add is not None:
        _need(add, "add", (n, H), torch.float32, dev)
    dx = _empty((n, H), dX_perm.dtype, dev) if dx is None else dx
    _need(dx, "dx", (n, H), dX_perm.dtype, dev)
    code = lib.moe_dispatch_backward(_ptr(dX_perm), _ptr(inv), _ptr(add), n, H, K, _dt(dX_perm), _ptr(dx),
                                     _stream(dev, stream))
    _check(code, "moe_dispatch_backward")
    return dx


@_on_stream
def moe_route_backward(x, W_gate, logits, topk_ids, topk_w, dw, renorm: bool, want_dx=True, want_weights=True,
                       ws=None, stream=None):
    """Gradient through routing given dw = dL/dtopk_w.

    Returns dict(dlogits, dx_router or None, dW_gate or None, dbias or None), all fp32."""
    lib = load_library()
    n, E = logits.shape
    K = topk_ids.shape[1]
    dev = logits.device
    src = W_gate if W_gate is not None else x
    H = 0 if src is None else (W_gate.shape[0] if W_gate is not None else x.shape[1])
    dt_t = torch.float32 if src is None else src.dtype
    _need(logits, "logits", (n, E), torch.float32, dev)
    _need(topk_ids, "topk_ids", (n, K), torch.int32, dev)
    _need(topk_w, "topk_w", (n, K), torch.float32, dev)
    _need(dw, "dw", (n, K), torch.float32, dev)
    if want_dx:
        _need(W_gate, "W_gate", (H, E), dt_t, dev)
    if want_weights:
        _need(x, "x", (n, H), dt_t, dev)
    out = dict(
        dlogits=_empty((n, E), torch.float32, dev),
        dx_router=_empty((n, H), torch.float32, dev) if want_dx else None,
        dW_gate=_empty((H, E), torch.float32, dev) if want_weights else None,
        dbias=_empty((E,), torch.float32, dev) if want_weights else None,
    )
    nbytes = lib.moe_route_backward_workspace_size(n, H, E) if (want_weights or want_dx) else 0
    ws = _workspace(nbytes, dev, ws)
    code = lib.moe_route_backward(
        _ptr(x), _ptr(W_gate), _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(dw), n, H, E, K, int(bool(renorm)),
        _dt(torch.empty(0, dtype=dt_t)), _ptr(out["dlogits"]), _ptr(out["dx_router"]), _ptr(out["dW_gate"]),
        _ptr(out["dbias"]), _ptr(ws), ws.numel(), _stream(dev, stream),
    )
    _check(code, "moe_route_backward")
    return out


@_on_stream
def moe_backward_workspace_size(n, H, I, E, K, dtype) -> int:  # noqa: E741
    return int(load_library().moe_backward_workspace_size(n, H, I, E, K, _dt(torch.empty(0, dtype=dtype))))


@_on_stream
def moe_backward(dy, x, W_gate, W13, W2, K: int, renorm: bool, saved, grads=None, ws=None, stream=None):
    """The layer's backward from moe_forward_train's saved buffers.

    Returns dict(dx, dW_gate (fp32), dbias (fp32), dW13, dW2); `grads` may
    supply any of them preallocated."""
    lib = load_library()
    n, H = x.shape
    E = W_gate.shape[1]
    I = W13.shape[2] // 2  # noqa: E741
    dev, dt_t = x.device, x.dtype
    _need(dy, "dy", (n, H), dt_t, dev)
    _need(x, "x", (n, H))
    _need(W_gate, "W_gate", (H, E), dt_t, dev)
    _need(W13, "W13", (E, H, 2 * I), dt_t, dev)
    _need(W2, "W2", (E, I, H), dt_t, dev)
    shapes = dict(
        logits=((n, E), torch.float32), topk_ids=((n, K), torch.int32), topk_w=((n, K), torch.float32),
        offsets=((E + 1,), torch.int32), perm=((n * K,), torch.int32), inv=((n * K,), torch.int32),
        gate_up=((n * K, 2 * I), dt_t), h=((n * K, I), dt_t), Y_perm=((n * K, H), dt_t),
    )
    for name, (shape, dtype) in shapes.items():
        _need(saved[name], name, shape, dtype, dev)
    gshapes = dict(dx=((n, H), dt_t), dW_gate=((H, E), torch.float32), dbias=((E,), torch.float32),
                   dW13=((E, H, 2 * I), dt_t), dW2=((E, I, H), dt_t))
    grads = dict(grads or {})
    for name, (shape, dtype) in gshapes.items():
        grads.setdefault(name, _empty(shape, dtype, dev))
        _need(grads[name], name, shape, dtype, dev)
    dt = _dt(x)
    ws = _workspace(lib.moe_backward_workspace_size(n, H, I, E, K, dt), dev, ws)
    code = lib.moe_backward(
        _ptr(dy), _ptr(x), _ptr(W_gate), _ptr(W13), _ptr(W2), n, H, I, E, K, int(bool(renorm)), dt,
        *[_ptr(saved[k]) for k in shapes], *[_ptr(grads[k]) for k in gshapes], _ptr(ws), ws.numel(),
        _stream(dev, stream),
    )
    _check(code, "moe_backward")
    return grads


# ---------------------------------------------------------------------------
# FP8 expert weights
# ---------------------------------------------------------------------------


@_on_stream
def moe_quantize_fp8(W, codes=None, scales=None, stream=None):
    """FP8 E4M3 codes (E, N, Kd) uint8 and column scales (E, N) fp32 of weights W (E, Kd, N)."""
    lib = load_library()
    E, Kd, N = W.shape
    dev = W.device
    _need(W, "W", (E, Kd, N))
    codes = _empty((E, N, Kd), torch.uint8, dev) if codes is None else codes
    scales = _empty((E, N), torch.float32, dev) if scales is None else scales
    _need(codes, "codes", (E, N, Kd), torch.uint8, dev)
    _need(scales, "scales", (E, N), torch.float32, dev)
    code = lib.moe_quantize_fp8(_ptr(W), E, Kd, N, _dt(W), _ptr(codes), _ptr(scales), _stream(dev, stream))
    _check(code, "moe_quantize_fp8")
    return codes, scales


@_on_stream
def moe_expert_w13_swiglu_gather_fp8(x, perm, K, offsets, W13q, s13, h=None, stream=None):
    """GEMM1 + SwiGLU with FP8 W13 (codes (E, 2I, H), scales (E, 2I)), rows gathered through perm."""
    lib = load_library()
    n, H = x.shape
    E, I2, _ = W13q.shape
    I = I2 // 2  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H))
    _need(perm, "perm", (n * K,), torch.int32, dev)
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(W13q, "W13q", (E, 2 * I, H), torch.uint8, dev)
    _need(s13, "s13", (E, 2 * I), torch.float32, dev)
    h = _empty((n * K, I), x.dtype, dev) if h is None else h
    _need(h, "h", (n * K, I), x.dtype, dev)
    code = lib.moe_expert_w13_swiglu_gather_fp8(_ptr(x), _ptr(perm), n, K, _ptr(offsets), _ptr(W13q), _ptr(s13), E,
                                                H, I, _dt(x), _ptr(h), _stream(dev, stream))
    _check(code, "moe_expert_w13_swiglu_gather_fp8")
    return h


@_on_stream
def moe_expert_w2_fp8(h, offsets, W2q, s2, Y_perm=None, stream=None):
    """GEMM2 with FP8 W2 (codes (E, H, I), scales (E, H))."""
    lib = load_library()
    rows, I = h.shape  # noqa: E741
    E, H, _ = W2q.shape
    dev = h.device
    _need(h, "h", (rows, I))
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(W2q, "W2q", (E, H, I), torch.uint8, dev)
    _need(s2, "s2", (E, H), torch.float32, dev)
    Y_perm = _empty((rows, H), h.dtype, dev) if Y_perm is None else Y_perm
    _need(Y_perm, "Y_perm", (rows, H), h.dtype, dev)
    code = lib.moe_expert_w2_fp8(_ptr(h), _ptr(offsets), rows, _ptr(W2q), _ptr(s2), E, H, I, _dt(h), _ptr(Y_perm),
                                 _stream(dev, stream))
    _check(code, "moe_expert_w2_fp8")
    return Y_perm


@_on_stream
def moe_forward_fp8(x, W_gate, W13q, s13, W2q, s2, K: int, renorm: bool, bias=None, y=None, ws=None,
                    routing_out=False, stream=None):
    """The layer with FP8 expert weights. Returns y, or (y, logits, topk_ids, topk_w, counts) with routing_out."""
    lib = load_library()
    n, H = x.shape
    E = W_gate.shape[1]
    I = W13q.shape[1] // 2  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H))
    _need(W_gate, "W_gate", (H, E), x.dtype, dev)
    _need(W13q, "W13q", (E, 2 * I, H), torch.uint8, dev)
    _need(s13, "s13", (E, 2 * I), torch.float32, dev)
    _need(W2q, "W2q", (E, H, I), torch.uint8, dev)
    _need(s2, "s2", (E, H), torch.float32, dev)
    if bias is not None:
        _need(bias, "bias", (E,), torch.float32, dev)
    y = _empty((n, H), x.dtype, dev) if y is None else y
    _need(y, "y", (n, H), x.dtype, dev)
    dt = _dt(x)
    ws = _workspace(lib.moe_forward_workspace_size(n, H, I, E, K, dt), dev, ws)
    extra = [None] * 4
    if routing_out:
        extra = [_empty((n, E), torch.float32, dev), _empty((n, K), torch.int32, dev),
                 _empty((n, K), torch.float32, dev), _empty((E,), torch.int32, dev)]
    code = lib.moe_forward_fp8(
        _ptr(x), _ptr(W_gate), _ptr(bias), _ptr(W13q), _ptr(s13), _ptr(W2q), _ptr(s2), n, H, I, E, K,
        int(bool(renorm)), dt, _ptr(y), *[_ptr(t) for t in extra], _ptr(ws), ws.numel(), _stream(dev, stream),
    )
    _check(code, "moe_forward_fp8")
    return (y, *extra) if routing_out else y


# ---------------------------------------------------------------------------
# FP8 activations
# ---------------------------------------------------------------------------


@_on_stream
def moe_quantize_rows_fp8(x, codes=None, scales=None, stream=None):
    """Per-token FP8 E4M3 codes (n, H) uint8 and fp32 scales (n,) of x (n, H)."""
    lib = load_library()
    n, H = x.shape
    dev = x.device
    _need(x, "x", (n, H))
    codes = _empty((n, H), torch.uint8, dev) if codes is None else codes
    scales = _empty((n,), torch.float32, dev) if scales is None else scales
    _need(codes, "codes", (n, H), torch.uint8, dev)
    _need(scales, "scales", (n,), torch.float32, dev)
    _check(lib.moe_quantize_rows_fp8(_ptr(x), n, H, _dt(x), _ptr(codes), _ptr(scales), _stream(dev, stream)),
           "moe_quantize_rows_fp8")
    return codes, scales


def moe_fp8_padded_rows(n: int, E: int, K: int) -> int:
    return int(load_library().moe_fp8_padded_rows(n, E, K))


@_on_stream
def moe_dispatch_fp8(meta, codes_tok, s_tok, K: int, out=None, stream=None):
    """The padded FP8 receive buffer from moe_permute's metadata (`meta`: counts, offsets, perm) and the
    per-token codes/scales. Returns dict(offsets_padded, x_q, x_scale, perm_padded, inv_padded)."""
    lib = load_library()
    n, H = codes_tok.shape
    E = meta["counts"].shape[0]
    dev = codes_tok.device
    R = moe_fp8_padded_rows(n, E, K)
    _need(codes_tok, "codes_tok", (n, H), torch.uint8, dev)
    _need(s_tok, "s_tok", (n,), torch.float32, dev)
    for k, shp in (("counts", (E,)), ("offsets", (E + 1,)), ("perm", (n * K,))):
        _need(meta[k], k, shp, torch.int32, dev)
    shapes = dict(offsets_padded=((E + 1,), torch.int32), x_q=((R, H), torch.uint8), x_scale=((R,), torch.float32),
                  perm_padded=((R,), torch.int32), inv_padded=((n * K,), torch.int32))
    out = dict(out or {})
    for k, (shp, dt) in shapes.items():
        out.setdefault(k, _empty(shp, dt, dev))
        _need(out[k], k, shp, dt, dev)
    _check(lib.moe_dispatch_fp8(_ptr(meta["counts"]), _ptr(meta["offsets"]), _ptr(meta["perm"]), n, E, K,
                                _ptr(codes_tok), _ptr(s_tok), H, *[_ptr(out[k]) for k in shapes],
                                _stream(dev, stream)), "moe_dispatch_fp8")
    return out


@_on_stream
def moe_expert_w13_swiglu_fp8a(x_q, x_scale, offsets_padded, W13q, s13, h=None, stream=None):
    """GEMM1 + SwiGLU on the FP8 receive buffer with FP8 W13 codes; h (rows, I) bf16."""
    lib = load_library()
    R, H = x_q.shape
    E, N, _ = W13q.shape
    I = N // 2  # noqa: E741
    dev = x_q.device
    _need(x_q, "x_q", (R, H), torch.uint8, dev)
    _need(x_scale, "x_scale", (R,), torch.float32, dev)
    _need(offsets_padded, "offsets_padded", (E + 1,), torch.int32, dev)
    _need(W13q, "W13q", (E, N, H), torch.uint8, dev)
    _need(s13, "s13", (E, N), torch.float32, dev)
    h = _empty((R, I), torch.bfloat16, dev) if h is None else h
    _need(h, "h", (R, I), torch.bfloat16, dev)
    _check(lib.moe_expert_w13_swiglu_fp8a(_ptr(x_q), _ptr(x_scale), _ptr(offsets_padded), R, _ptr(W13q), _ptr(s13),
                                          E, H, I, _ptr(h), _stream(dev, stream)), "moe_expert_w13_swiglu_fp8a")
    return h


@_on_stream
def moe_expert_w13_swiglu_gather_fp8a(codes_tok, s_tok, perm, K: int, offsets, W13q, s13, h=None, stream=None):
    """GEMM1 + SwiGLU on FP8 activations read in place: row r of the expert-major order is token perm[r] // K
    of the per-token codes (n, H) and scales (n,). Returns h (n*K, I) bf16."""
    lib = load_library()
    n, H = codes_tok.shape
    E, twoI = s13.shape
    I = twoI // 2  # noqa: E741
    dev = codes_tok.device
    _need(codes_tok, "codes_tok", (n, H), torch.uint8)
    _need(s_tok, "s_tok", (n,), torch.float32, dev)
    _need(perm, "perm", (n * K,), torch.int32, dev)
    _need(offsets, "offsets", (E + 1,), torch.int32, dev)
    _need(W13q, "W13q", (E, 2 * I, H), torch.uint8, dev)
    h = _empty((n * K, I), torch.bfloat16, dev) if h is None else h
    _need(h, "h", (n * K, I), torch.bfloat16, dev)
    _check(lib.moe_expert_w13_swiglu_gather_fp8a(_ptr(codes_tok), _ptr(s_tok), _ptr(perm), n, K, _ptr(offsets),
                                                 _ptr(W13q), _ptr(s13), E, H, I, _ptr(h), _stream(dev, stream)),
           "moe_expert_w13_swiglu_gather_fp8a")
    return h


@_on_stream
def moe_expert_w13_swiglu_from_ids_fp8(x, topk_ids, W13q, s13, ep: int = 1, h=None, out=None, stream=None):
    """GEMM1 with FP8 weights on a decode-sized batch straight from the routing ids: h (n*K, I) bf16 and the
    moe_permute metadata dict (counts, offsets, splits, perm, inv) from one launch. Returns (h, meta)."""
    lib = load_library()
    n, H = x.shape
    K = topk_ids.shape[1]
    E, I2, _ = W13q.shape
    I = I2 // 2  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H), torch.bfloat16)
    _need(topk_ids, "topk_ids", (n, K), torch.int32, dev)
    _need(W13q, "W13q", (E, 2 * I, H), torch.uint8, dev)
    _need(s13, "s13", (E, 2 * I), torch.float32, dev)
    h = _empty((n * K, I), torch.bfloat16, dev) if h is None else h
    _need(h, "h", (n * K, I), torch.bfloat16, dev)
    out = dict(out or {})
    for name, shape in (("counts", (E,)), ("offsets", (E + 1,)), ("splits", (ep,)), ("perm", (n * K,)),
                        ("inv", (n * K,))):
        out.setdefault(name, _empty(shape, torch.int32, dev))
        _need(out[name], name, shape, torch.int32, dev)
    code = lib.moe_expert_w13_swiglu_from_ids_fp8(
        _ptr(x), _ptr(topk_ids), n, K, _ptr(W13q), _ptr(s13), E, H, I, ep, _ptr(h), _ptr(out["counts"]),
        _ptr(out["offsets"]), _ptr(out["splits"]), _ptr(out["perm"]), _ptr(out["inv"]), _stream(dev, stream),
    )
    _check(code, "moe_expert_w13_swiglu_from_ids_fp8")
    return h, out


@_on_stream
def moe_expert_w13_swiglu_from_ids_fp8a(codes_tok, s_tok, topk_ids, W13q, s13, ep: int = 1, h=None, out=None,
                                        stream=None):
    """The FP8 x FP8 GEMM1 of a decode-sized batch straight from the routing ids: h (n*K, I) bf16 and the
    moe_permute metadata dict (counts, offsets, splits, perm, inv) from one launch. Returns (h, meta)."""
    lib = load_library()
    n, H = codes_tok.shape
    K = topk_ids.shape[1]
    E, I2, _ = W13q.shape
    I = I2 // 2  # noqa: E741
    dev = codes_tok.device
    _need(codes_tok, "codes_tok", (n, H), torch.uint8)
    _need(s_tok, "s_tok", (n,), torch.float32, dev)
    _need(topk_ids, "topk_ids", (n, K), torch.int32, dev)
    _need(W13q, "W13q", (E, 2 * I, H), torch.uint8, dev)
    _need(s13, "s13", (E, 2 * I), torch.float32, dev)
    h = _empty((n * K, I), torch.bfloat16, dev) if h is None else h
    _need(h, "h", (n * K, I), torch.bfloat16, dev)
    out = dict(out or {})
    for name, shape in (("counts", (E,)), ("offsets", (E + 1,)), ("splits", (ep,)), ("perm", (n * K,)),
                        ("inv", (n * K,))):
        out.setdefault(name, _empty(shape, torch.int32, dev))
        _need(out[name], name, shape, torch.int32, dev)
    code = lib.moe_expert_w13_swiglu_from_ids_fp8a(
        _ptr(codes_tok), _ptr(s_tok), _ptr(topk_ids), n, K, _ptr(W13q), _ptr(s13), E, H, I, ep, _ptr(h),
        _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["splits"]), _ptr(out["perm"]), _ptr(out["inv"]),
        _stream(dev, stream),
    )
    _check(code, "moe_expert_w13_swiglu_from_ids_fp8a")
    return h, out


@_on_stream
def moe_expert_w2_fp8a(h_q, h_scale, offsets_padded, W2q, s2, Y_perm=None, stream=None):
    """GEMM2 with FP8 activations over the padded receive buffer: Y_perm (rows_max, H) bf16 from h quantized
    per row (h_q (rows_max, I) uint8, h_scale (rows_max,) fp32) and the FP8 W2 codes/scales."""
    lib = load_library()
    R, I = h_q.shape  # noqa: E741
    E, H = s2.shape
    dev = h_q.device
    _need(h_q, "h_q", (R, I), torch.uint8)
    _need(h_scale, "h_scale", (R,), torch.float32, dev)
    _need(offsets_padded, "offsets_padded", (E + 1,), torch.int32, dev)
    _need(W2q, "W2q", (E, H, I), torch.uint8, dev)
    Y_perm = _empty((R, H), torch.bfloat16, dev) if Y_perm is None else Y_perm
    _need(Y_perm, "Y_perm", (R, H), torch.bfloat16, dev)
    _check(lib.moe_expert_w2_fp8a(_ptr(h_q), _ptr(h_scale), _ptr(offsets_padded), R, _ptr(W2q), _ptr(s2), E, H, I,
                                  _ptr(Y_perm), _stream(dev, stream)), "moe_expert_w2_fp8a")
    return Y_perm


def moe_forward_fp8a_workspace_size(n, H, I, E, K) -> int:  # noqa: E741
    return int(load_library().moe_forward_fp8a_workspace_size(n, H, I, E, K))


@_on_stream
def moe_forward_fp8a(x, W_gate, W13q, s13, W2q, s2, K: int, renorm: bool, bias=None, y=None, ws=None,
                     routing_out=False, stream=None):
    """The layer with FP8 activations and FP8 weights. Returns y, or (y, logits, topk_ids, topk_w, counts)."""
    lib = load_library()
    n, H = x.shape
    E = W_gate.shape[1]
    I = W13q.shape[1] // 2  # noqa: E741
    dev = x.device
    _need(x, "x", (n, H), torch.bfloat16)
    _need(W_gate, "W_gate", (H, E), torch.bfloat16, dev)
    _need(W13q, "W13q", (E, 2 * I, H), torch.uint8, dev)
    _need(s13, "s13", (E, 2 * I), torch.float32, dev)
    _need(W2q, "W2q", (E, H, I), torch.uint8, dev)
    _need(s2, "s2", (E, H), torch.float32, dev)
    if bias is not None:
        _need(bias, "bias", (E,), torch.float32, dev)
    y = _empty((n, H), torch.bfloat16, dev) if y is None else y
    _need(y, "y", (n, H), torch.bfloat16, dev)
    ws = _workspace(lib.moe_forward_fp8a_workspace_size(n, H, I, E, K), dev, ws)
    extra = [None] * 4
    if routing_out:
        extra = [_empty((n, E), torch.float32, dev), _empty((n, K), torch.int32, dev),
                 _empty((n, K), torch.float32, dev), _empty((E,), torch.int32, dev)]
    code = lib.moe_forward_fp8a(
        _ptr(x), _ptr(W_gate), _ptr(bias), _ptr(W13q), _ptr(s13), _ptr(W2q), _ptr(s2), n, H, I, E, K,
        int(bool(renorm)), MOE_BF16, _ptr(y), *[_ptr(t) for t in extra], _ptr(ws), ws.numel(), _stream(dev, stream),
    )
    _check(code, "moe_forward_fp8a")
    return (y, *extra) if routing_out else y

