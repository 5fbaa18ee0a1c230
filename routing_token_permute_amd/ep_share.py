"""One GPU's expert-parallel share with two micro-batches on two HIP streams.

What it models: the rows this GPU received for its local experts in an
expert-parallel exchange arrive rank-major; `_permute` makes them
expert-major for the grouped GEMM, the local experts run, and `_unpermute`
puts the results back in arrival order before the reverse exchange ("0. goin",
§2.2, torchtitan's standard dispatcher). With two micro-batches, one
micro-batch's expert GEMMs cover the other's dispatch/combine work: the
Domino-style interleave of "XTuner Domino EP" (execution path: a compute
stream, a communication stream and events placed at the first consumer) and
"大模型系统中的通算融合" §3.1 (MB0's expert GEMM covers MB1's dispatch, MB1's
covers MB0's combine). On one GPU the exchange itself is absent; the permute
and unpermute kernels stand on the second stream.

This module only orders library calls on streams; every step runs in the
HIP kernels of libmoe.so (moe_permute with K = 1, moe_grouped_swiglu,
moe_unpermute_combine with unit weights).

The fused schedule does the same work with no expert-major copies: the
permute writes only the metadata, the first GEMM reads the received rows
through perm (the `x[T_b]` gather of "MoE 分布式推理基础（基于 vLLM）" §2.3),
and the second GEMM stores each output row straight at its arrival position
(the weighted scatter epilogue with unit weights, as in the second fused MoE
layer of "大模型系统中的通算融合" §4.2.5). A weight of exactly 1 leaves the
fp32 accumulator unchanged, so the result is bitwise the serial schedule's.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _lib


@dataclasses.dataclass
class MicroBatch:
    """Device buffers of one micro-batch: received rows, their local expert ids
    (R, 1) int32, and the outputs/scratch the schedule fills."""

    x: torch.Tensor  # (R, H) received rows, arrival order
    eid: torch.Tensor  # (R, 1) int32 local expert of each row
    meta: dict = dataclasses.field(default_factory=dict)
    Y_perm: Optional[torch.Tensor] = None
    out: Optional[torch.Tensor] = None
    ws_perm: Optional[torch.Tensor] = None
    ws_gemm: Optional[torch.Tensor] = None
    h: Optional[torch.Tensor] = None  # fused schedule: SwiGLU activations, expert-major
    ones: Optional[torch.Tensor] = None  # fused schedule: unit weights (R, 1) fp32
    out_fused: Optional[torch.Tensor] = None  # fused schedule: outputs, arrival order


def prepare(mb: MicroBatch, E_local: int, I: int) -> MicroBatch:  # noqa: E741
    """Allocate every buffer the schedule writes (torch allocations, outside the timed work)."""
    R, H = mb.x.shape
    dev = mb.x.device
    lib = _lib.load_library()
    mb.meta = {
        "x_perm": torch.empty((R, H), dtype=mb.x.dtype, device=dev),
        "counts": torch.empty((E_local,), dtype=torch.int32, device=dev),
        "offsets": torch.empty((E_local + 1,), dtype=torch.int32, device=dev),
        "splits": torch.empty((1,), dtype=torch.int32, device=dev),
        "perm": torch.empty((R,), dtype=torch.int32, device=dev),
        "inv": torch.empty((R,), dtype=torch.int32, device=dev),
    }
    mb.Y_perm = torch.empty((R, H), dtype=mb.x.dtype, device=dev)
    mb.out = torch.empty((R, H), dtype=mb.x.dtype, device=dev)
    mb.ws_perm = torch.empty(lib.moe_permute_workspace_size(R, E_local, 1), dtype=torch.uint8, device=dev)
    dt = _lib._dt(mb.x)
    mb.ws_gemm = torch.empty(lib.moe_grouped_swiglu_workspace_size(R, I, dt), dtype=torch.uint8, device=dev)
    mb.h = torch.empty((R, I), dtype=mb.x.dtype, device=dev)
    mb.ones = torch.ones((R, 1), dtype=torch.float32, device=dev)
    mb.out_fused = torch.empty((R, H), dtype=mb.x.dtype, device=dev)
    return mb


def permute(mb: MicroBatch, E_local: int, stream) -> None:
    _lib.moe_permute(mb.eid, mb.x, E_local, out=mb.meta, ws=mb.ws_perm, stream=stream)


def experts(mb: MicroBatch, W13: torch.Tensor, W2: torch.Tensor, stream) -> None:
    _lib.moe_grouped_swiglu(mb.meta["x_perm"], mb.meta["offsets"], W13, W2, Y_perm=mb.Y_perm, ws=mb.ws_gemm,
                            stream=stream)


def unpermute(mb: MicroBatch, stream) -> None:
    R = mb.x.shape[0]
    _lib.moe_unpermute_combine(mb.Y_perm, mb.meta["inv"], None, R, 1, y=mb.out, stream=stream)


def permute_meta(mb: MicroBatch, E_local: int, stream) -> None:
    """counts, offsets, perm and inv only (no expert-major copy of the rows)."""
    meta = {k: v for k, v in mb.meta.items() if k != "x_perm"}
    _lib.moe_permute(mb.eid, None, E_local, out=meta, ws=mb.ws_perm, stream=stream)


def experts_fused(mb: MicroBatch, W13: torch.Tensor, W2: torch.Tensor, stream, packed=None) -> None:
    """GEMM1 + SwiGLU reading the received rows through perm, then GEMM2 storing
    each row at its arrival position. `packed`: (W13p, W2p) as moe_pack_w13 /
    moe_pack_w2 write them, used in place of W13 and W2 (the same results)."""
    perm, offsets = mb.meta["perm"], mb.meta["offsets"]
    if packed is not None:
        I = mb.h.shape[1]  # noqa: E741
        _lib.moe_expert_w13_swiglu_gather_packed(mb.x, perm, 1, offsets, packed[0], I, h=mb.h, stream=stream)
        _lib.moe_expert_w2_scatter_packed(mb.h, offsets, perm, mb.ones, packed[1], mb.x.shape[1], Y_tok=mb.out_fused,
                                          stream=stream)
        return
    _lib.moe_expert_w13_swiglu_gather(mb.x, perm, 1, offsets, W13, h=mb.h, stream=stream)
    _lib.moe_expert_w2_scatter(mb.h, offsets, perm, mb.ones, W2, Y_tok=mb.out_fused, stream=stream)


def run_fused(a: MicroBatch, b: MicroBatch, W13, W2, E_local: int, stream, packed=None) -> None:
    """Both micro-batches on one stream with the permute and unpermute folded
    into the GEMMs; outputs in out_fused. `packed`: optional (W13p, W2p)."""
    for mb in (a, b):
        permute_meta(mb, E_local, stream)
        experts_fused(mb, W13, W2, stream, packed)


def run_serial(a: MicroBatch, b: MicroBatch, W13, W2, E_local: int, stream) -> None:
    """Both micro-batches, every step on one stream (the serial control)."""
    for mb in (a, b):
        permute(mb, E_local, stream)
        experts(mb, W13, W2, stream)
        unpermute(mb, stream)


def run_two_streams(a: MicroBatch, b: MicroBatch, W13, W2, E_local: int, compute, comm) -> None:
    """permute(A); [experts(A) || permute(B)]; [experts(B) || unpermute(A)]; unpermute(B).

    `compute` runs the expert GEMMs, `comm` the permute/unpermute kernels;
    each dependency is an event recorded after the producer and waited on by
    the first consumer only. Both streams must be current-device torch
    streams; the caller synchronises on both when it needs the outputs.
    """
    ev = {k: torch.cuda.Event() for k in ("permA", "permB", "gemmA", "gemmB")}
    permute(a, E_local, comm)
    ev["permA"].record(comm)
    permute(b, E_local, comm)
    ev["permB"].record(comm)
    compute.wait_event(ev["permA"])
    experts(a, W13, W2, compute)
    ev["gemmA"].record(compute)
    compute.wait_event(ev["permB"])
    experts(b, W13, W2, compute)
    ev["gemmB"].record(compute)
    comm.wait_event(ev["gemmA"])
    unpermute(a, comm)
    comm.wait_event(ev["gemmB"])
    unpermute(b, comm)


# ---------------------------------------------------------------------------
# CU-masked stream split
# ---------------------------------------------------------------------------
#
# "大模型系统中的通算融合" §6.4 models the split of a GPU's compute units
# between communication and compute as T_total(S_comm) = max(T_compute(S -
# S_comm), T_comm(S_comm)) + T_sync. Here the permute/unpermute stream gets
# S_comm compute units and the GEMM stream the rest, through HIP stream CU
# masks; the grouped GEMM sizes its persistent grid by its stream's mask.


def comm_cu_bits(n_comm: int, n_cus: int = 256, xcds: int = 8):
    """CU indices for the communication stream: n_comm / xcds per XCD, spread
    so that they stay balanced across XCDs whether the mask's bit i counts CUs
    XCD by XCD (i // (n_cus / xcds)) or round-robin (i % xcds)."""
    per = n_cus // xcds
    if n_comm % xcds or not 0 < n_comm <= n_cus // 2:
        raise ValueError(f"n_comm={n_comm} must be a positive multiple of {xcds} up to {n_cus // 2}")
    m = n_comm // xcds
    bits = []
    for x in range(xcds):
        picked = []
        z = 0
        while len(picked) < m:
            for y in range(per // xcds):
                b = x * per + (x + xcds * y + z) % per
                if b not in picked:
                    picked.append(b)
                if len(picked) == m:
                    break
            z += 1
        bits += picked
    return sorted(bits)


class MaskedStreams:
    """A compute stream and a communication stream with complementary CU masks
    (HIP streams created with hipExtStreamCreateWithCUMask, default priority),
    usable as torch streams. Call close() to destroy them."""

    def __init__(self, n_comm: int, device):
        import ctypes

        self._hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch has loaded
        n_cus = torch.cuda.get_device_properties(device).multi_processor_count
        comm = set(comm_cu_bits(n_comm, n_cus))
        words = (n_cus + 31) // 32

        def mask(bits):
            m = (ctypes.c_uint32 * words)()
            for b in bits:
                m[b // 32] |= 1 << (b % 32)
            return m

        self._handles = []
        streams = []
        for bits in ([b for b in range(n_cus) if b not in comm], sorted(comm)):
            h = ctypes.c_void_p()
            rc = self._hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), ctypes.c_uint32(words), mask(bits))
            if rc != 0:
                self.close()
                raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({rc})")
            self._handles.append(h)
            streams.append(torch.cuda.ExternalStream(h.value, device=device))
        self.compute, self.comm = streams
        self.n_comm, self.n_compute = n_comm, n_cus - n_comm

    def close(self):
        for h in self._handles:
            self._hip.hipStreamDestroy(h)
        self._handles = []
