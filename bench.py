"""Benchmark of the MoE expert-layer forward on one MI355X.

One step = one `moe_forward` call (router GEMM, softmax/top-K, counts,
offsets and permutation, grouped SwiGLU GEMM1 with the row gather fused,
GEMM2, weighted combine) over the OLMoE-shaped layer: n=4096 tokens, H=2048,
I=1024, E=64 experts, top-8, bf16 storage with fp32 accumulation, synthetic
seeded inputs already resident in HBM.

Prints ONE JSON line with tokens/s for the whole layer, the grouped-GEMM
TFLOP/s, per-stage times and bandwidths, the roofline of the dominant kernel
(the GEMM1 + SwiGLU launch) timed with HIP events on the stream it runs on,
and the CPU oracle timed on the host as a reported baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/s + grouped-GEMM TFLOP/s (% bf16 peak), OLMoE n=4096"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="olmoe_bf16",
                   choices=["olmoe_bf16", "olmoe_skewed_bf16", "decode_bf16", "ep_share_bf16", "olmoe_train_bf16",
                            "decode_fp8", "olmoe_fp8", "decode_fp8a", "olmoe_fp8a"])
    p.add_argument("--stage-reps", type=int, default=20)
    p.add_argument("--settle-ms", type=float, default=300.0,
                   help="after the warmup steps, keep running untimed steps until this much wall time has passed "
                        "since the first (the device's clocks ramp up under load)")
    p.add_argument("--comm-cus", type=int, nargs="*", default=[8, 16, 32, 64],
                   help="ep_share_bf16: compute units given to the permute/unpermute stream in the CU-masked runs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--headline-only", action="store_true",
                   help="olmoe_bf16: leave out the other configurations (tiny, skewed, decode, EP share)")
    p.add_argument("--profile-forward", type=int, default=0, metavar="N",
                   help="only run N moe_forward calls of the workload (for rocprofv3 counter passes)")
    p.add_argument("--profile-layer", choices=["packed", "bf16", "fp8a", "persistent", "persistent_packed"],
                   default="packed",
                   help="with --profile-forward: moe_forward_packed (bf16, the weights packed once first), "
                        "moe_forward (bf16), moe_forward_fp8a, moe_forward_persistent or "
                        "moe_forward_persistent_packed")
    p.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                   help="turn rocprofv3 --pmc csv directories into the per-kernel counter summary printed on stdout")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle wall time for the CPU baseline")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy kernel (a known-bytes check of the HBM counters)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# rocprofv3 counter summaries
# ---------------------------------------------------------------------------
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_moe_forward_olmoe_n4096.md")
GEMM_SOURCE = os.path.join(ROOT, "routing_token_permute_amd", "csrc", "grouped_gemm.hip")
COPY_BYTES = 1 << 30


def _source_hash():
    """Hash of the GEMM source's code: comment text and blank lines are left out,
    so that editing a comment does not orphan the counter summary."""
    import hashlib
    import re

    code = []
    for line in open(GEMM_SOURCE, encoding="utf-8"):
        line = re.sub(r"//.*", "", line).rstrip()
        if line:
            code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def _kernel_label(name):
    if "route_bf16_kernel" in name or "route_f32_kernel" in name or "route_bf16_rows_kernel" in name:
        return "route"
    for k in ("permute_single_kernel", "permute_count_kernel", "permute_place_kernel", "gather_rows_kernel",
              "sum_slots_kernel"):
        if k in name:
            return k.replace("_kernel", "")
    if "combine_kernel" in name:
        return "combine"
    if "gemm_bf16_kernel<" in name:
        args = name.split("gemm_bf16_kernel<", 1)[1].split(">", 1)[0].split(",")
        gated, bm = args[0].strip() == "true", args[3].strip()
        ids = len(args) > 8 and args[8].strip() == "true"
        packed = len(args) > 9 and args[9].strip() == "true"
        return (("gemm1_swiglu" if gated else "gemm2") + ("_from_ids" if ids else "") + f"_bm{bm}"
                + ("_packed" if packed else ""))
    if "gemm_f8f8_kernel<" in name:
        args = name.split("gemm_f8f8_kernel<", 1)[1].split(">", 1)[0].split(",")
        gated, gather, bm = args[0].strip() == "true", args[1].strip() == "true", args[2].strip()
        ids = len(args) > 7 and args[7].strip() == "true"
        return (("gemm1_swiglu_f8f8" if gated else "gemm2_f8f8") + ("_from_ids" if ids else "_gather" if gather else "")
                + f"_bm{bm}")
    for k, lab in (("quantize_rows_kernel", "quantize_rows_fp8"), ("dispatch_fp8_kernel", "dispatch_fp8"),
                   ("quantize_fp8_kernel", "quantize_weights_fp8"), ("fused_ffn_kernel", "fused_ffn"),
                   ("fill_zero_kernel", "fill_zero"), ("pack_weights_kernel", "pack_weights")):
        if k in name:
            return lab
    if "FillFunctor" in name:
        return "fill_1GiB"
    if "copy" in name.lower() or "elementwise" in name.lower():
        return "copy_1GiB"
    return name.split("(")[0][-60:]


def _summarize_counters(dirs):
    """Per-kernel means over the dispatches of every --pmc pass (the first
    dispatch of each kernel, with cold caches, is left out when there are more),
    and the figures derived from them: MFMA busy share of the SIMD cycles, bf16
    MFMA TFLOP/s, LDS / TA / TD busy shares of the CU cycles, L2 hit rate, and
    HBM bytes from the per-size memory request counters of L2 (32/64/128-byte
    reads, 64-byte and other writes)."""
    import csv
    import glob
    from collections import defaultdict

    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(list)
    agent = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Agent_Type") == "GPU":
                    agent = {k: int(r[k]) for k in ("Num_Xcc", "Cu_Count", "Simd_Count", "Max_Engine_Clk_Fcompute")}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            per = defaultdict(list)
            for r in csv.DictReader(open(f)):
                per[(r["Kernel_Name"], r["Counter_Name"])].append(
                    (int(r["Dispatch_Id"]), float(r["Counter_Value"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
            for (kname, cname), rows in per.items():
                rows.sort()
                if len(rows) > 1:
                    rows = rows[1:]
                lab = _kernel_label(kname)
                vals[lab][cname] += [v for _, v, _ in rows]
                durs[lab] += [t for _, _, t in rows]
    xcc = agent.get("Num_Xcc", 8)
    cus = agent.get("Cu_Count", 256)
    simds = agent.get("Simd_Count", 1024)
    out = {"agent": agent, "source_sha256_16": _source_hash(), "kernels": {}}
    for lab, cv in sorted(vals.items()):
        m = {c: sum(v) / len(v) for c, v in cv.items()}
        dur = sum(durs[lab]) / len(durs[lab]) * 1e-9
        k = {"duration_us": round(dur * 1e6, 2), "dispatches_per_pass": len(next(iter(cv.values())))}
        cyc = m.get("GRBM_GUI_ACTIVE", 0) / xcc
        if cyc:
            k["sclk_GHz_effective"] = round(cyc / dur / 1e9, 3)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                k["mfma_busy"] = round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cyc), 4)
            for c, key in (("SQ_LDS_IDX_ACTIVE", "lds_busy"), ("TA_TA_BUSY_sum", "ta_busy"), ("TD_TD_BUSY_sum", "td_busy")):
                if c in m:
                    k[key] = round(m[c] / (cus * cyc), 4)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
            k["mfma_bf16_TFLOP/s"] = round(m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / dur / 1e12, 1)
        if "SQ_INSTS_VALU_MFMA_MOPS_F8" in m:
            k["mfma_f8_TFLOP/s"] = round(m["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512 / dur / 1e12, 1)
        if "SQ_WAIT_ANY" in m and m.get("SQ_WAVE_CYCLES"):
            k["wave_wait_share"] = round(m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"], 4)
        if "SQ_LDS_BANK_CONFLICT" in m:
            k["lds_bank_conflict_cycles"] = m["SQ_LDS_BANK_CONFLICT"]
        if m.get("TCC_REQ_sum"):
            k["l2_hit_rate"] = round(m.get("TCC_HIT_sum", 0) / m["TCC_REQ_sum"], 4)
        if "TCC_EA0_RDREQ_128B_sum" in m:
            rd = 32 * m.get("TCC_EA0_RDREQ_32B_sum", 0) + 64 * m.get("TCC_EA0_RDREQ_64B_sum", 0) + \
                128 * m["TCC_EA0_RDREQ_128B_sum"]
            k["hbm_read_bytes"] = round(rd)
        if "TCC_EA0_WRREQ_sum" in m:
            w64 = m.get("TCC_EA0_WRREQ_64B_sum", 0)
            k["hbm_write_bytes"] = round(64 * w64 + 32 * (m["TCC_EA0_WRREQ_sum"] - w64))
        if "hbm_read_bytes" in k and "hbm_write_bytes" in k:
            k["hbm_bytes"] = k["hbm_read_bytes"] + k["hbm_write_bytes"]
            k["hbm_GB/s"] = round(k["hbm_bytes"] / dur / 1e9, 1)
        out["kernels"][lab] = k
    print(json.dumps(out, indent=1))


def _traffic_bytes():
    """HBM bytes per GEMM1 launch (read + write, from L2's per-size memory request
    counters) from the committed counter summary, or None when the summary is
    missing or was taken on a different GEMM source."""
    try:
        d = json.loads(open(COUNTERS_FILE).read().split("\n```json\n", 1)[-1].split("\n```", 1)[0])
    except (OSError, ValueError):
        return None
    if d.get("source_sha256_16") != _source_hash():
        return None
    return d.get("kernels", {}).get("gemm1_swiglu_bm256_packed", {}).get("hbm_bytes")


def _copy_calibration():
    import torch

    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}))


def _warm(fn, n, torch, settle_ms):
    """n untimed calls of fn(), then more until settle_ms of wall time have passed
    since the first. Under load the device's clocks take tens of milliseconds to
    settle, and calls in that window run several percent slower."""
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


class _TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: recording it writes a
    timestamp without the system-scope cache write-back and invalidation a default event performs, which
    would otherwise slow the kernels that follow it. The HIP runtime is the one the library runs on
    (its symbols resolved through the library's handle)."""

    _DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        self._lib = _moe_lib()
        self._ct = ctypes
        h = ctypes.c_void_p()
        if self._lib.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(self._DISABLE_SYSTEM_FENCE)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.handle = h.value

    def elapsed_ms(self, end):
        ct = self._ct
        if self._lib.hipEventSynchronize(ct.c_void_p(end.handle)) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ct.c_float()
        if self._lib.hipEventElapsedTime(ct.byref(ms), ct.c_void_p(self.handle), ct.c_void_p(end.handle)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        try:
            self._lib.hipEventDestroy(self._ct.c_void_p(self.handle))
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass


class _TorchTimingEvent:
    """torch.cuda.Event with the interface of _TimingEvent."""

    def __init__(self, torch):
        self.ev = torch.cuda.Event(enable_timing=True)
        self.ev.record()  # torch creates the event on its first record
        self.handle = self.ev.cuda_event

    def elapsed_ms(self, end):
        end.ev.synchronize()
        return self.ev.elapsed_time(end.ev)


def _moe_lib():
    import routing_token_permute_amd as moe

    return moe.load_library()


def _time_region(fn, reps, torch):
    """Average ms per call of fn() over `reps` calls, HIP events on the current stream."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def _time_region_graph(fn, reps, torch):
    """Average ms per call of fn() with `reps` calls captured in one HIP graph
    and the graph replayed: the host's per-call launch cost (which exceeds the
    kernel time of the small decode-size stages) drops out. Returns the eager
    figure instead if capture fails."""
    dev = torch.device("cuda:0")
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    try:
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
    except RuntimeError:
        torch.cuda.synchronize()
        return _time_region(fn, reps, torch)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(3):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (3 * reps)


def _time_each(fn, reps, torch, flush=None):
    """Per-call ms of fn() over `reps` calls, one HIP event pair per call on the
    current stream; flush() (not timed) runs before each call when given."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        if flush is not None:
            flush()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def _pcts(ms):
    q = np.percentile(np.asarray(ms), [10, 50, 90])
    return {"p10_ms": round(float(q[0]), 5), "p50_ms": round(float(q[1]), 5), "p90_ms": round(float(q[2]), 5)}


def _to_dev_bits(w, name, dev, torch):
    b = w.bits(name)
    if w.dtype == "bf16":
        return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.float32)).to(dev)


def _expert_load(counts):
    """Per-expert row counts n_e: histogram, coefficient of variation, hot/empty experts."""
    c = np.asarray(counts, dtype=np.int64)
    edges = [0, 1, 2, 3, 5, 9, 17, 33, 65, 129, 257, 513, 1025, 2049, 4097, 1 << 30]
    hist = {}
    for lo, hi in zip(edges[:-1], edges[1:]):
        k = int(((c >= lo) & (c < hi)).sum())
        if k:
            hist[f"{lo}" if hi == lo + 1 else f"{lo}-{hi - 1}"] = k
    mu = float(c.mean())
    return {"n_e_hist": hist, "cv": round(float(c.std()) / mu, 4) if mu > 0 else None,
            "n_e_min": int(c.min()), "n_e_max": int(c.max()), "experts_hit": int((c > 0).sum()),
            "empty_experts": int((c == 0).sum())}


def _layer_bench(w, args, torch, moe, dev, detail):
    """One layer workload: moe_forward timed over args.steps calls (HIP events on the
    current stream, after the warmup and clock-settle phase), the stages moe_forward
    enqueues timed alone from HIP-graph replays, the expert load, and GEMM1's roofline
    (MFMA-bound or weight-stream-bound by its algorithmic intensity against the ridge)."""
    n, H, I, E, K = w.n, w.H, w.I, w.E, w.K  # noqa: E741
    x, Wg, W13, W2 = (_to_dev_bits(w, k, dev, torch) for k in ("x", "W_gate", "W13", "W2"))
    bias = None if w.bias is None else torch.from_numpy(w.bias).to(dev)
    tdt = x.dtype
    esz = 2 if w.dtype == "bf16" else 4
    y = torch.empty((n, H), dtype=tdt, device=dev)
    ws = torch.empty(moe.moe_forward_workspace_size(n, H, I, E, K, tdt), dtype=torch.uint8, device=dev)

    # bf16 layers run over weights packed once into the GEMMs' tile order (moe_pack_w13 / moe_pack_w2,
    # before any timing: the weights are static); the plain-layout moe_forward is timed beside it.
    packed = w.dtype == "bf16"
    if packed:
        W13p, W2p = moe.moe_pack_w13(W13), moe.moe_pack_w2(W2)

    def step_plain():
        moe.moe_forward(x, Wg, W13, W2, K, w.renorm, bias=bias, y=y, ws=ws)

    def step():
        if packed:
            moe.moe_forward_packed(x, Wg, W13p, W2p, K, w.renorm, bias=bias, y=y, ws=ws)
        else:
            step_plain()

    # The timed steps record a pair of HIP events around the layer's GEMM1 launch (moe_forward_packed's or
    # moe_forward_timed's event arguments, on the stream the layer runs on), which gives the dominant
    # kernel's duration inside the timed region.
    # The events skip the system-scope fence on record, so they cost the steps no cache write-back.
    n_warm_ev = 4  # event pairs recorded before the timed region, so that no first record falls inside it
    try:
        g1_ev = [(_TimingEvent(), _TimingEvent()) for _ in range(args.steps + n_warm_ev)]
        fence_free = True
    except RuntimeError:  # the runtime refused the flag: torch's default timing events instead
        g1_ev = [(_TorchTimingEvent(torch), _TorchTimingEvent(torch)) for _ in range(args.steps + n_warm_ev)]
        fence_free = False
    g1_iter = iter(g1_ev)

    def step_timed():
        a_, b_ = next(g1_iter)
        if packed:
            moe.moe_forward_packed(x, Wg, W13p, W2p, K, w.renorm, bias=bias, y=y, ws=ws, gemm1_begin=a_.handle,
                                   gemm1_end=b_.handle)
        else:
            moe.moe_forward_timed(x, Wg, W13, W2, K, w.renorm, a_.handle, b_.handle, bias=bias, y=y, ws=ws)

    # The timed call path itself first, events included (its first call in a process can stall the host for
    # tens of milliseconds), then the warm-up and clock-settle phase right before the timed region.
    for _ in range(n_warm_ev):
        step_timed()
    g1_ev = g1_ev[n_warm_ev:]
    _warm(step, args.warmup, torch, args.settle_ms)
    t0 = time.perf_counter()
    ms = _time_region(step_timed, args.steps, torch)
    wall = time.perf_counter() - t0
    g1_live_ms = sum(a_.elapsed_ms(b_) for a_, b_ in g1_ev) / len(g1_ev)
    spread = _pcts(_time_each(step, max(args.steps, 10), torch))
    ms_plain = None
    if packed:
        _warm(step_plain, args.warmup, torch, 0)
        ms_plain = _time_region(step_plain, args.steps, torch)
    logits, ids, wts = moe.moe_route(x, Wg, bias, K, w.renorm)
    meta = moe.moe_permute(ids, None, E)
    h = moe.moe_expert_w13_swiglu_gather(x, meta["perm"], K, meta["offsets"], W13)
    Yp = moe.moe_expert_w2(h, meta["offsets"], W2)
    yc = moe.moe_unpermute_combine(Yp, meta["inv"], wts, n, K)
    torch.cuda.synchronize()
    counts = meta["counts"].cpu().numpy()
    # Decode-sized bf16 batches: the layer runs GEMM1 straight from the ids (the GEMM places the pairs
    # itself and writes the metadata) in place of moe_permute + the gathered GEMM1.
    try:
        h_ids, meta_ids = moe.moe_expert_w13_swiglu_from_ids(x, ids, W13)
    except moe.MoEError:
        h_ids = meta_ids = None
    R = args.stage_reps
    if packed:  # the GEMM stages the timed layer runs: over the packed weights
        g1_call = lambda: moe.moe_expert_w13_swiglu_gather_packed(x, meta["perm"], K, meta["offsets"], W13p, I, h=h)  # noqa: E731
        g2_call = lambda: moe.moe_expert_w2_packed(h, meta["offsets"], W2p, H, Y_perm=Yp)  # noqa: E731
        ids_call = lambda: moe.moe_expert_w13_swiglu_from_ids_packed(x, ids, W13p, I, h=h_ids, out=meta_ids)  # noqa: E731
    else:
        g1_call = lambda: moe.moe_expert_w13_swiglu_gather(x, meta["perm"], K, meta["offsets"], W13, h=h)  # noqa: E731
        g2_call = lambda: moe.moe_expert_w2(h, meta["offsets"], W2, Y_perm=Yp)  # noqa: E731
        ids_call = lambda: moe.moe_expert_w13_swiglu_from_ids(x, ids, W13, h=h_ids, out=meta_ids)  # noqa: E731
    st = {
        "route": _time_region_graph(lambda: moe.moe_route(x, Wg, bias, K, w.renorm, logits=logits, topk_ids=ids, topk_w=wts), R, torch),
        "permute": _time_region_graph(lambda: moe.moe_permute(ids, None, E, out=meta), R, torch),
        "gemm1_swiglu": _time_region_graph(g1_call, R, torch),
        "gemm2": _time_region_graph(g2_call, R, torch),
        "combine": _time_region_graph(lambda: moe.moe_unpermute_combine(Yp, meta["inv"], wts, n, K, y=yc), R, torch),
    }
    if meta_ids is not None:
        st["gemm1_swiglu_from_ids"] = _time_region_graph(ids_call, R, torch)
    if packed and detail:  # the same GEMMs over the plain weight layout
        st["alt_gemm1_swiglu_plain_weights"] = _time_region_graph(
            lambda: moe.moe_expert_w13_swiglu_gather(x, meta["perm"], K, meta["offsets"], W13, h=h), R, torch)
        st["alt_gemm2_plain_weights"] = _time_region_graph(
            lambda: moe.moe_expert_w2(h, meta["offsets"], W2, Y_perm=Yp), R, torch)
    nk = n * K
    hit = int((counts > 0).sum())
    flops1 = 2.0 * nk * H * 2 * I
    flops2 = 2.0 * nk * I * H
    # Algorithmic bytes per call (each input read once, each output written once;
    # weights of the experts that received rows).
    bytes_ = {
        "route": n * H * esz + H * E * esz + n * E * 4 + nk * 8,
        "permute": nk * 4 + nk * 8 + (2 * E + 2) * 4,
        "gemm1_swiglu": nk * H * esz + hit * H * 2 * I * esz + nk * I * esz + nk * 4,
        "gemm2": nk * I * esz + hit * I * H * esz + nk * H * esz,
        "combine": nk * H * esz + nk * 8 + n * H * esz,
        # ids read once, rows gathered once, weights of the hit experts once, h and the metadata written once
        "gemm1_swiglu_from_ids": nk * 4 + nk * H * esz + hit * H * 2 * I * esz + nk * I * esz + nk * 8 + (2 * E + 2) * 4,
    }
    bytes_["alt_gemm1_swiglu_plain_weights"] = bytes_["gemm1_swiglu"]
    bytes_["alt_gemm2_plain_weights"] = bytes_["gemm2"]
    g1 = "gemm1_swiglu_from_ids" if meta_ids is not None else "gemm1_swiglu"
    stages = {}
    for k, v in st.items():
        s_ = {"ms": round(v, 5), "GB/s": round(bytes_[k] / (v * 1e-3) / 1e9, 1)}
        s_["frac_hbm"] = round(s_["GB/s"] / PEAK_HBM_GBPS, 4)
        if k in ("gemm1_swiglu", "gemm1_swiglu_from_ids", "alt_gemm1_swiglu_plain_weights"):
            s_["TFLOP/s"] = round(flops1 / (v * 1e-3) / 1e12, 1)
        if k in ("gemm2", "alt_gemm2_plain_weights"):
            s_["TFLOP/s"] = round(flops2 / (v * 1e-3) / 1e12, 1)
        stages[k] = s_
    gg_ms = st[g1] + st["gemm2"]
    gg = (flops1 + flops2) / (gg_ms * 1e-3) / 1e12
    over = ", over the packed weights" if packed else ""
    g1_kernel = (f"gemm_bf16_kernel<GATED=true, GATHER=true, IDS=true{', BPK=true' if packed else ''}> (decode GEMM1 "
                 f"that places the routing ids itself, with fused row gather + SwiGLU epilogue{over})"
                 if meta_ids is not None else
                 f"gemm_bf16_kernel<GATED=true, GATHER=true{', BPK=true' if packed else ''}> (GEMM1 with fused row "
                 f"gather + SwiGLU epilogue{over})")
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if flops1 / bytes_[g1] >= ridge:
        a = round(flops1 / (g1_live_ms * 1e-3) / 1e12, 1)
        roof = {"kernel": g1_kernel, "bound": "mfma", "achieved": a, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(a / PEAK_BF16_TFLOPS, 4)}
    else:
        a = round(bytes_[g1] / (g1_live_ms * 1e-3) / 1e9, 1)
        roof = {"kernel": g1_kernel, "bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(a / PEAK_HBM_GBPS, 4)}
    roof["traffic"] = None
    roof["kernel_ms"] = round(g1_live_ms, 5)
    roof["timing"] = ("mean of HIP events recorded right before and after the GEMM1 launch inside each timed "
                      + ("moe_forward_packed call" if packed else "moe_forward call (moe_forward_timed)")
                      + ", on the layer's stream"
                      + ("" if fence_free else "; default events (the fence-free flag was refused)"))
    roof["kernel_ms_alone"] = round(st[g1], 5)  # the same launch replayed alone from a HIP graph
    out = {"ms": round(ms, 5), "tokens/s": round(n / (ms * 1e-3), 1), "step_spread": spread,
           "wall_s_timed_region": round(wall, 3),
           "weights": ("packed once into the GEMMs' tile order before timing (moe_pack_w13 / moe_pack_w2); "
                       "the layer is moe_forward_packed" if packed else "plain layout; the layer is moe_forward"),
           "ms_plain_weights": None if ms_plain is None else round(ms_plain, 5),
           "grouped_gemm": {"TFLOP/s": round(gg, 1), "frac_bf16_peak": round(gg / PEAK_BF16_TFLOPS, 4),
                            "GFLOP": round((flops1 + flops2) / 1e9, 1)},
           "forward_stages": (["route", "gemm1_swiglu_from_ids", "gemm2", "combine"] if meta_ids is not None else
                              ["route", "permute", "gemm1_swiglu", "gemm2", "combine"]),
           "stages": stages, "expert_load": _expert_load(counts), "roofline": roof}
    if w.dtype == "bf16" and nk > 64 * E:
        out["persistent_experiment"] = _persistent_bench(w, args, torch, moe, dev, (x, Wg, W13, W2, bias), ms,
                                                         ms_plain, (W13p, W2p) if packed else None)
    if not detail:
        return out
    # The alternative second half (routing weights and un-permutation in GEMM2's
    # epilogue, then a contiguous sum of each token's K rows), cold-cache times of
    # the memory-bound stages, and the standalone row gather of moe_permute.
    Yt = moe.moe_expert_w2_scatter(h, meta["offsets"], meta["perm"], wts, W2)
    ys = moe.moe_sum_slots(Yt, n, K)
    alt = {
        "alt_gemm2_scatter": (_time_region_graph(
            lambda: moe.moe_expert_w2_scatter(h, meta["offsets"], meta["perm"], wts, W2, Y_tok=Yt), R, torch),
            nk * I * esz + hit * I * H * esz + nk * H * esz + nk * 8, flops2),
        "alt_slot_sum": (_time_region_graph(lambda: moe.moe_sum_slots(Yt, n, K, y=ys), R, torch),
                         nk * H * esz + n * H * esz, None),
    }
    for k, (v, b, f) in alt.items():
        stages[k] = {"ms": round(v, 5), "GB/s": round(b / (v * 1e-3) / 1e9, 1),
                     "frac_hbm": round(b / (v * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        if f:
            stages[k]["TFLOP/s"] = round(f / (v * 1e-3) / 1e12, 1)
    # Cold-cache times: a 512 MB buffer is read before every call so that the
    # stage's inputs are in neither L2 nor the 256 MB MALL.
    junk = torch.zeros((512 << 20) // 4, dtype=torch.float32, device=dev)
    flush = lambda: junk.sum()  # noqa: E731
    cold = {
        "route": _time_each(lambda: moe.moe_route(x, Wg, bias, K, w.renorm, logits=logits, topk_ids=ids, topk_w=wts),
                            R, torch, flush),
        "permute": _time_each(lambda: moe.moe_permute(ids, None, E, out=meta), R, torch, flush),
        "combine": _time_each(lambda: moe.moe_unpermute_combine(Yp, meta["inv"], wts, n, K, y=yc), R, torch, flush),
    }
    del junk
    for k, v in cold.items():
        c = _pcts(v)
        c["GB/s_at_p50"] = round(bytes_[k] / (c["p50_ms"] * 1e-3) / 1e9, 1)
        stages[k]["cold"] = c
    meta_x = moe.moe_permute(ids, x, E)
    gather_ms = _time_region_graph(lambda: moe.moe_permute(ids, x, E, out=meta_x), R, torch) - st["permute"]
    stages["row_gather_standalone"] = {"ms": round(gather_ms, 5),
                                       "GB/s": round((n * H * esz + nk * H * esz) / (gather_ms * 1e-3) / 1e9, 1)}
    return out


def _persistent_bench(w, args, torch, moe, dev, tensors, forward_ms, plain_ms=None, packed=None):
    """The persistent single kernel (GEMM1 + SwiGLU and GEMM2 with per-XCD task queues, a warm-up of L1
    row tiles and an optional ring pool for h) timed like the layer, for two schedules: a deep warm-up
    without a ring, and a ring of 16 row-tile slots per queue; over the packed weights when given
    (moe_forward_persistent_packed), else the plain ones. Compared with the timed layer and with
    moe_forward on the plain weights."""
    x, Wg, W13, W2, bias = tensors
    y = torch.empty((w.n, w.H), dtype=x.dtype, device=dev)
    res = {"forward_ms": round(forward_ms, 5), "weights": "packed" if packed is not None else "plain"}
    if plain_ms is not None:
        res["forward_plain_weights_ms"] = round(plain_ms, 5)
    for warm, pool in ((16, 0), (8, 16)):
        nbytes = moe.moe_forward_persistent_workspace_size(w.n, w.H, w.I, w.E, w.K, pool)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

        def step():
            if packed is not None:
                moe.moe_forward_persistent_packed(x, Wg, packed[0], packed[1], w.K, w.renorm, bias=bias,
                                                  warmup_row_tiles=warm, pool_row_tiles=pool, y=y, ws=ws)
            else:
                moe.moe_forward_persistent(x, Wg, W13, W2, w.K, w.renorm, bias=bias, warmup_row_tiles=warm,
                                           pool_row_tiles=pool, y=y, ws=ws)

        _warm(step, args.warmup, torch, args.settle_ms)
        pm = _time_region(step, args.steps, torch)
        flag = int(ws[nbytes - 4:].view(torch.int32).item())
        key = f"warm{warm}_pool{pool}"
        res[key] = {"ms": round(pm, 5), "speedup_over_forward": round(forward_ms / pm, 3), "flag": flag,
                    "h_bytes": (w.n * w.K * w.I * 2) if pool == 0 else 8 * pool * 256 * w.I * 2}
        if plain_ms is not None:
            res[key]["speedup_over_plain_forward"] = round(plain_ms / pm, 3)
    return res


def _peaks(moe):
    """The published MI355X peaks the roofline uses, beside the figures derived
    from the device's own properties (compute units x 4096 bf16 FLOP per clock
    per CU x peak shader clock)."""
    try:
        d = moe.device_info()
    except Exception as e:  # noqa: BLE001
        return {"error": str(e)}
    cu, sclk = d["compute_units"], d["sclk_khz"] * 1e3
    return {"used": {"bf16_dense_TFLOP/s": PEAK_BF16_TFLOPS, "hbm_GB/s": PEAK_HBM_GBPS, "source": "published"},
            "device": {"compute_units": cu, "peak_sclk_MHz": round(sclk / 1e6, 1),
                       "bf16_dense_TFLOP/s": round(cu * 4096 * sclk / 1e12, 1),
                       "mem_clk_MHz": round(d["mem_clk_khz"] / 1e3, 1), "mem_bus_bits": d["mem_bus_bits"]}}


def main():
    args = _parse()
    if args.summarize_counters:
        _summarize_counters(args.summarize_counters)
        return
    if args.copy_calibration:
        _copy_calibration()
        return
    if args.gpus != 1:
        print(
            f"bench.py measures one GPU only: the layer runs on a single MI355X and the library has no "
            f"multi-GPU path (asked for --gpus {args.gpus}).",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    import routing_token_permute_amd as moe
    from workloads import make_config

    if args.profile_forward:
        _profile_forward(args, torch, moe)
        return
    if args.workload == "ep_share_bf16":
        _bench_ep_share(args)
        return
    if args.workload == "olmoe_train_bf16":
        _bench_train(args)
        return
    if args.workload in ("decode_fp8", "olmoe_fp8", "decode_fp8a", "olmoe_fp8a"):
        print(json.dumps(_bench_fp8(args)), flush=True)
        return
    dev = torch.device("cuda:0")
    w = make_config(args.workload)
    head = _layer_bench(w, args, torch, moe, dev, detail=True)
    roof = dict(head["roofline"])
    if args.workload == "olmoe_bf16":
        roof["traffic"] = _traffic_bytes()

    # The other configurations of the same layer, each with its own roofline.
    configs = {}
    if args.workload == "olmoe_bf16" and not args.headline_only:
        for name in ("tiny_f32", "olmoe_skewed_bf16", "decode_bf16"):
            wc = make_config(name)
            r = _layer_bench(wc, args, torch, moe, dev, detail=False)
            if name == "tiny_f32":  # parity configuration: launch-bound, no roofline
                r = {k: r[k] for k in ("ms", "tokens/s", "step_spread", "expert_load")}
                r["note"] = "parity configuration (n=64, H=128): launch-bound, time reported, no roofline"
            if name == "decode_bf16":
                hit = r["expert_load"]["experts_hit"]
                wbytes = hit * 3 * wc.H * wc.I * 2  # W13 (H x 2I) and W2 (I x H) of the hit experts
                r["weight_stream"] = {"bytes": wbytes, "GB/s_over_forward": round(wbytes / (r["ms"] * 1e-3) / 1e9, 1),
                                      "frac_hbm_over_forward": round(wbytes / (r["ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
            if not args.no_cpu_baseline:  # a short oracle sample of the same configuration, all threads and one
                r["cpu_baseline"] = _cpu_baseline(wc, min_seconds=2.0, one_core_seconds=2.0)
            configs[name] = r
        configs["ep_share_bf16"] = _ep_share_core(args, torch, dev, cu_split=False, cpu=False)[0]
        # The FP8 layers ([Fusion] §8.4): FP8 activations with per-row scales and FP8 weights, on the FP8 MFMA.
        for name in ("olmoe_fp8a", "decode_fp8a"):
            r = _bench_fp8(args, workload=name, cpu_leg=False)
            configs[name] = {k: r[k] for k in ("ms_per_step", "value", "unit", "step_spread", "ms_per_step_bf16_weights",
                                               "speedup_over_bf16_weights", "dtype", "stages", "roofline")}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline(w, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": head["tokens/s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": head["ms"],
        "step_spread": head["step_spread"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights, OLMoE layer shapes; no checkpoint)",
        "config": {"workload": args.workload, "n": w.n, "H": w.H, "I": w.I, "E": w.E, "K": w.K,
                   "renorm": bool(w.renorm), "skewed_bias": w.bias is not None},
        "weights": head["weights"],
        "ms_per_step_plain_weights": head["ms_plain_weights"],
        "grouped_gemm": head["grouped_gemm"],
        "stages": head["stages"],
        "roofline": roof,
        "expert_load": head["expert_load"],
        "wall_s_timed_region": head["wall_s_timed_region"],
        "persistent_experiment": head.get("persistent_experiment"),
        "configs": configs,
        "peaks": _peaks(moe),
        "cpu_baseline": cpu,
        "device": _device_name(torch, dev),
    }
    print(json.dumps(out), flush=True)


def _profile_forward(args, torch, moe):
    """A few moe_forward calls of the workload and nothing else, for rocprofv3
    counter passes (no timing, no CPU work beyond the input upload)."""
    from workloads import make_config

    dev = torch.device("cuda:0")
    w = make_config(args.workload)
    x, Wg, W13, W2 = (_to_dev_bits(w, k, dev, torch) for k in ("x", "W_gate", "W13", "W2"))
    bias = None if w.bias is None else torch.from_numpy(w.bias).to(dev)
    if args.profile_layer == "fp8a":  # FP8 activations and weights (the weights quantized once, first)
        q13, s13 = moe.moe_quantize_fp8(W13)
        q2, s2 = moe.moe_quantize_fp8(W2)
        step = lambda: moe.moe_forward_fp8a(x, Wg, q13, s13, q2, s2, w.K, w.renorm, bias=bias)  # noqa: E731
    elif args.profile_layer == "persistent":
        step = lambda: moe.moe_forward_persistent(x, Wg, W13, W2, w.K, w.renorm, bias=bias)  # noqa: E731
    elif args.profile_layer == "persistent_packed":
        W13p, W2p = moe.moe_pack_w13(W13), moe.moe_pack_w2(W2)
        step = lambda: moe.moe_forward_persistent_packed(x, Wg, W13p, W2p, w.K, w.renorm, bias=bias)  # noqa: E731
    elif args.profile_layer == "packed":
        W13p, W2p = moe.moe_pack_w13(W13), moe.moe_pack_w2(W2)
        step = lambda: moe.moe_forward_packed(x, Wg, W13p, W2p, w.K, w.renorm, bias=bias)  # noqa: E731
    else:
        step = lambda: moe.moe_forward(x, Wg, W13, W2, w.K, w.renorm, bias=bias)  # noqa: E731
    for _ in range(args.profile_forward):
        step()
    torch.cuda.synchronize()
    print(json.dumps({"profiled": args.workload, "layer": args.profile_layer, "forwards": args.profile_forward}),
          flush=True)


def _ep_share_core(args, torch, dev, cu_split=True, cpu=True):
    """One GPU's expert-parallel share, two micro-batches of 16384 received rows,
    8 local experts: the four controls of a two-stream overlap measurement.

    T_A: both micro-batches' expert GEMMs alone (one stream); T_B: their
    permute + unpermute alone (one stream); T_C: everything serial on one
    stream; T_D: the two-stream schedule permute(A); [GEMM(A) || permute(B)];
    [GEMM(B) || unpermute(A)]; unpermute(B). Hidden fraction of the
    permute/unpermute time: 1 - (T_D - T_A) / T_B. T_F: the fused one-stream
    schedule. Returns a dict (and the CPU oracle baseline when `cpu`).
    """
    import oracle
    import routing_token_permute_amd as moe
    from routing_token_permute_amd import ep_share as eps
    from workloads import make_config

    ep = make_config("ep_share_bf16")
    tb = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    W13, W2 = tb(ep.bits("W13")), tb(ep.bits("W2"))
    mbs = [eps.prepare(eps.MicroBatch(tb(m.x_bits()), torch.from_numpy(m.eid.reshape(-1, 1)).to(dev)), ep.E_local, ep.I)
           for m in ep.micro_batches]
    a, b = mbs
    s0 = torch.cuda.current_stream(dev)
    compute, comm = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    eps.run_serial(a, b, W13, W2, ep.E_local, s0)  # fills every buffer the controls read
    torch.cuda.synchronize()

    def timed(fn, streams):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        _warm(fn, args.warmup, torch, args.settle_ms)
        first = streams[0]
        start.record(first)
        for st in streams[1:]:
            st.wait_event(start)
        for _ in range(args.steps):
            fn()
        for st in streams[1:]:
            e = torch.cuda.Event()
            e.record(st)
            first.wait_event(e)
        end.record(first)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    t_a = timed(lambda: (eps.experts(a, W13, W2, s0), eps.experts(b, W13, W2, s0)), [s0])
    t_b = timed(lambda: (eps.permute(a, ep.E_local, s0), eps.permute(b, ep.E_local, s0), eps.unpermute(a, s0),
                         eps.unpermute(b, s0)), [s0])
    t_c = timed(lambda: eps.run_serial(a, b, W13, W2, ep.E_local, s0), [s0])
    t_d = timed(lambda: eps.run_two_streams(a, b, W13, W2, ep.E_local, compute, comm), [compute, comm])
    # The same work with the permute and unpermute folded into the GEMMs (one stream).
    t_f = timed(lambda: eps.run_fused(a, b, W13, W2, ep.E_local, s0), [s0])
    packed = (moe.moe_pack_w13(W13), moe.moe_pack_w2(W2))  # once, outside the timed work
    t_fp = timed(lambda: eps.run_fused(a, b, W13, W2, ep.E_local, s0, packed=packed), [s0])
    # The dominant kernel: micro-batch A's GEMM1 + SwiGLU alone (graph replays).
    g1 = _time_region_graph(lambda: moe.moe_expert_w13_swiglu(a.meta["x_perm"], a.meta["offsets"], W13, h=a.h),
                            args.stage_reps, torch)
    g1_tf = 2.0 * ep.R * ep.H * 2 * ep.I / (g1 * 1e-3) / 1e12
    # CU-masked split ([Fusion] §6.4's T_total(S_comm) = max(T_compute(S - S_comm), T_comm(S_comm)) + T_sync):
    # the permute/unpermute stream gets S_comm compute units, the GEMM stream the rest.
    split = []
    for n_comm in (args.comm_cus if cu_split else []):
        ms = eps.MaskedStreams(n_comm, dev)
        try:
            tc = ms.compute
            t_comp = timed(lambda: (eps.experts(a, W13, W2, tc), eps.experts(b, W13, W2, tc)), [tc])
            cm = ms.comm
            t_comm = timed(lambda: (eps.permute(a, ep.E_local, cm), eps.permute(b, ep.E_local, cm),
                                    eps.unpermute(a, cm), eps.unpermute(b, cm)), [cm])
            t_tot = timed(lambda: eps.run_two_streams(a, b, W13, W2, ep.E_local, tc, cm), [tc, cm])
        finally:
            torch.cuda.synchronize()
            ms.close()
        split.append({"S_comm_cus": n_comm, "T_compute_ms": round(t_comp, 4), "T_comm_ms": round(t_comm, 4),
                      "T_total_ms": round(t_tot, 4), "T_sync_ms": round(t_tot - max(t_comp, t_comm), 4)})
    rows = 2 * ep.R
    flops = 2 * ep.flops_per_micro_batch
    out = {
        "rows/s_two_streams": round(rows / (t_d * 1e-3), 1),
        "rows/s_fused": round(rows / (t_f * 1e-3), 1),
        "rows/s_fused_packed": round(rows / (t_fp * 1e-3), 1),
        "overlap": {"T_A_gemm_ms": round(t_a, 4), "T_B_permute_unpermute_ms": round(t_b, 4),
                    "T_C_serial_ms": round(t_c, 4), "T_D_two_streams_ms": round(t_d, 4),
                    "hidden_fraction": round(1 - (t_d - t_a) / t_b, 4), "speedup_serial_over_overlap": round(t_c / t_d, 4),
                    "gemm_TFLOP/s_alone": round(flops / (t_a * 1e-3) / 1e12, 1),
                    "gemm_TFLOP/s_in_overlap": round(flops / (t_d * 1e-3) / 1e12, 1)},
        "fused_schedule": {"T_F_ms": round(t_f, 4), "speedup_over_two_streams": round(t_d / t_f, 4),
                           "T_F_packed_weights_ms": round(t_fp, 4),
                           "what": "metadata-only permute, GEMM1 reading rows through perm, GEMM2 storing rows at "
                                   "their arrival positions (unit weights); one stream"},
        "expert_load": [_expert_load(m.counts) for m in ep.micro_batches],
        "roofline": {"kernel": "gemm_bf16_kernel<GATED=true, GATHER=false> (micro-batch A GEMM1 + SwiGLU)",
                     "bound": "mfma", "achieved": round(g1_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g1_tf / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "config": {"rows_per_micro_batch": ep.R, "micro_batches": 2, "E_local": ep.E_local, "H": ep.H, "I": ep.I},
    }
    if split:
        out["overlap"]["cu_split"] = split
    if cpu:
        reps, t0 = 0, time.perf_counter()
        while True:
            for m in ep.micro_batches:
                oracle.ep_share_forward(m.x_f32, m.eid, ep.W13_f32, ep.W2_f32)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(rows * reps / el, 1), "unit": "rows/s", "cores": _blas_threads(),
                               "kind": "oracle", "sample": f"both micro-batches, {reps} repetitions, {el:.1f} s"}
    return out, ep


def _bench_ep_share(args):
    """The EP share as its own bench line (rows/s of the two-stream schedule),
    with the CU-masked split sweep."""
    import torch

    dev = torch.device("cuda:0")
    core, ep = _ep_share_core(args, torch, dev, cu_split=True, cpu=not args.no_cpu_baseline)
    t_d = core["overlap"]["T_D_two_streams_ms"]
    out = {
        "metric": "EP-share two-micro-batch expert layer rows/s (permute + SwiGLU grouped GEMM + unpermute)",
        "value": core["rows/s_two_streams"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": t_d,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (Dirichlet(0.5) expert shares, 8 source ranks, N(0,1) rows, N(0,0.02) weights)",
        "config": dict(workload="ep_share_bf16", **core["config"],
                       counts=[m.counts.tolist() for m in ep.micro_batches]),
        "overlap": core["overlap"],
        "fused_schedule": dict(core["fused_schedule"], **{"rows/s": core["rows/s_fused"]}),
        "roofline": core["roofline"],
        "cpu_baseline": core.get("cpu_baseline"),
        "device": _device_name(torch, dev),
    }
    print(json.dumps(out), flush=True)


def _bench_train(args):
    """Training step of the OLMoE n=4096 layer: moe_forward_train then
    moe_backward for a seeded upstream gradient. Reports fwd+bwd tokens/s, the
    two halves, and each backward stage alone with its FLOP rate or bandwidth."""
    import torch

    import routing_token_permute_amd as moe
    from workloads import make_config, random_bf16_matrix

    dev = torch.device("cuda:0")
    w = make_config("olmoe_bf16")
    n, H, I, E, K = w.n, w.H, w.I, w.E, w.K  # noqa: E741

    def to_dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)

    x, Wg, W13, W2 = (to_dev(w.bits(k)) for k in ("x", "W_gate", "W13", "W2"))
    dy = to_dev(random_bf16_matrix(np.random.default_rng(w.n), (n, H))[0])
    y, saved = moe.moe_forward_train(x, Wg, W13, W2, K, w.renorm)
    grads = moe.moe_backward(dy, x, Wg, W13, W2, K, w.renorm, saved)
    fws = torch.empty(moe.load_library().moe_forward_train_workspace_size(n, E, K), dtype=torch.uint8, device=dev)
    bws = torch.empty(moe.moe_backward_workspace_size(n, H, I, E, K, torch.bfloat16), dtype=torch.uint8, device=dev)

    def fwd():
        moe.moe_forward_train(x, Wg, W13, W2, K, w.renorm, saved=saved, y=y, ws=fws)

    def bwd():
        moe.moe_backward(dy, x, Wg, W13, W2, K, w.renorm, saved, grads=grads, ws=bws)

    def step():
        fwd()
        bwd()

    _warm(step, args.warmup, torch, args.settle_ms)
    t0 = time.perf_counter()
    ms_step = _time_region(step, args.steps, torch)
    wall = time.perf_counter() - t0
    R = args.stage_reps
    ms_fwd = _time_region(fwd, R, torch)
    ms_bwd = _time_region(bwd, R, torch)

    # Backward stages alone, on the saved tensors.
    off, perm, inv = saved["offsets"], saved["perm"], saved["inv"]
    dY, dw = moe.moe_combine_backward(dy, saved["Y_perm"], inv, saved["topk_w"], n, K)
    dgu = moe.moe_expert_w2_backward(dY, off, W2, saved["gate_up"])
    dX = moe.moe_expert_w13_backward(dgu, off, W13)
    rb = moe.moe_route_backward(x, Wg, saved["logits"], saved["topk_ids"], saved["topk_w"], dw, w.renorm)
    dx = moe.moe_dispatch_backward(dX, inv, n, K, add=rb["dx_router"])
    xmeta = moe.moe_permute(saved["topk_ids"], x, E)
    x_perm = xmeta["x_perm"]
    dW2 = moe.moe_expert_weight_grad(saved["h"], dY, off)
    dW13 = moe.moe_expert_weight_grad(x_perm, dgu, off)
    meta = moe.moe_permute(saved["topk_ids"], None, E)
    torch.cuda.synchronize()
    hit = int((meta["counts"].cpu().numpy() > 0).sum())
    st = {
        "combine_bwd": _time_region(lambda: moe.moe_combine_backward(dy, saved["Y_perm"], inv, saved["topk_w"], n, K,
                                                                     dY_perm=dY, dw=dw), R, torch),
        "route_bwd": _time_region(lambda: moe.moe_route_backward(x, Wg, saved["logits"], saved["topk_ids"],
                                                                 saved["topk_w"], dw, w.renorm), R, torch),
        "gemm2_dgrad_swiglu": _time_region(lambda: moe.moe_expert_w2_backward(dY, off, W2, saved["gate_up"],
                                                                              dgate_up=dgu), R, torch),
        "gemm2_wgrad": _time_region(lambda: moe.moe_expert_weight_grad(saved["h"], dY, off, dW=dW2), R, torch),
        "gemm1_dgrad": _time_region(lambda: moe.moe_expert_w13_backward(dgu, off, W13, dX_perm=dX), R, torch),
        "dispatch_bwd": _time_region(lambda: moe.moe_dispatch_backward(dX, inv, n, K, add=rb["dx_router"], dx=dx),
                                     R, torch),
        "gemm1_wgrad": _time_region(lambda: moe.moe_expert_weight_grad(x_perm, dgu, off, dW=dW13), R, torch),
        "gemm1_wgrad_gather": _time_region(lambda: moe.moe_expert_weight_grad_gather(x, perm, K, dgu, off, dW=dW13),
                                           R, torch),
        "x_gather": _time_region(lambda: moe.moe_permute(saved["topk_ids"], x, E, out=xmeta), R, torch)
        - _time_region(lambda: moe.moe_permute(saved["topk_ids"], None, E, out=meta), R, torch),
    }
    nk = n * K
    f_small, f_big = 2.0 * nk * H * I, 2.0 * nk * H * 2 * I
    flops = {"gemm2_dgrad_swiglu": f_small, "gemm2_wgrad": f_small, "gemm1_dgrad": f_big, "gemm1_wgrad": f_big,
             "gemm1_wgrad_gather": f_big}
    bytes_ = {
        "combine_bwd": n * H * 2 + 2 * nk * H * 2 + nk * 12,
        "route_bwd": n * E * 4 + nk * 12 + n * H * 2 + H * E * 2 + n * E * 4 + n * H * 4 + H * E * 4,
        "dispatch_bwd": nk * H * 2 + nk * 4 + n * H * 4 + n * H * 2,
        "x_gather": n * H * 2 + nk * H * 2 + nk * 4,
    }
    stages = {}
    for k, ms in st.items():
        s_ = {"ms": round(ms, 5)}
        if k in flops:
            s_["TFLOP/s"] = round(flops[k] / (ms * 1e-3) / 1e12, 1)
            s_["frac_bf16_peak"] = round(flops[k] / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        else:
            s_["GB/s"] = round(bytes_[k] / (ms * 1e-3) / 1e9, 1)
            s_["frac_hbm"] = round(bytes_[k] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)
        stages[k] = s_
    # the backward uses the explicit gather + dW13, not the gathered alternative
    bwd_gemm_ms = sum(st[k] for k in flops if k != "gemm1_wgrad_gather")
    bwd_flops = sum(v for k, v in flops.items() if k != "gemm1_wgrad_gather")
    bwd_gemm_tf = bwd_flops / (bwd_gemm_ms * 1e-3) / 1e12
    dom = max((k for k in flops if k != "gemm1_wgrad_gather"), key=lambda k: st[k])
    dom_tf = flops[dom] / (st[dom] * 1e-3) / 1e12
    cpu = None if args.no_cpu_baseline else _cpu_baseline_train(w, dy_seed=w.n, min_seconds=args.cpu_seconds)
    out = {
        "metric": "MoE layer fwd+bwd tokens/s (training step of one layer), OLMoE n=4096",
        "value": round(n / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 5),
        "ms_forward_train": round(ms_fwd, 5),
        "ms_backward": round(ms_bwd, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens and upstream gradient, N(0,0.02) weights, OLMoE layer shapes)",
        "config": {"workload": "olmoe_train_bf16", "n": n, "H": H, "I": I, "E": E, "K": K, "renorm": bool(w.renorm)},
        "backward_grouped_gemm": {"TFLOP/s": round(bwd_gemm_tf, 1),
                                  "frac_bf16_peak": round(bwd_gemm_tf / PEAK_BF16_TFLOPS, 4),
                                  "GFLOP": round(bwd_flops / 1e9, 1)},
        "stages": stages,
        "roofline": {"kernel": f"gemm_bwd_bf16_kernel ({dom})", "bound": "mfma", "achieved": round(dom_tf, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "experts_hit": hit,
        "wall_s_timed_region": round(wall, 3),
        "cpu_baseline": cpu,
        "device": _device_name(torch, dev),
    }
    print(json.dumps(out), flush=True)


def _bench_fp8(args, workload=None, cpu_leg=True):
    """The layer with FP8 E4M3 expert weights (per-column fp32 scales, quantized
    on the device before timing) on the decode (n=32) or OLMoE (n=4096) batch:
    tokens/s, the FP8 GEMMs' bandwidth against their weight bytes, and the bf16
    layer on the same inputs for comparison. The *_fp8a workloads also carry the
    activations as per-token FP8 (moe_forward_fp8a: FP8 x FP8 GEMMs, the token
    rows read in place; the padded receive buffer timed beside it)."""
    import torch

    import routing_token_permute_amd as moe
    from workloads import make_config

    dev = torch.device("cuda:0")
    wl = workload or args.workload
    base = "decode_bf16" if wl.startswith("decode") else "olmoe_bf16"
    act8 = wl.endswith("fp8a")
    w = make_config(base)
    n, H, I, E, K = w.n, w.H, w.I, w.E, w.K  # noqa: E741

    def to_dev(name):
        return torch.from_numpy(w.bits(name).view(np.int16)).view(torch.bfloat16).to(dev)

    x, Wg, W13, W2 = (to_dev(k) for k in ("x", "W_gate", "W13", "W2"))
    q13, s13 = moe.moe_quantize_fp8(W13)
    q2, s2 = moe.moe_quantize_fp8(W2)
    y = torch.empty((n, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moe.moe_forward_workspace_size(n, H, I, E, K, torch.bfloat16), dtype=torch.uint8, device=dev)

    ws8 = torch.empty(moe.moe_forward_fp8a_workspace_size(n, H, I, E, K), dtype=torch.uint8, device=dev)

    def step():
        if act8:
            moe.moe_forward_fp8a(x, Wg, q13, s13, q2, s2, K, w.renorm, y=y, ws=ws8)
        else:
            moe.moe_forward_fp8(x, Wg, q13, s13, q2, s2, K, w.renorm, y=y, ws=ws)

    W13p, W2p = moe.moe_pack_w13(W13), moe.moe_pack_w2(W2)

    def step_bf16():  # the bf16 layer as the headline runs it (packed weights)
        moe.moe_forward_packed(x, Wg, W13p, W2p, K, w.renorm, y=y, ws=ws)

    _warm(step, args.warmup, torch, args.settle_ms)
    t0 = time.perf_counter()
    ms = _time_region(step, args.steps, torch)
    wall = time.perf_counter() - t0
    spread = _pcts(_time_each(step, max(args.steps, 10), torch))
    _warm(step_bf16, args.warmup, torch, args.settle_ms)
    ms_bf16 = _time_region(step_bf16, args.steps, torch)
    logits, ids, wts = moe.moe_route(x, Wg, None, K, w.renorm)
    meta = moe.moe_permute(ids, None, E)
    h = moe.moe_expert_w13_swiglu_gather_fp8(x, meta["perm"], K, meta["offsets"], q13, s13)
    Yp = moe.moe_expert_w2_fp8(h, meta["offsets"], q2, s2)
    torch.cuda.synchronize()
    hit = int((meta["counts"].cpu().numpy() > 0).sum())
    R = args.stage_reps
    st = {
        "gemm1_swiglu_fp8": _time_region_graph(
            lambda: moe.moe_expert_w13_swiglu_gather_fp8(x, meta["perm"], K, meta["offsets"], q13, s13, h=h), R, torch),
        "gemm2_fp8": _time_region_graph(lambda: moe.moe_expert_w2_fp8(h, meta["offsets"], q2, s2, Y_perm=Yp), R, torch),
    }
    nk = n * K
    if not act8:  # decode-sized batches: the layer runs the FP8-weight GEMM1 straight from the ids
        try:
            h8w, meta8w = moe.moe_expert_w13_swiglu_from_ids_fp8(x, ids, q13, s13)
        except moe.MoEError:
            meta8w = None
        if meta8w is not None:
            st["gemm1_swiglu_fp8_from_ids"] = _time_region_graph(
                lambda: moe.moe_expert_w13_swiglu_from_ids_fp8(x, ids, q13, s13, h=h8w, out=meta8w), R, torch)
    if act8:  # the stages moe_forward_fp8a runs: FP8 rows read in place, FP8 x FP8 GEMMs, h quantized per row
        codes_tok, s_tok = moe.moe_quantize_rows_fp8(x)
        h8 = moe.moe_expert_w13_swiglu_gather_fp8a(codes_tok, s_tok, meta["perm"], K, meta["offsets"], q13, s13)
        hq, hs = moe.moe_quantize_rows_fp8(h8)
        Y8 = moe.moe_expert_w2_fp8a(hq, hs, meta["offsets"], q2, s2)
        d8 = moe.moe_dispatch_fp8(meta, codes_tok, s_tok, K)
        torch.cuda.synchronize()
        rpad = int(d8["offsets_padded"][-1].item())
        st["quantize_rows_fp8"] = _time_region_graph(lambda: moe.moe_quantize_rows_fp8(x, codes=codes_tok, scales=s_tok),
                                                     R, torch)
        st["gemm1_swiglu_fp8a"] = _time_region_graph(
            lambda: moe.moe_expert_w13_swiglu_gather_fp8a(codes_tok, s_tok, meta["perm"], K, meta["offsets"], q13, s13,
                                                          h=h8), R, torch)
        st["quantize_h_fp8"] = _time_region_graph(lambda: moe.moe_quantize_rows_fp8(h8, codes=hq, scales=hs), R, torch)
        st["gemm2_fp8a"] = _time_region_graph(
            lambda: moe.moe_expert_w2_fp8a(hq, hs, meta["offsets"], q2, s2, Y_perm=Y8), R, torch)
        # The padded receive buffer an expert-parallel exchange would deliver (not on the one-GPU layer's path).
        st["alt_dispatch_fp8"] = _time_region_graph(lambda: moe.moe_dispatch_fp8(meta, codes_tok, s_tok, K, out=d8),
                                                    R, torch)
        # Decode-sized batches: the layer runs GEMM1 straight from the ids (no permute launch).
        try:
            h8i, meta8i = moe.moe_expert_w13_swiglu_from_ids_fp8a(codes_tok, s_tok, ids, q13, s13)
        except moe.MoEError:
            meta8i = None
        if meta8i is not None:
            st["gemm1_swiglu_fp8a_from_ids"] = _time_region_graph(
                lambda: moe.moe_expert_w13_swiglu_from_ids_fp8a(codes_tok, s_tok, ids, q13, s13, h=h8i, out=meta8i),
                R, torch)
    bytes_ = {  # algorithmic: activations once, FP8 codes and scales of the hit experts once, outputs once
        "gemm1_swiglu_fp8": nk * H * 2 + hit * (2 * I * H + 2 * I * 4) + nk * I * 2 + nk * 4,
        "gemm2_fp8": nk * I * 2 + hit * (H * I + H * 4) + nk * H * 2,
    }
    flops = {"gemm1_swiglu_fp8": 2.0 * nk * H * 2 * I, "gemm2_fp8": 2.0 * nk * I * H}
    bytes_["gemm1_swiglu_fp8_from_ids"] = bytes_["gemm1_swiglu_fp8"] + nk * 8 + (2 * E + 2) * 4
    flops["gemm1_swiglu_fp8_from_ids"] = flops["gemm1_swiglu_fp8"]
    if act8:
        bytes_["quantize_rows_fp8"] = n * H * 2 + n * H + n * 4
        bytes_["alt_dispatch_fp8"] = nk * H + rpad * H + rpad * 8 + nk * 4
        bytes_["gemm1_swiglu_fp8a"] = n * (H + 4) + nk * 4 + hit * (2 * I * H + 2 * I * 4) + nk * I * 2
        flops["gemm1_swiglu_fp8a"] = 2.0 * nk * H * 2 * I
        bytes_["quantize_h_fp8"] = nk * I * 2 + nk * I + nk * 4
        bytes_["gemm2_fp8a"] = nk * (I + 4) + hit * (H * I + H * 4) + nk * H * 2
        flops["gemm2_fp8a"] = 2.0 * nk * I * H
        bytes_["gemm1_swiglu_fp8a_from_ids"] = bytes_["gemm1_swiglu_fp8a"] + nk * 8 + (2 * E + 2) * 4
        flops["gemm1_swiglu_fp8a_from_ids"] = flops["gemm1_swiglu_fp8a"]
    stages = {}
    for k, v in st.items():
        gbs = bytes_[k] / (v * 1e-3) / 1e9
        stages[k] = {"ms": round(v, 5), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBPS, 4)}
        if k in flops:
            stages[k]["TFLOP/s"] = round(flops[k] / (v * 1e-3) / 1e12, 1)
    dom = "gemm1_swiglu_fp8a" if act8 else "gemm1_swiglu_fp8"
    kname = ("gemm_f8f8_kernel<GATED, GATHER> (GEMM1 + SwiGLU, FP8 token rows read through perm x FP8 weights, "
             "FP8 MFMA 32x32x64)" if act8 else
             "gemm_w8_kernel<GATED=true, GATHER=true> (GEMM1 + SwiGLU, FP8 weights)")
    if "gemm1_swiglu_fp8_from_ids" in st:
        dom = "gemm1_swiglu_fp8_from_ids"
        kname = ("gemm_w8_kernel<GATED, GATHER, IDS> (decode GEMM1 + SwiGLU that places the routing ids itself, "
                 "FP8 weights)")
    if "gemm1_swiglu_fp8a_from_ids" in st:
        dom = "gemm1_swiglu_fp8a_from_ids"
        kname = ("gemm_f8f8_kernel<GATED, GATHER, IDS> (decode GEMM1 + SwiGLU that places the routing ids itself, "
                 "FP8 token rows x FP8 weights, FP8 MFMA 32x32x64)")
    if base == "decode_bf16":
        roof = {"kernel": kname, "bound": "hbm", "achieved": stages[dom]["GB/s"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": stages[dom]["frac_hbm"], "traffic": None}
    else:
        tf = stages[dom]["TFLOP/s"]
        peak = PEAK_FP8_TFLOPS if act8 else PEAK_BF16_TFLOPS  # FP8 x FP8 products run on the FP8 MFMA
        roof = {"kernel": kname, "bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                "frac": round(tf / peak, 4), "traffic": None}
    cpu = None
    if cpu_leg and not args.no_cpu_baseline:
        import oracle

        c13, r13 = oracle.fp8.quantize_columns(w.W13_f32)
        c2, r2 = oracle.fp8.quantize_columns(w.W2_f32)
        m = min(n, 512)
        reps, t1 = 0, time.perf_counter()
        while True:
            oracle.fp8.forward_fp8(w.x_f32[:m], w.W_gate_f32, c13, r13, c2, r2, K, w.renorm)
            reps += 1
            if time.perf_counter() - t1 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t1
        cpu = {"value": round(m * reps / el, 1), "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
               "sample": f"fp64 layer on the dequantized FP8 weights, first {m} tokens, {reps} repetitions, {el:.1f} s "
                         f"(weight quantization not timed)"}
    out = {
        "metric": (f"MoE layer fwd tokens/s with FP8 E4M3 expert weights"
                   f"{' and per-token FP8 activations' if act8 else ''}, {base.split('_')[0]} n={n}"),
        "value": round(n / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms, 5),
        "step_spread": spread,
        "ms_per_step_bf16_weights": round(ms_bf16, 5),
        "speedup_over_bf16_weights": round(ms_bf16 / ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 e4m3 activations (per-token scales) and weights" if act8 else "bf16 activations, fp8 e4m3 weights",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights quantized per output column; OLMoE layer shapes)",
        "config": {"workload": wl, "n": n, "H": H, "I": I, "E": E, "K": K, "renorm": bool(w.renorm)},
        "stages": stages,
        "roofline": roof,
        "experts_hit": hit,
        "wall_s_timed_region": round(wall, 3),
        "cpu_baseline": cpu,
        "device": _device_name(torch, dev),
    }
    return out


def _cpu_baseline_train(w, dy_seed, min_seconds, sample_tokens=512):
    """The fp64 oracle's gradient on the host, on the first `sample_tokens` tokens of the layer."""
    import oracle
    from workloads import random_bf16_matrix

    m = min(sample_tokens, w.n)
    dy = random_bf16_matrix(np.random.default_rng(dy_seed), (w.n, w.H))[1][:m]
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.backward(w.x_f32[:m], w.W_gate_f32, w.W13_f32, w.W2_f32, w.K, w.renorm, dy, bias=w.bias)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    return {
        "value": round(m * reps / el, 1),
        "unit": "tokens/s",
        "cores": _blas_threads(),
        "kind": "oracle",
        "sample": f"fp64 forward + gradient of the first {m} tokens of the layer, {reps} repetitions, {el:.1f} s",
    }


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info

        return int(max([d.get("num_threads", 1) for d in threadpool_info()] or [1]))
    except Exception:  # noqa: BLE001
        return len(os.sched_getaffinity(0))


def _device_name(torch, dev):
    """The device's name with its architecture (hosts without the marketing
    name table report a generic or empty name)."""
    name = torch.cuda.get_device_name(dev) or ""
    arch = getattr(torch.cuda.get_device_properties(dev), "gcnArchName", "") or ""
    return f"{name} ({arch})" if name and arch else (name or arch)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _cpu_baseline(w, min_seconds, one_core_seconds=5.0, one_core_tokens=256):
    """The fp64 oracle (as it stands) on the host: full-layer forwards until
    min_seconds pass, with the BLAS threads it uses; then a one-thread run on the
    first `one_core_tokens` tokens. Also the oracle's rate in GFLOP/s (the
    grouped GEMM's 6*K*H*I and the router's 2*H*E per token)."""
    import oracle

    threads = _blas_threads()
    flop_per_token = 6.0 * w.K * w.H * w.I + 2.0 * w.H * w.E

    def run(x, secs):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.forward(x, w.W_gate_f32, w.W13_f32, w.W2_f32, w.K, w.renorm, bias=w.bias)
            reps += 1
            if time.perf_counter() - t0 >= secs:
                return reps, time.perf_counter() - t0

    reps, el = run(w.x_f32, min_seconds)
    tps = w.n * reps / el
    out = {
        "value": round(tps, 1),
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"the full {w.n}-token layer forward (fp64 numpy, OpenBLAS), {reps} repetitions, {el:.1f} s",
        "GFLOP/s": round(tps * flop_per_token / 1e9, 2),
        "cpu": _cpu_model(),
        "visible_cores": len(os.sched_getaffinity(0)),
    }
    try:
        from threadpoolctl import threadpool_limits

        m = min(one_core_tokens, w.n)
        with threadpool_limits(limits=1):
            r1, e1 = run(w.x_f32[:m], one_core_seconds)
        t1 = m * r1 / e1
        out["one_core"] = {"value": round(t1, 1), "unit": "tokens/s", "GFLOP/s": round(t1 * flop_per_token / 1e9, 2),
                           "sample": f"first {m} tokens, 1 BLAS thread, {r1} repetitions, {e1:.1f} s"}
    except Exception as e:  # noqa: BLE001
        out["one_core"] = {"error": str(e)}
    return out


if __name__ == "__main__":
    main()
