"""Helpers shared by the GPU tests: moving generator arrays to the device and
measuring errors against the oracle. No layer arithmetic lives here."""

from __future__ import annotations

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import routing_token_permute_amd as m

    m.load_library()  # raises when the HIP library is not built: no fallback
    return torch.device("cuda:0")


def dev_tensor(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Generator storage -> device tensor. bf16: uint16 bit patterns; f32: float32."""
    if dtype == "bf16":
        assert arr.dtype == np.uint16
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def layer_tensors(w, device):
    """x, W_gate, W13, W2 (storage dtype) and bias (fp32 or None) of a LayerWorkload on the device."""
    t = {k: dev_tensor(w.bits(k), w.dtype, device) for k in ("x", "W_gate", "W13", "W2")}
    t["bias"] = None if w.bias is None else torch.from_numpy(w.bias).to(device)
    return t


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    """(max-abs error, relative Frobenius error)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    nr = np.linalg.norm(ref)
    return float(np.abs(d).max()) if d.size else 0.0, float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d))


# Layer-output bounds: max-abs and relative Frobenius, per storage dtype.
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-5, 1e-5)}


def assert_close(got, ref, dtype: str, what: str, intermediate: bool = False):
    """The layer's bounds (max-abs and relative Frobenius), plus the largest error
    relative to the largest reference value under the same relative bound, which
    stays meaningful when outputs are much smaller than one.

    `intermediate`: the SwiGLU activation h, whose values reach ~10 at the
    OLMoE scale; stored in bf16 its rounding alone can exceed the layer's
    absolute bound, which is stated for the layer output y. Such arrays are
    held to the two relative bounds only."""
    ma, rf = errors(got, ref)
    tol_ma, tol_rf = TOL[dtype]
    if intermediate:
        tol_ma = float("inf")
    scale = float(np.abs(ref).max()) if np.size(ref) else 0.0
    rmax = ma / scale if scale > 0 else ma
    print(f"[{what}] max_abs={ma:.3e} rel_frob={rf:.3e} max_rel_to_peak={rmax:.3e} "
          f"(bounds {tol_ma:g}, {tol_rf:g}, {tol_rf:g}; |ref|max={scale:.3g})", flush=True)
    assert ma <= tol_ma and rf <= tol_rf and rmax <= tol_rf, (
        f"{what}: max_abs={ma:.3e} rel_frob={rf:.3e} max_rel_to_peak={rmax:.3e}")
