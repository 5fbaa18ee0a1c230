"""Seeded generators for the five MoE-layer workloads and for small test shapes.

Shapes follow the OLMoE-1B-7B layer that the page "LLM 分布式推理基础（一）/
MoE 分布式推理基础（基于 vLLM）" (cnblogs, paitsai) uses throughout: E=64
experts, top-K=8, hidden H=2048, expert intermediate I=1024 (its header and
notation section). Weight shapes follow that page's notation: W_gate is (H, E),
each expert's W13 is (H, 2I) with the gate half in columns [0, I) and the up
half in [I, 2I), and W2 is (I, H).

Every array is drawn with numpy's PCG64 (`numpy.random.default_rng(seed)`) as
float32 standard normals times the stated standard deviation, in the fixed
order x, W_gate, W13 (expert 0..E-1), W2 (expert 0..E-1). For bf16 workloads
the float32 draw is rounded to bfloat16 with round-to-nearest-even; the
`*_f32` arrays then hold exactly the bf16 values (widening bf16 to float32 is
exact), and `bits(name)` returns the raw 16-bit patterns the device consumes.
No public dataset or trained checkpoint is involved: these synthetic arrays
stand in for OLMoE activations and weights.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# --------------------------------------------------------------------------
# bfloat16 storage helpers (input preparation only)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits.

    Inputs must be finite (the generators never produce NaN or infinity); for
    finite values the 32-bit sum below cannot overflow.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    lsb += np.uint32(0x7FFF)
    lsb += u
    lsb >>= 16
    return lsb.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def random_bf16_matrix(rng: np.random.Generator, shape, std: float = 1.0):
    """Draw N(0, std^2) float32 values and round them to bf16.

    Returns (bits uint16, exact values float32).
    """
    v = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    bits = f32_to_bf16_bits(v)
    return bits, bf16_bits_to_f32(bits)


# --------------------------------------------------------------------------
# Skewed-routing bias (input data for the skewed workload)
# --------------------------------------------------------------------------


def zipf_bias(E: int, s: float = 1.2, scale: float = 3.0, forced_zero_every: int = 8):
    """Per-expert logit bias: scale * ln(Zipf(s) probability of rank e+1).

    Expert e gets rank r = e + 1, with q_r = r^-s / sum_{j=1..E} j^-s, and
    bias_e = scale * ln q_r. Experts with e % forced_zero_every ==
    forced_zero_every - 1 get -inf, so they receive no rows, and these empty
    experts sit both among the hot and the cold ones. Returned as float32.
    """
    r = np.arange(1, E + 1, dtype=np.float64)
    q = r ** (-s)
    q = q / q.sum()
    bias = scale * np.log(q)
    if forced_zero_every:
        bias[forced_zero_every - 1 :: forced_zero_every] = -np.inf
    return bias.astype(np.float32)


# --------------------------------------------------------------------------
# Layer workloads
# --------------------------------------------------------------------------


@dataclasses.dataclass
class LayerWorkload:
    name: str
    n: int
    H: int
    I: int  # noqa: E741  (the pages' name for the expert intermediate size)
    E: int
    K: int
    dtype: str  # "bf16" or "f32": storage / compute dtype of x, weights and y
    renorm: bool
    seed: int
    x_f32: np.ndarray  # (n, H)
    W_gate_f32: np.ndarray  # (H, E)
    W13_f32: np.ndarray  # (E, H, 2I)
    W2_f32: np.ndarray  # (E, I, H)
    bias: Optional[np.ndarray]  # (E,) float32 or None
    _bits: dict = dataclasses.field(default_factory=dict, repr=False)

    def bits(self, name: str) -> np.ndarray:
        """Raw storage of `x`, `W_gate`, `W13` or `W2`: uint16 bf16 bits or float32."""
        arr = getattr(self, name + "_f32")
        if self.dtype == "f32":
            return arr
        if name not in self._bits:
            self._bits[name] = f32_to_bf16_bits(arr)
        return self._bits[name]

    @property
    def flops_grouped_gemm(self) -> float:
        """2 flops per multiply-add: GEMM1 2*nK*H*2I plus GEMM2 2*nK*I*H = 6*nK*H*I."""
        return 6.0 * self.n * self.K * self.H * self.I


def _draw(rng, shape, std, dtype, bits_out=None, key=None):
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    if dtype == "bf16":
        b = f32_to_bf16_bits(v)
        if bits_out is not None:
            bits_out[key] = b
        return bf16_bits_to_f32(b)
    return v


def make_layer(
    n: int,
    H: int,
    I: int,  # noqa: E741
    E: int,
    K: int,
    dtype: str = "bf16",
    renorm: bool = False,
    seed: int = 0,
    bias: Optional[np.ndarray] = None,
    x_std: float = 1.0,
    w_std: float = 0.02,
    name: str = "custom",
) -> LayerWorkload:
    """Draw one layer workload: x ~ N(0, x_std^2), all weights ~ N(0, w_std^2)."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    rng = np.random.default_rng(seed)
    bits: dict = {}
    x = _draw(rng, (n, H), x_std, dtype, bits, "x")
    W_gate = _draw(rng, (H, E), w_std, dtype, bits, "W_gate")
    W13 = _draw(rng, (E, H, 2 * I), w_std, dtype, bits, "W13")
    W2 = _draw(rng, (E, I, H), w_std, dtype, bits, "W2")
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (E,)
    return LayerWorkload(name, n, H, I, E, K, dtype, renorm, seed, x, W_gate, W13, W2, bias, bits)


# --------------------------------------------------------------------------
# One GPU's expert-parallel share: pre-received rows, two micro-batches
# --------------------------------------------------------------------------


@dataclasses.dataclass
class EPShareMicroBatch:
    seed: int
    counts: np.ndarray  # (E_local,) rows per local expert
    source_counts: np.ndarray  # (S, E_local) rows each source rank sent per expert
    eid: np.ndarray  # (R,) int32 local expert of each arrival row, in arrival order
    src: np.ndarray  # (R,) int32 arrival position of each row (the combine order)
    x_f32: np.ndarray  # (R, H) exact bf16 values
    _bits: Optional[np.ndarray] = dataclasses.field(default=None, repr=False)

    def x_bits(self) -> np.ndarray:
        if self._bits is None:
            self._bits = f32_to_bf16_bits(self.x_f32)
        return self._bits


@dataclasses.dataclass
class EPShareWorkload:
    name: str
    R: int
    H: int
    I: int  # noqa: E741
    E_local: int
    S: int
    W13_f32: np.ndarray  # (E_local, H, 2I)
    W2_f32: np.ndarray  # (E_local, I, H)
    micro_batches: list
    _bits: dict = dataclasses.field(default_factory=dict, repr=False)

    def bits(self, name: str) -> np.ndarray:
        if name not in self._bits:
            self._bits[name] = f32_to_bf16_bits(getattr(self, name + "_f32"))
        return self._bits[name]

    @property
    def flops_per_micro_batch(self) -> float:
        return 6.0 * self.R * self.H * self.I


def make_micro_batch(seed: int, R: int, H: int, E_local: int, S: int, alpha: float) -> EPShareMicroBatch:
    """Rows one GPU receives in one micro-batch of an expert-parallel exchange.

    Draw order: expert shares ~ Dirichlet(alpha * 1), counts c ~ Multinomial(R,
    shares); for each local expert e, its c_e rows are split over S source ranks
    by Multinomial(c_e, uniform); then the row payload X ~ N(0, 1). Rows arrive
    rank-major (source 0's rows first) and each source's chunk is sorted by
    expert, as an all-to-all of expert-sorted local buffers delivers them.
    """
    rng = np.random.default_rng(seed)
    shares = rng.dirichlet(np.full(E_local, alpha))
    counts = rng.multinomial(R, shares)
    source_counts = np.zeros((S, E_local), dtype=np.int64)
    for e in range(E_local):
        source_counts[:, e] = rng.multinomial(int(counts[e]), np.full(S, 1.0 / S))
    eid = np.concatenate(
        [np.full(int(source_counts[s, e]), e, dtype=np.int32) for s in range(S) for e in range(E_local)]
    ).astype(np.int32)
    assert eid.shape == (R,)
    bits: dict = {}
    x = _draw(rng, (R, H), 1.0, "bf16", bits, "x")
    src = np.arange(R, dtype=np.int32)
    return EPShareMicroBatch(seed, counts.astype(np.int64), source_counts, eid, src, x, bits["x"])


def make_ep_share(
    R: int = 16384,
    H: int = 2048,
    I: int = 1024,  # noqa: E741
    E_local: int = 8,
    S: int = 8,
    alpha: float = 0.5,
    weight_seed: int = 0,
    batch_seeds=(1, 2),
    w_std: float = 0.02,
    name: str = "ep_share_bf16",
) -> EPShareWorkload:
    rng = np.random.default_rng(weight_seed)
    bits: dict = {}
    W13 = _draw(rng, (E_local, H, 2 * I), w_std, "bf16", bits, "W13")
    W2 = _draw(rng, (E_local, I, H), w_std, "bf16", bits, "W2")
    mbs = [make_micro_batch(s, R, H, E_local, S, alpha) for s in batch_seeds]
    return EPShareWorkload(name, R, H, I, E_local, S, W13, W2, mbs, bits)


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------

CONFIGS = {
    # Tiny fp32 layer: softmax then top-2 with renormalised weights.
    "tiny_f32": dict(n=64, H=128, I=64, E=8, K=2, dtype="f32", renorm=True, seed=0),
    # OLMoE-shaped layer, bf16 storage with fp32 accumulation, no renormalisation.
    "olmoe_bf16": dict(n=4096, H=2048, I=1024, E=64, K=8, dtype="bf16", renorm=False, seed=0),
    # Skewed routing at the OLMoE shape: Zipf(1.2) logit bias, 8 experts forced empty.
    "olmoe_skewed_bf16": dict(
        n=4096, H=2048, I=1024, E=64, K=8, dtype="bf16", renorm=False, seed=0, bias="zipf"
    ),
    # Decode-like small batch: weight streaming dominates.
    "decode_bf16": dict(n=32, H=2048, I=1024, E=64, K=8, dtype="bf16", renorm=False, seed=0),
    # One GPU's expert-parallel share with two micro-batches (built by make_ep_share).
    "ep_share_bf16": dict(R=16384, H=2048, I=1024, E_local=8, S=8, alpha=0.5),
}


def make_config(name: str):
    """Build one of the named workloads."""
    cfg = dict(CONFIGS[name])
    if name == "ep_share_bf16":
        return make_ep_share(**cfg, name=name)
    bias = None
    if cfg.pop("bias", None) == "zipf":
        bias = zipf_bias(cfg["E"])
    return make_layer(**cfg, bias=bias, name=name)
