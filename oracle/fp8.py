"""fp64 CPU oracle of the layer with FP8 expert weights.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the test
suite, the smoke check and the benchmark's CPU-baseline leg, never by the
product path.

[Fusion] §8.4 ("低精度通信") lists FP8 payloads with per-token or per-block
scales and asks that the GEMM consume the low-precision format directly, and
§4.4 describes Mega MoE's first linear with low-precision weights prepared
ahead of time. Here the expert weights W13 and W2 are stored as FP8 E4M3 with
one fp32 scale per output column (a per-block scale whose block is the whole
contraction dimension), prepared once, and the layer is otherwise Algorithm 2.

FP8 E4M3 (the OCP 8-bit floating-point format, "E4M3FN"): 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
subnormals m * 2^-9; no infinities; the two codes with all exponent and
mantissa bits set (0x7F, 0xFF) are NaN, so the largest finite value is
1.75 * 2^8 = 448 (code 0x7E).

Readings (also listed with the design notes):
  * Scale of column n: s = amax_k |w[k, n]| / 448 in fp32 (one rounded
    division); s = 1 when the column is all zero.
  * Code of w: the E4M3 value nearest to the fp32 quotient w / s (one rounded
    fp32 division), ties to the code with an even mantissa, magnitudes beyond
    448 saturated to 448 (they can only arise from the rounding of w / s).
  * Dequantized weight: decode(code) * s, exact in fp64.

FP8 activations (the dispatch payload of §8.4: FP8 values that travel with a
scale per token, in a receive buffer that the FP8 GEMM reads as it is) and the
token-group padding of "0. goin" §2.1 (the quantized dispatcher pads each expert's group
of rows to a multiple of 16 for FP8 so that a quantized grouped GEMM sees
aligned groups). Readings:
  * Scale of token row i: s_i = amax_h |x[i, h]| / 448 in fp32, 1 for an
    all-zero row; codes as for the weights (nearest E4M3 of fp32 x / s_i).
    Each token is quantized once; its K copies in the receive buffer share
    the codes and the scale.
  * Receive buffer: expert-major rows in Algorithm 2's I_e order (ascending
    flat pair index), expert e's group starting at the padded offset
    P[e] = sum_{e' < e} 16 * ceil(n_e' / 16); the padding rows hold code 0
    and scale 0 (they contribute nothing and their outputs are never read).
  * The layer on FP8 activations: routing on the original activations (the
    router is not part of the dispatch payload), experts on the dequantized
    rows decode(code) * s_i and the dequantized FP8 weights.
"""

from __future__ import annotations

import numpy as np

from . import moe_oracle

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 codes (float64; NaN for 0x7F and 0xFF), from the format's definition."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m * 2.0**-9
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_decode_table()


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.int64)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to even mantissa, saturating at +-448); uint8.

    Written from the format: below the smallest normal 2^-6 the values are
    m * 2^-9, so the code is rint(|x| * 2^9) (m = 8 lands on code 8, the
    smallest normal); above it |x| = f * 2^E with f in [1, 2), the mantissa is
    rint((f - 1) * 8) with ties to even, a mantissa of 8 carries into the
    exponent, and the code is (E + 7) * 8 + m. Works on the exact values given
    (the callers pass fp32 quotients); NaN is not expected. oracle/brute.py
    restates the same map as a nearest-value search over the 127 non-negative
    codes, and the pins compare the two.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    sub = a < 2.0**-6
    m_sub = np.rint(a * 512.0)
    mant, ex = np.frexp(np.where(sub, 1.0, a))  # a = mant * 2^ex, mant in [0.5, 1)
    E = ex - 1
    m = np.rint((mant * 2.0 - 1.0) * 8.0)
    carry = m == 8
    E = np.where(carry, E + 1, E)
    m = np.where(carry, 0, m)
    code = np.where(sub, m_sub, (E + 7) * 8 + m).astype(np.int64)
    sign = (np.signbit(x) & (code != 0)).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def quantize_columns(W) -> tuple:
    """FP8 weights of one stack of matrices W (E, K, N) (row-major, K rows of N
    columns), one scale per output column n.

    Returns (codes (E, N, K) uint8 -- each column's K codes contiguous, the
    layout the device GEMMs read -- and scales (E, N) float32).
    """
    W32 = np.asarray(W, dtype=np.float32)
    amax = np.max(np.abs(W32), axis=1)  # (E, N) fp32, exact
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (W32 / scale[:, None, :]).astype(np.float32)  # one rounded fp32 division per weight
    codes = e4m3_encode(q)  # (E, K, N)
    return np.ascontiguousarray(np.transpose(codes, (0, 2, 1))), scale


def dequantize_columns(codes, scale) -> np.ndarray:
    """W'[e, k, n] = decode(codes[e, n, k]) * scale[e, n] in fp64, shape (E, K, N)."""
    v = e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[:, :, None]
    return np.transpose(v, (0, 2, 1))


def forward_fp8(x, W_gate, W13_codes, s13, W2_codes, s2, K: int, renorm: bool, bias=None, **kw):
    """Algorithm 2 with the dequantized FP8 expert weights (moe_oracle.forward on W13', W2')."""
    W13 = dequantize_columns(W13_codes, s13)
    W2 = dequantize_columns(W2_codes, s2)
    return moe_oracle.forward(x, W_gate, W13, W2, K, renorm, bias=bias, **kw)


TOKEN_GROUP = 16  # rows per padded expert group for FP8 ("0. goin" §2.1)


def quantize_rows(X) -> tuple:
    """Per-token FP8 of the rows of X (n, H): (codes (n, H) uint8, scales (n,) float32)."""
    X32 = np.asarray(X, dtype=np.float32)
    amax = np.max(np.abs(X32), axis=1) if X32.shape[1] else np.zeros(X32.shape[0], np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (X32 / scale[:, None]).astype(np.float32)  # one rounded fp32 division per element
    return e4m3_encode(q), scale


def dequantize_rows(codes, scale) -> np.ndarray:
    """X'[i, h] = decode(codes[i, h]) * scale[i] in fp64."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[:, None]


def round_to_bf16(a) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, fp32's exponent range), ties to
    the even significand, as fp64: frexp gives a in [0.5, 1) * 2^e, the
    significand is rounded to 2^-8 steps half-to-even, and scaled back."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def fp8_round_rows(X) -> np.ndarray:
    """X as per-row FP8 holds it: dequantize_rows(quantize_rows(X)), fp64."""
    return dequantize_rows(*quantize_rows(X))


def padded_offsets(counts, group: int = TOKEN_GROUP) -> np.ndarray:
    """Start of each expert's padded group: P[0] = 0, P[e+1] = P[e] + group * ceil(n_e / group)."""
    c = np.asarray(counts, dtype=np.int64)
    out = np.zeros(c.size + 1, dtype=np.int64)
    out[1:] = np.cumsum((c + group - 1) // group * group)
    return out


def dispatch_fp8(x, e_top, E: int, group: int = TOKEN_GROUP) -> dict:
    """The FP8 receive buffer of one GPU's experts.

    Returns dict(codes (R_pad, H) uint8, scales (R_pad,) float32, offsets (E+1)
    padded group starts, perm (R_pad,) flat pair index i*K + k of each row or -1
    for padding, inv (nK,) padded row of each pair, counts (E,)), where R_pad =
    offsets[E].
    """
    e_top = np.asarray(e_top)
    n, K = e_top.shape
    codes_tok, s_tok = quantize_rows(x)
    counts = moe_oracle.expert_counts(e_top, E)
    offs = moe_oracle.offsets_from_counts(counts)
    perm, _ = moe_oracle.permutation(e_top, E)
    P = padded_offsets(counts, group)
    R = int(P[-1])
    H = np.asarray(x).shape[1]
    codes = np.zeros((R, H), dtype=np.uint8)
    scales = np.zeros(R, dtype=np.float32)
    perm_p = np.full(R, -1, dtype=np.int64)
    inv_p = np.zeros(n * K, dtype=np.int64)
    for e in range(E):
        seg = perm[offs[e] : offs[e + 1]]  # I_e in ascending flat order
        rows = P[e] + np.arange(seg.size)
        codes[rows] = codes_tok[seg // K]
        scales[rows] = s_tok[seg // K]
        perm_p[rows] = seg
        inv_p[seg] = rows
    return dict(codes=codes, scales=scales, offsets=P, perm=perm_p, inv=inv_p, counts=counts)


def forward_fp8a(x, W_gate, W13_codes, s13, W2_codes, s2, K: int, renorm: bool, bias=None, routing_logits_f32=None,
                 fp8_h: bool = True):
    """Algorithm 2 with FP8 activations and FP8 weights: routed on x, the experts
    run on the dequantized per-token FP8 rows and the dequantized weights (fp64).
    With fp8_h (the layer's form), each expert's intermediate rows
    h = SiLU(gate) * up are quantized the same way before the down projection
    ([Fusion] §8.4 lists FP8 activations among its low-precision forms): h is
    rounded to bf16 as the bf16 layer stores it between the two products, then
    one fp32 scale per row and the nearest E4M3 code, decided in fp32 like the
    token rows' codes."""
    if routing_logits_f32 is None:
        routing_logits_f32 = moe_oracle.round_to_f32(moe_oracle.router_logits(x, W_gate, bias))
    codes, scales = quantize_rows(x)
    x_deq = dequantize_rows(codes, scales)
    W13 = dequantize_columns(W13_codes, s13)
    W2 = dequantize_columns(W2_codes, s2)
    out = moe_oracle.forward(x_deq, W_gate, W13, W2, K, renorm, bias=bias, routing_logits_f32=routing_logits_f32)
    if not fp8_h:
        return out
    # Steps 8-11 again with h quantized per row between the two products.
    n, H = x_deq.shape
    E = W13.shape[0]
    perm, offsets, w_top = out["perm"], out["offsets"], out["w_top"]
    y = np.zeros((n, H), dtype=np.float64)
    for e in range(E):
        seg = perm[offsets[e] : offsets[e + 1]]
        if seg.size == 0:
            continue
        tok, slot = seg // K, seg % K
        h = moe_oracle.expert_gate_up(x_deq[tok], W13[e])
        Y_e = fp8_round_rows(round_to_bf16(h)) @ W2[e]
        np.add.at(y, tok, Y_e * w_top[tok, slot][:, None])
    out["y"] = y
    return out
