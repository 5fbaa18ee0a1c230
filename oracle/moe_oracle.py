"""fp64 CPU oracle of the single-GPU MoE expert layer: forward and its gradient.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does, and this module imports nothing from the product path.

It is the plain definition of what the layer computes, written from
[MoE-vLLM] §1.2 "MoE Forward": the Hugging Face `OlmoeTopKRouter` /
`OlmoeExperts.forward` source the page quotes, and its Algorithm 2
"Single-GPU MoE Forward". Floating point is fp64 throughout; inputs are the
exact values the device sees (bf16 or fp32, widened). Library primitives used
as steps: numpy matmul, exp, sort and nonzero. Nothing is blocked, fused or
reordered beyond what the definition states. The backward at the end of the
file is the chain rule of that forward, pinned by finite differences.

Readings taken where the pages leave a step open (each is also stated where it
is used):
  * Selection runs on the fp32 router logits, ordered by (logit descending,
    expert index ascending). Softmax is strictly increasing, so this is the
    same order as ranking the probabilities with ties to the lowest index, but
    it does not depend on how exp rounds. Slot 0 holds the largest.
  * Softmax subtracts the row maximum; an expert whose logit is -inf gets
    probability 0.
  * Within one expert's segment the pairs (i, k) are kept in ascending flat
    index f = i*K + k, which is ascending token order (a token picks an expert
    at most once). The moe_align_block_size example in [MoE-vLLM] §2.3 fixes
    this order.
  * gate = columns [0, I) of W13, up = columns [I, 2I); SiLU(z) = z / (1 + e^-z).
  * The per-rank split sizes are Algorithm 5 step 3 of [MoE-vLLM] §2.4 applied
    to one GPU's routing: split j counts the pairs whose expert e has
    floor(e / (E/ep)) = j.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Router: Algorithm 2 steps 1-3 ([MoE-vLLM] §1.2, OlmoeTopKRouter)
# ---------------------------------------------------------------------------


def router_logits(x, W_gate, bias=None) -> np.ndarray:
    """Algorithm 2 step 1: logits = x · W_gate, shape (n, E), in fp64.

    `bias` (E,) is an optional per-expert logit offset added after the
    product; -inf entries stay -inf. Exact up to fp64 rounding.
    """
    logits = np.asarray(x, dtype=np.float64) @ np.asarray(W_gate, dtype=np.float64)
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits


def round_to_f32(a) -> np.ndarray:
    """Round to float32 (round-to-nearest-even): the precision routing decisions are taken in."""
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def route_from_logits(logits_f32, K: int, renorm: bool, keep_fp64: bool = False):
    """Algorithm 2 steps 2-3: p = softmax(logits); (w_top, e_top) = TopK(p, K).

    The router code in [MoE-vLLM] §1.2 takes `torch.topk(router_probs, k=K)`
    and, when `norm_topk_prob` is set, divides the K weights by their sum.
    The ranking key is the fp32 logit (descending) with ties to the lowest
    expert index; the weights are the fp64 softmax of those fp32 logits.

    `keep_fp64` takes the logits as given (no rounding to fp32): the same
    definition in exact arithmetic, which the finite-difference check of the
    gradients needs (rounding the logits to fp32 would swamp a small step).

    Returns e_top (n, K) int32, w_top (n, K) fp64, p (n, E) fp64.
    """
    if keep_fp64:
        L = np.asarray(logits_f32, dtype=np.float64)
    else:
        L = np.asarray(logits_f32, dtype=np.float32).astype(np.float64)
    n, E = L.shape
    if not 1 <= K <= E:
        raise ValueError(f"K={K} must lie in [1, E={E}]")
    # A stable sort of the negated logits keeps equal logits in ascending
    # expert order (negation is exact; -0.0 and +0.0 compare equal).
    order = np.argsort(-L, axis=1, kind="stable")
    e_top = order[:, :K]
    m = L.max(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        ex = np.exp(L - m)
    p = ex / ex.sum(axis=1, keepdims=True)
    w_top = np.take_along_axis(p, e_top, axis=1)
    if renorm:
        w_top = w_top / w_top.sum(axis=1, keepdims=True)
    return e_top.astype(np.int32), w_top, p


def topk_margin(logits_f32, K: int) -> np.ndarray:
    """Per row, (K-th largest logit) - ((K+1)-th largest); +inf when K == E.

    Not part of the method: tests use it to tell rows whose top-K set is
    decided by a wide margin from near-ties, where a rounding difference in
    the logits may legitimately select a different expert.
    """
    L = np.sort(np.asarray(logits_f32, dtype=np.float64), axis=1)[:, ::-1]
    if K >= L.shape[1]:
        return np.full(L.shape[0], np.inf)
    with np.errstate(invalid="ignore"):
        return L[:, K - 1] - L[:, K]


# ---------------------------------------------------------------------------
# Dispatch metadata: counts, offsets, splits, permutation
# ---------------------------------------------------------------------------


def expert_counts(e_top, E: int) -> np.ndarray:
    """n_e = sum over (i, k) of 1[e_top[i, k] = e] ([MoE-vLLM] §1.2, hit statistics)."""
    e_top = np.asarray(e_top)
    return np.array([np.count_nonzero(e_top == e) for e in range(E)], dtype=np.int64)


def offsets_from_counts(counts) -> np.ndarray:
    """Exclusive prefix sum: offsets[0] = 0, offsets[e+1] = offsets[e] + n_e (length E+1)."""
    counts = np.asarray(counts, dtype=np.int64)
    out = np.zeros(counts.size + 1, dtype=np.int64)
    out[1:] = np.cumsum(counts)
    return out


def splits_from_offsets(offsets, ep: int) -> np.ndarray:
    """Split j = offsets[(j+1)E/ep] - offsets[jE/ep]: rows for the j-th block of E/ep experts."""
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.size - 1
    if ep < 1 or E % ep:
        raise ValueError(f"ep={ep} must divide E={E}")
    El = E // ep
    return np.array([offsets[(j + 1) * El] - offsets[j * El] for j in range(ep)], dtype=np.int64)


def splits_by_rank(e_top, E: int, ep: int) -> np.ndarray:
    """Algorithm 5 step 3 of [MoE-vLLM] §2.4: send_sizes[j] = sum 1[floor(e_top / E_l) = j]."""
    if ep < 1 or E % ep:
        raise ValueError(f"ep={ep} must divide E={E}")
    El = E // ep
    owner = np.asarray(e_top) // El
    return np.array([np.count_nonzero(owner == j) for j in range(ep)], dtype=np.int64)


def permutation(e_top, E: int):
    """Expert-major order of the n*K (token, slot) pairs, and its inverse.

    Algorithm 2 step 5 builds I_e = {(i, k) : e_top[i, k] = e} for e = 0..E-1;
    laying the sets end to end, each in ascending flat index f = i*K + k,
    gives perm[p] = f (the torchtitan `_local_reorder` / vLLM
    moe_align_block_size order, [goin] §2.2 and [MoE-vLLM] §2.3), and
    inv[perm[p]] = p (the E-major to T-major inversion of [goin] §2.3's kernel
    table). Both int64, length n*K.
    """
    flat = np.asarray(e_top).reshape(-1)
    parts = [np.flatnonzero(flat == e) for e in range(E)]
    perm = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    perm = perm.astype(np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int64)
    return perm, inv


# ---------------------------------------------------------------------------
# Experts: Algorithm 2 steps 7-9 and the SwiGLU two-GEMM form (§1.2)
# ---------------------------------------------------------------------------


def expert_gate_up(X_e, W13_e) -> np.ndarray:
    """Algorithm 2 step 8: G_e = SiLU(X_e·W13[:, :I]) * (X_e·W13[:, I:]), in fp64.

    [MoE-vLLM] §1.2: gate_up = X_e @ W13[e] of shape (n_e, 2I); gate, up =
    gate_up.chunk(2, -1); h = silu(gate) * up.
    """
    X_e = np.asarray(X_e, dtype=np.float64)
    W13_e = np.asarray(W13_e, dtype=np.float64)
    I = W13_e.shape[1] // 2  # noqa: E741
    gate_up = X_e @ W13_e
    gate, up = gate_up[:, :I], gate_up[:, I:]
    with np.errstate(over="ignore"):
        return gate / (1.0 + np.exp(-gate)) * up


def expert_ffn(X_e, W13_e, W2_e) -> np.ndarray:
    """Algorithm 2 steps 8-9: Y_e = G_e · W2[e], with G_e from expert_gate_up; fp64."""
    return expert_gate_up(X_e, W13_e) @ np.asarray(W2_e, dtype=np.float64)


def weighted_rows_token_order(Y_perm, inv, w_top, n: int, K: int) -> np.ndarray:
    """Z[i*K + k] = w_top[i, k] · Y_perm[inv[i*K + k]]; fp64.

    The summands of Algorithm 2 step 11 ([MoE-vLLM] §1.2: each expert output
    row times its routing weight), laid out in flat pair (token-major) order,
    which is where the fused second MoE layer of [Fusion] §4.2.5 lands them
    (gather back to token order and weighting folded into the expert GEMM).
    Summing each token's K consecutive rows gives combine_slot_order.
    """
    Y_perm = np.asarray(Y_perm, dtype=np.float64)
    inv = np.asarray(inv).reshape(n * K)
    w = np.asarray(w_top, dtype=np.float64).reshape(n * K)
    return w[:, None] * Y_perm[inv]


def combine_slot_order(Y_perm, inv, w_top, n: int, K: int) -> np.ndarray:
    """y[i] = sum_{k=0..K-1} w_top[i, k] · Y_perm[inv[i*K + k]], k ascending; fp64.

    Algorithm 2 steps 10-11 (scatter-add of each row times its routing
    weight), gathered per token as the top-K slot reduction of [goin] §2.3.
    `w_top=None` means unit weights (a plain un-permute when K = 1).
    """
    Y_perm = np.asarray(Y_perm, dtype=np.float64)
    inv = np.asarray(inv).reshape(n, K)
    y = np.zeros((n, Y_perm.shape[1]), dtype=np.float64)
    for k in range(K):
        rows = Y_perm[inv[:, k]]
        if w_top is None:
            y += rows
        else:
            y += np.asarray(w_top, dtype=np.float64)[:, k : k + 1] * rows
    return y


# ---------------------------------------------------------------------------
# Whole layer: Algorithm 2
# ---------------------------------------------------------------------------


def forward(
    x,
    W_gate,
    W13,
    W2,
    K: int,
    renorm: bool,
    bias=None,
    routing_logits_f32=None,
    ep: int = 1,
    keep_permuted: bool = False,
    fp64_routing: bool = False,
):
    """Algorithm 2 of [MoE-vLLM] §1.2, with its dispatch metadata.

    Steps 1-3 route (from `routing_logits_f32` when given, else from the fp64
    logits rounded to fp32); steps 4-12 loop over experts e = 0..E-1, skip
    empty ones, gather X_e, run the SwiGLU expert and scatter-add each output
    row times its weight into y (fp64, starting at zero). `fp64_routing`
    routes from the fp64 logits themselves (see route_from_logits).

    Returns a dict with logits (fp64 or None), logits_f32, e_top, w_top, p,
    counts, offsets, splits, perm, inv, y, and Y_perm (expert-major expert
    outputs, fp64) when keep_permuted.
    """
    x = np.asarray(x)
    n, H = x.shape
    E = np.asarray(W_gate).shape[1]
    logits = None
    if routing_logits_f32 is None:
        logits = router_logits(x, W_gate, bias)
        routing_logits_f32 = logits if fp64_routing else round_to_f32(logits)
    e_top, w_top, p = route_from_logits(routing_logits_f32, K, renorm, keep_fp64=fp64_routing)

    counts = expert_counts(e_top, E)
    offsets = offsets_from_counts(counts)
    splits = splits_by_rank(e_top, E, ep)
    perm, inv = permutation(e_top, E)

    y = np.zeros((n, H), dtype=np.float64)
    Y_perm = np.zeros((n * K, H), dtype=np.float64) if keep_permuted else None
    for e in range(E):
        seg = perm[offsets[e] : offsets[e + 1]]  # I_e, ascending (i, k)
        if seg.size == 0:
            continue
        tok, slot = seg // K, seg % K
        Y_e = expert_ffn(x[tok], W13[e], W2[e])
        if keep_permuted:
            Y_perm[offsets[e] : offsets[e + 1]] = Y_e
        np.add.at(y, tok, Y_e * w_top[tok, slot][:, None])
    return dict(
        logits=logits,
        logits_f32=np.asarray(routing_logits_f32, dtype=np.float32),
        routing_logits=np.asarray(routing_logits_f32, dtype=np.float64 if fp64_routing else np.float32),
        e_top=e_top,
        w_top=w_top,
        p=p,
        counts=counts,
        offsets=offsets,
        splits=splits,
        perm=perm,
        inv=inv,
        y=y,
        Y_perm=Y_perm,
    )


def grouped_swiglu(x_perm, offsets, W13, W2) -> np.ndarray:
    """Expert outputs for rows already in expert-major order: segment e of
    `x_perm` (rows offsets[e]..offsets[e+1]) goes through expert e's SwiGLU
    FFN (Algorithm 2 steps 8-9). fp64, shape (rows, H)."""
    x_perm = np.asarray(x_perm)
    offsets = np.asarray(offsets, dtype=np.int64)
    H = np.asarray(W2).shape[2]
    out = np.zeros((x_perm.shape[0], H), dtype=np.float64)
    for e in range(offsets.size - 1):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            out[a:b] = expert_ffn(x_perm[a:b], W13[e], W2[e])
    return out


def grouped_gate_up(x_perm, offsets, W13) -> np.ndarray:
    """Algorithm 2 step 8 for every expert segment of expert-major rows; (rows, I) fp64."""
    x_perm = np.asarray(x_perm)
    offsets = np.asarray(offsets, dtype=np.int64)
    I = np.asarray(W13).shape[2] // 2  # noqa: E741
    out = np.zeros((x_perm.shape[0], I), dtype=np.float64)
    for e in range(offsets.size - 1):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            out[a:b] = expert_gate_up(x_perm[a:b], W13[e])
    return out


def grouped_down(h, offsets, W2) -> np.ndarray:
    """Algorithm 2 step 9 for every expert segment: Y_e = G_e · W2[e]; (rows, H) fp64."""
    h = np.asarray(h)
    offsets = np.asarray(offsets, dtype=np.int64)
    H = np.asarray(W2).shape[2]
    out = np.zeros((h.shape[0], H), dtype=np.float64)
    for e in range(offsets.size - 1):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            out[a:b] = np.asarray(h[a:b], dtype=np.float64) @ np.asarray(W2[e], dtype=np.float64)
    return out


def ep_share_forward(x_recv, eid, W13, W2):
    """One GPU's expert-parallel share for one micro-batch of received rows.

    [goin] §2.2: received rows arrive rank-major; `_permute` makes them
    expert-major for the grouped GEMM, the local experts run, and `_unpermute`
    restores arrival order before the reverse exchange (whose weighted top-K
    reduction happens on the source GPU). With one row per pair this is the
    layer's permutation at K = 1 with unit weights.

    Returns dict(counts, offsets, perm, inv, Y_perm, out) with out (R, H) fp64.
    """
    eid = np.asarray(eid).reshape(-1, 1)
    E = np.asarray(W13).shape[0]
    R = eid.shape[0]
    counts = expert_counts(eid, E)
    offsets = offsets_from_counts(counts)
    perm, inv = permutation(eid, E)
    Y_perm = grouped_swiglu(np.asarray(x_recv)[perm], offsets, W13, W2)
    out = combine_slot_order(Y_perm, inv, None, R, 1)
    return dict(counts=counts, offsets=offsets, perm=perm, inv=inv, Y_perm=Y_perm, out=out)


# ---------------------------------------------------------------------------
# Backward: the gradient of the layer above (chain rule, fp64)
# ---------------------------------------------------------------------------
#
# The pages give no formulas for the training backward; they name its pieces:
# the backward of a dispatch is a combine and the backward of a combine is a
# dispatch that also yields the routing-score gradient ([Fusion] §6.2.4,
# [goin] §2.3 (d) and the top-K gradient kernels of its table (e)). What is
# computed is the plain definition: the derivative of `forward`, with the
# top-K selection held fixed (it is piecewise constant), written out step by
# step in the reverse order of Algorithm 2.


def gate_up_preactivations(x_perm, offsets, W13) -> np.ndarray:
    """[gate | up] = X_e · W13[e] for every expert segment of expert-major rows; (rows, 2I) fp64."""
    x_perm = np.asarray(x_perm, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    out = np.zeros((x_perm.shape[0], np.asarray(W13).shape[2]), dtype=np.float64)
    for e in range(offsets.size - 1):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            out[a:b] = x_perm[a:b] @ np.asarray(W13[e], dtype=np.float64)
    return out


def combine_backward(dy, Y_perm, inv, w_top, n: int, K: int):
    """Gradient of combine_slot_order (the backward of a combine is a dispatch).

    With y[i] = sum_k w[i,k] · Y_perm[inv[iK+k]]:
      dY_perm[inv[iK+k]] = w[i,k] · dy[i]     (dy sent to each of the token's rows)
      dw[i,k] = <dy[i], Y_perm[inv[iK+k]]>     (the routing-score gradient)
    Returns dY_perm (n*K, H) and dw (n, K), fp64.
    """
    dy = np.asarray(dy, dtype=np.float64)
    Y_perm = np.asarray(Y_perm, dtype=np.float64)
    inv = np.asarray(inv).reshape(n, K)
    w = np.asarray(w_top, dtype=np.float64).reshape(n, K)
    dY_perm = np.zeros_like(Y_perm)
    dw = np.zeros((n, K), dtype=np.float64)
    for k in range(K):
        dY_perm[inv[:, k]] = w[:, k : k + 1] * dy
        dw[:, k] = np.sum(dy * Y_perm[inv[:, k]], axis=1)
    return dY_perm, dw


def dispatch_backward(dX_perm, inv, n: int, K: int) -> np.ndarray:
    """Gradient of the row gather X_perm[p] = x[perm[p] / K] (the backward of a
    dispatch is a combine with unit weights): dx[i] = sum_k dX_perm[inv[iK+k]]."""
    return combine_slot_order(dX_perm, inv, None, n, K)


def swiglu_backward(dh, gate_up) -> np.ndarray:
    """Gradient of h = SiLU(g) · u with respect to [g | u].

    SiLU(g) = g·s with s = 1 / (1 + e^-g), so d SiLU/dg = s · (1 + g·(1 - s)):
      dg = dh · u · s · (1 + g·(1 - s)),   du = dh · g · s.
    Returns [dg | du], shape (rows, 2I), fp64.
    """
    dh = np.asarray(dh, dtype=np.float64)
    gu = np.asarray(gate_up, dtype=np.float64)
    I = gu.shape[1] // 2  # noqa: E741
    g, u = gu[:, :I], gu[:, I:]
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-g))
    return np.concatenate([dh * u * s * (1.0 + g * (1.0 - s)), dh * g * s], axis=1)


def grouped_data_grad(dout, offsets, W) -> np.ndarray:
    """Gradient of out_e = in_e · W[e] with respect to in_e: din_e = dout_e · W[e]^T per segment; fp64."""
    dout = np.asarray(dout, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    W = np.asarray(W)
    din = np.zeros((dout.shape[0], W.shape[1]), dtype=np.float64)
    for e in range(offsets.size - 1):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            din[a:b] = dout[a:b] @ np.asarray(W[e], dtype=np.float64).T
    return din


def grouped_weight_grad(inp, dout, offsets) -> np.ndarray:
    """Gradient of out_e = in_e · W[e] with respect to W[e]: dW[e] = in_e^T · dout_e.

    An expert with no rows gets a zero gradient. Returns (E, cols(in), cols(dout)) fp64.
    """
    inp = np.asarray(inp, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.size - 1
    dW = np.zeros((E, inp.shape[1], dout.shape[1]), dtype=np.float64)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            dW[e] = inp[a:b].T @ dout[a:b]
    return dW


def router_backward(routing_logits, e_top, dw, K: int, renorm: bool, x=None, W_gate=None, keep_fp64: bool = False):
    """Gradient through Algorithm 2 steps 1-3 given dw = dL/dw_top.

    Top-K picks s[i,k] = p[i, e_top[i,k]] (the selection is held fixed). With
    renormalisation w = s / S, S = sum_k s, so ds_k = (dw_k - sum_j dw_j w_j) / S;
    without it ds = dw. The dense dp has ds at the selected experts and zero
    elsewhere, and the softmax backward gives dlogits = p ⊙ (dp - <p, dp>).
    The router product logits = x · W_gate + bias then gives
    dx = dlogits · W_gate^T, dW_gate = x^T · dlogits, dbias = sum_i dlogits[i].

    Returns dict(dlogits (n, E), and when x and W_gate are given dx, dW_gate,
    dbias), fp64.
    """
    e_top = np.asarray(e_top).astype(np.int64)
    dw = np.asarray(dw, dtype=np.float64)
    _, w_top, p = route_from_logits(routing_logits, K, renorm, keep_fp64=keep_fp64)
    if renorm:
        s = np.take_along_axis(p, e_top, axis=1)
        S = s.sum(axis=1, keepdims=True)
        ds = (dw - np.sum(dw * w_top, axis=1, keepdims=True)) / S
    else:
        ds = dw
    dp = np.zeros_like(p)
    np.put_along_axis(dp, e_top, ds, axis=1)
    dlogits = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    out = dict(dlogits=dlogits)
    if x is not None and W_gate is not None:
        out["dx"] = dlogits @ np.asarray(W_gate, dtype=np.float64).T
        out["dW_gate"] = np.asarray(x, dtype=np.float64).T @ dlogits
        out["dbias"] = dlogits.sum(axis=0)
    return out


def backward(x, W_gate, W13, W2, K: int, renorm: bool, dy, bias=None, fp64_routing: bool = False,
             routing_logits_f32=None):
    """Gradients of the layer's y = forward(...)["y"] for an upstream dy (n, H).

    `routing_logits_f32`, when given, is the routing input of steps 1-3 (as in
    forward); the router's own gradients are then taken at those logits.

    Steps, in the reverse order of Algorithm 2:
      1. combine backward: dY_perm, dw (combine_backward);
      2. GEMM2: dh = dY_perm · W2[e]^T, dW2[e] = h_e^T · dY_e;
      3. SwiGLU: [dg | du] from dh and the pre-activations (swiglu_backward);
      4. GEMM1: dX_perm = [dg | du] · W13[e]^T, dW13[e] = X_e^T · [dg | du];
      5. dispatch backward: dx = sum over each token's rows of dX_perm;
      6. router: dlogits, and its share of dx, dW_gate and dbias.
    Returns dict(dx, dW_gate, dbias, dW13, dW2, dlogits, dw, plus the
    intermediates dY_perm, dgu, dX_perm, gate_up, h, x_perm) in fp64, and the
    forward dict under "fwd".
    """
    x = np.asarray(x)
    n, H = x.shape
    f = forward(x, W_gate, W13, W2, K, renorm, bias=bias, keep_permuted=True, fp64_routing=fp64_routing,
                routing_logits_f32=routing_logits_f32)
    perm, inv, offsets = f["perm"], f["inv"], f["offsets"]
    x_perm = np.asarray(x, dtype=np.float64)[perm // K]
    gate_up = gate_up_preactivations(x_perm, offsets, W13)
    I = gate_up.shape[1] // 2  # noqa: E741
    with np.errstate(over="ignore"):
        h = gate_up[:, :I] / (1.0 + np.exp(-gate_up[:, :I])) * gate_up[:, I:]

    dY_perm, dw = combine_backward(dy, f["Y_perm"], inv, f["w_top"], n, K)
    dh = grouped_data_grad(dY_perm, offsets, W2)
    dW2 = grouped_weight_grad(h, dY_perm, offsets)
    dgu = swiglu_backward(dh, gate_up)
    dX_perm = grouped_data_grad(dgu, offsets, W13)
    dW13 = grouped_weight_grad(x_perm, dgu, offsets)
    dx = dispatch_backward(dX_perm, inv, n, K)
    r = router_backward(f["routing_logits"], f["e_top"], dw, K, renorm, x=x, W_gate=W_gate, keep_fp64=fp64_routing)
    return dict(
        dx=dx + r["dx"],
        dW_gate=r["dW_gate"],
        dbias=r["dbias"],
        dW13=dW13,
        dW2=dW2,
        dlogits=r["dlogits"],
        dw=dw,
        dY_perm=dY_perm,
        dgu=dgu,
        dX_perm=dX_perm,
        gate_up=gate_up,
        h=h,
        x_perm=x_perm,
        fwd=f,
    )
