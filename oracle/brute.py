"""Brute-force forms of the MoE layer for tiny inputs (test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of this package. This module is a
second, separately written statement of the same definitions as
`moe_oracle`, kept deliberately different in structure so that a slip in one
shows up as a disagreement with the other:

  * top-K by K passes of arg-max and by a full Python sort, instead of a
    stable numpy sort of negated logits;
  * softmax with Python's math.exp, one row at a time;
  * the permutation as the literal triple loop over (e, i, k);
  * the layer output token by token, with no permutation at all, and in the
    dense form sum_e 1[e in top(i)] w(i, e) FFN_e(x[i]).

Definitions follow [MoE-vLLM] §1.2 (router and experts source, Algorithm 2).
Pure-Python loops: use only for tiny sizes.
"""

from __future__ import annotations

import math

import numpy as np


def _key(v: float) -> float:
    return float(v)


def topk_argmax_passes(row, K: int):
    """K passes; each takes the largest remaining logit, lowest index on ties."""
    taken = [False] * len(row)
    out = []
    for _ in range(K):
        best = -1
        for e, v in enumerate(row):
            if taken[e]:
                continue
            if best < 0 or _key(v) > _key(row[best]):
                best = e
        taken[best] = True
        out.append(best)
    return out


def topk_full_sort(row, K: int):
    """Sort all experts by (logit descending, index ascending) and keep the first K."""
    return sorted(range(len(row)), key=lambda e: (-_key(row[e]), e))[:K]


def softmax_row(row):
    m = max(_key(v) for v in row)
    ex = [math.exp(_key(v) - m) if _key(v) != -math.inf else 0.0 for v in row]
    s = sum(ex)
    return [v / s for v in ex]


def route(logits_f32, K: int, renorm: bool):
    """Returns (e_top list of lists, w_top list of lists) by arg-max passes."""
    L = np.asarray(logits_f32, dtype=np.float32)
    e_top, w_top = [], []
    for row in L.tolist():
        ids = topk_argmax_passes(row, K)
        p = softmax_row(row)
        w = [p[e] for e in ids]
        if renorm:
            s = sum(w)
            w = [v / s for v in w]
        e_top.append(ids)
        w_top.append(w)
    return e_top, w_top


def permutation_triple_loop(e_top, E: int):
    """pos = 0; for e: for i: for k: if e_top[i][k] == e: perm[pos] = i*K + k; pos += 1."""
    n = len(e_top)
    K = len(e_top[0]) if n else 0
    perm = []
    for e in range(E):
        for i in range(n):
            for k in range(K):
                if e_top[i][k] == e:
                    perm.append(i * K + k)
    inv = [0] * len(perm)
    for p, f in enumerate(perm):
        inv[f] = p
    return perm, inv


def gate_up_token(x_i, W13_e):
    """One token's SwiGLU activation h (length I), with explicit loops over I."""
    x_i = np.asarray(x_i, dtype=np.float64)
    W13_e = np.asarray(W13_e, dtype=np.float64)
    I = W13_e.shape[1] // 2  # noqa: E741
    h = np.zeros(I, dtype=np.float64)
    for j in range(I):
        g = float(np.dot(x_i, W13_e[:, j]))
        u = float(np.dot(x_i, W13_e[:, I + j]))
        h[j] = g * (1.0 / (1.0 + math.exp(-g))) * u
    return h


def down_token(h_i, W2_e):
    """One row of the down projection, column by column."""
    h_i = np.asarray(h_i, dtype=np.float64)
    W2_e = np.asarray(W2_e, dtype=np.float64)
    return np.array([float(np.dot(h_i, W2_e[:, c])) for c in range(W2_e.shape[1])])


def ffn_token(x_i, W13_e, W2_e):
    """One token through one SwiGLU expert."""
    return down_token(gate_up_token(x_i, W13_e), W2_e)


def layer_per_token(x, e_top, w_top, W13, W2):
    """y[i] = sum_k w_top[i][k] · FFN_{e_top[i][k]}(x[i]); no permutation."""
    x = np.asarray(x, dtype=np.float64)
    n, H = x.shape
    y = np.zeros((n, H), dtype=np.float64)
    for i in range(n):
        for k, e in enumerate(e_top[i]):
            y[i] += w_top[i][k] * ffn_token(x[i], W13[e], W2[e])
    return y


def layer_dense(x, e_top, w_top, W13, W2):
    """y[i] = sum_e 1[e in top(i)] · w(i, e) · FFN_e(x[i]), summed over all experts."""
    x = np.asarray(x, dtype=np.float64)
    n, H = x.shape
    E = len(W13)
    y = np.zeros((n, H), dtype=np.float64)
    for i in range(n):
        weight = {e: w for e, w in zip(e_top[i], w_top[i])}
        for e in range(E):
            if e in weight:
                y[i] += weight[e] * ffn_token(x[i], W13[e], W2[e])
    return y


def e4m3_encode_by_search(x) -> np.ndarray:
    """The E4M3 encoder as a search: among the 127 non-negative finite values
    (codes 0x00..0x7E), the one nearest |x| (clamped to 448), the even code on
    a tie, with the sign of x unless the code is 0."""
    from .fp8 import e4m3_decode_table

    vals = e4m3_decode_table()[:0x7F]
    out = np.empty(np.shape(x), dtype=np.uint8)
    flat_x = np.asarray(x, dtype=np.float64).reshape(-1)
    flat_o = out.reshape(-1)
    for i, v in enumerate(flat_x):
        a = min(abs(v), 448.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        flat_o[i] = c | (0x80 if (np.signbit(v) and c != 0) else 0)
    return out
