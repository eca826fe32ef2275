"""Plain fp64 grouped GEMM for a mixture-of-experts layer (TEST INFRASTRUCTURE).

What is computed
----------------
Routing sends each token to a few experts, so expert e receives a variable
number n_e of rows; the layer multiplies each expert's rows by that expert's
weight.  With the routed rows sorted by expert (rows offsets[e] ..
offsets[e+1] - 1 belong to expert e):

    Y[r, :] = X[r, :] @ W[e]^T      for offsets[e] <= r < offsets[e+1]

X is [R, K] (R routed rows, K hidden), W is [E, N, K] (each expert's weight in
the [out, in] layout of a linear layer), Y is [R, N].  This is the MoE
workload whose uneven per-expert token counts the MeldKernel summary names as
the second source of SM imbalance ("Problem and motivation": expert token
counts differ from SM to SM; "Core method": the mapping is chosen from the
real counts at run time).

Readings: the pages give no formula, shapes or precision for the MoE kernel;
the plainest reading is the grouped product above, bf16 inputs, fp32
accumulation on the GPU, fp32 output.  An expert with no rows contributes
nothing.  Every value here is fp64; bf16 inputs are widened exactly.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def grouped_gemm(x_bits: np.ndarray, w_bits: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Y = X_e W_e^T per expert, fp64.  x_bits uint16 [R, K], w_bits uint16
    [E, N, K], offsets int [E + 1] (non-decreasing, offsets[0] = 0,
    offsets[E] = R).  Returns float64 [R, N]."""
    E, N, K = w_bits.shape
    R = x_bits.shape[0]
    offsets = np.asarray(offsets, dtype=np.int64)
    if offsets.shape != (E + 1,) or offsets[0] != 0 or offsets[-1] != R or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must run from 0 to R without decreasing")
    y = np.zeros((R, N))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b] = bf16_to_f64(x_bits[a:b]) @ bf16_to_f64(w_bits[e]).T
    return y


def abs_product_sums(x_bits: np.ndarray, w_bits: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """S[r, n] = sum_k |X[r, k] W_e[n, k]|: the scale of the error bound of a
    sum of K products accumulated in any order (Higham, "Accuracy and
    Stability of Numerical Algorithms", section 3.1: |fl(sum) - sum| <=
    gamma_{K} sum |terms|, gamma_K = K u / (1 - K u))."""
    E = w_bits.shape[0]
    y = np.zeros((x_bits.shape[0], w_bits.shape[1]))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b] = np.abs(bf16_to_f64(x_bits[a:b])) @ np.abs(bf16_to_f64(w_bits[e])).T
    return y


def gamma(n: int, unit_roundoff: float = 2.0 ** -24) -> float:
    """gamma_n = n u / (1 - n u) for fp32 (u = 2^-24)."""
    return n * unit_roundoff / (1 - n * unit_roundoff)
