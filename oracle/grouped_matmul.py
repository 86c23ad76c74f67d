"""GroupedMatMul, written out from its definition (float64, explicit loops).

Source: ONNX operator page "GroupedMatMul - 29", section Summary: for input
[M, K], weights [G, K, N] and group_indices [M, S], output [M, S, N] with
output[m, i] = input[m] @ weights[group_indices[m, i]], plus
bias[group_indices[m, i]] when the optional bias [G, N] is given.  Indices
outside [0, G) are invalid input; negative values do not wrap.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def grouped_matmul(inp, weights, group_indices, bias=None, out_dtype=None):
    inp = np.asarray(inp)
    weights = np.asarray(weights)
    idx = np.asarray(group_indices)
    if inp.ndim != 2 or weights.ndim != 3 or idx.ndim != 2:
        raise ValueError("ranks must be input 2, weights 3, group_indices 2")
    M, K = inp.shape
    G, K2, N = weights.shape
    if K2 != K or idx.shape[0] != M:
        raise ValueError("shape mismatch")
    if bias is not None:
        bias = np.asarray(bias)
        if bias.shape != (G, N):
            raise ValueError("bias must be [G, N]")
    S = idx.shape[1]
    if idx.size and (idx.min() < 0 or idx.max() >= G):
        raise ValueError("group index outside [0, G)")
    out = np.zeros((M, S, N), dtype=np.float64)
    for m in range(M):
        for i in range(S):
            g = int(idx[m, i])
            for n in range(N):
                acc = 0.0
                for c in range(K):
                    acc += float(inp[m, c]) * float(weights[g, c, n])
                if bias is not None:
                    acc += float(bias[g, n])
                out[m, i, n] = acc
    if out_dtype is None:
        out_dtype = inp.dtype
    return out.astype(out_dtype)


def grouped_matmul_rows(inp, weights, group_indices, bias=None, rows=None):
    """The same definition for selected token rows, one float64 vector-matrix
    product per (m, i) pair: output[r, i] = input[m] @ weights[g] (+ bias[g])
    with m = rows[r] and g = group_indices[m, i].  Returns float64 [len(rows),
    S, N]; rows=None means every row.  Fast enough for full-size samples;
    checked against the loop form above on random inputs."""
    inp = np.asarray(inp)
    weights = np.asarray(weights)
    idx = np.asarray(group_indices)
    M, K = inp.shape
    G, K2, N = weights.shape
    if K2 != K or idx.ndim != 2 or idx.shape[0] != M:
        raise ValueError("shape mismatch")
    if bias is not None:
        bias = np.asarray(bias)
        if bias.shape != (G, N):
            raise ValueError("bias must be [G, N]")
    rows = np.arange(M) if rows is None else np.asarray(rows)
    S = idx.shape[1]
    out = np.zeros((len(rows), S, N), dtype=np.float64)
    for r, m in enumerate(rows):
        x = inp[m].astype(np.float64)
        for i in range(S):
            g = int(idx[m, i])
            if g < 0 or g >= G:
                raise ValueError("group index outside [0, G)")
            out[r, i] = x @ weights[g].astype(np.float64)
            if bias is not None:
                out[r, i] += bias[g].astype(np.float64)
    return out
