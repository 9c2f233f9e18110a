"""Oracle of the expert layer's backward pass (TEST INFRASTRUCTURE ONLY: only
tests/, __graft_entry__.smoke() and bench.py's cpu_baseline may import it).

The learning path of the miniTE summary (§4.2 "The Native NVFP4 Learning
Path") differentiates the layer with a straight-through approximation: the
forward uses the NVFP4 operands, the backward multiplies BF16 operands with
BF16 GEMMs.  Those operands are either the saved BF16 originals (its
default) or, in the dequantized backward of "The 4-bitter Lesson"
("Improving Gradient Stability"), the bf16 values of the exact quantized
tensors the forward used; this module takes whichever operands it is given.

Notation (routed row r of expert e = E(r), token t = row_src[r], router
weight p_r; gate g = C[r, :I], up u = C[r, I:], the forward's FC1 output):
    D[r]      = silu(g) * u * p_r                 (the forward's FC2 input)
    y[t]      = sum over t's rows r of D[r] @ W2[E(r)]^T
Given dy [T, H]:
    dYr[r]    = dy[t]                             (the combine is a sum)
    dD[r]     = dYr[r] @ W2[E(r)]                 dgrad of FC2
    dW2[e]    = sum_{r in e} dYr[r]^T  Dop[r]     wgrad of FC2 (Dop: D as a bf16 operand)
    dg        = dD * u * p * silu'(g),  du = dD * silu(g) * p
    dp[t, j]  = sum_i dD[r, i] * silu(g_i) * u_i  (the entry's router weight)
    dC[r]     = [dg | du]
    dXr[r]    = dC[r] @ W1[E(r)]                  dgrad of FC1
    dW1[e]    = sum_{r in e} dC[r]^T  X[t]        wgrad of FC1
    dx[t]     = sum over t's rows r of dXr[r]
with silu(g) = g s, s = 1 / (1 + e^-g), silu'(g) = s (1 + g (1 - s)).

Each step is written out on its own so a test can replay it on the GPU's
inputs: float64 numpy, matrix products via numpy's matmul (a library
primitive), no blocking or reordering beyond the definitions.
"""
from __future__ import annotations

import numpy as np

from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32


def bf16(u16) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values."""
    return bf16_bits_to_f32(np.asarray(u16, np.uint16)).astype(np.float64)


def _groups(offsets):
    off = np.asarray(offsets, np.int64)
    return [(e, int(off[e]), int(off[e + 1])) for e in range(off.size - 1)]


def gather_rows(dy, row_src, rows):
    """dYr[r] = dy[row_src[r]] for r < rows (padding rows, row_src < 0: zero)."""
    dy = np.asarray(dy, np.float64)
    out = np.zeros((rows, dy.shape[1]), np.float64)
    src = np.asarray(row_src[:rows])
    ok = src >= 0
    out[ok] = dy[src[ok]]
    return out


def grouped_dgrad(a, w, offsets):
    """out[r] = a[r] @ w[e] for the rows r of group e (w: [G, K, N], the
    forward's weight matrix, whose rows the gradient flows back through)."""
    a = np.asarray(a, np.float64)
    w = np.asarray(w, np.float64)
    out = np.zeros((a.shape[0], w.shape[2]), np.float64)
    babs = np.zeros_like(out)
    for e, r0, r1 in _groups(offsets):
        if r1 > r0:
            out[r0:r1] = a[r0:r1] @ w[e]
            babs[r0:r1] = np.abs(a[r0:r1]) @ np.abs(w[e])
    return out, babs


def grouped_wgrad(a, b, offsets):
    """out[e] = sum over the rows r of group e of outer(a[r], b[r])
    ([G, Na, Nb]); bound: the same sum of |a| |b|."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    G = len(offsets) - 1
    out = np.zeros((G, a.shape[1], b.shape[1]), np.float64)
    babs = np.zeros_like(out)
    for e, r0, r1 in _groups(offsets):
        if r1 > r0:
            out[e] = a[r0:r1].T @ b[r0:r1]
            babs[e] = np.abs(a[r0:r1]).T @ np.abs(b[r0:r1])
    return out, babs


def swiglu_backward(dD, C, prob):
    """(dC [rows, 2I], dp [rows]) from dD [rows, I], the FC1 output C and the
    rows' router weights."""
    dD = np.asarray(dD, np.float64)
    C = np.asarray(C, np.float64)
    p = np.asarray(prob, np.float64)[:, None]
    I = dD.shape[1]
    g, u = C[:, :I], C[:, I:]
    s = 1.0 / (1.0 + np.exp(-g))
    silu = g * s
    dsilu = s * (1.0 + g * (1.0 - s))
    dg = dD * u * p * dsilu
    du = dD * silu * p
    dp = np.sum(dD * silu * u, axis=1)
    return np.concatenate([dg, du], axis=1), dp


def combine_rows(rows, dst_row):
    """dx[t] = sum_j rows[dst_row[t, j]] (entries with dst_row < 0 add nothing)."""
    rows = np.asarray(rows, np.float64)
    T, k = dst_row.shape
    out = np.zeros((T, rows.shape[1]), np.float64)
    for j in range(k):
        ok = dst_row[:, j] >= 0
        out[ok] += rows[dst_row[ok, j]]
    return out


def entry_grad(dp_rows, dst_row):
    """dprob[t, j] = dp of the entry's row (0 for entries not routed)."""
    dp_rows = np.asarray(dp_rows, np.float64)
    out = np.zeros(dst_row.shape, np.float64)
    ok = dst_row >= 0
    out[ok] = dp_rows[dst_row[ok]]
    return out


def moe_backward(dy, x, C, D, row_src, row_prob, offsets, dst_row, W1, W2):
    """The whole backward from the layer's operands (float64 values: x [T, H],
    C [rows, 2I], D [rows, I], W1 [G, 2I, H], W2 [G, H, I]; rows =
    offsets[-1]).  Returns dict(dx, dW1, dW2, dprob) and the intermediates
    (dYr, dD, dC, dXr)."""
    rows = int(np.asarray(offsets)[-1])
    dYr = gather_rows(dy, row_src, rows)
    dD, _ = grouped_dgrad(dYr, W2, offsets)
    dW2, _ = grouped_wgrad(dYr, D[:rows], offsets)
    dC, dp = swiglu_backward(dD, C[:rows], row_prob[:rows])
    dXr, _ = grouped_dgrad(dC, W1, offsets)
    Xr = gather_rows(x, row_src, rows)
    dW1, _ = grouped_wgrad(dC, Xr, offsets)
    return dict(dx=combine_rows(dXr, dst_row), dW1=dW1, dW2=dW2,
                dprob=entry_grad(dp, dst_row)), dict(dYr=dYr, dD=dD, dC=dC, dXr=dXr)
