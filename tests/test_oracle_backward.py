"""Pins of the backward-pass oracle (oracle/backward.py).

The straight-through backward differentiates the layer as if its operands
were the BF16 ones.  With C and D the exact products of those operands, it
is then the exact gradient of a plain float64 function:
    y[t] = sum over the entries (t, j) of silu(g) * u * p_tj @ W2[e]^T,
    [g | u] = x[t] @ W1[e]^T.
torch's autograd (an independent differentiation of that function) fixes
dx, dW1, dW2 and the router-weight gradients.  Planted mistakes in a copy of
the oracle (wrong SwiGLU derivative, a dropped router weight, transposed
weights, a wgrad over the wrong operand, gate and up swapped, a skipped
entry in the combine) are each caught."""
import inspect
import types

import numpy as np
import pytest
import torch

from oracle import backward as B
from oracle import oracle as O


def _case(seed, T=24, H=32, I=16, E=3, k=2, align=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    W1 = rng.standard_normal((E, 2 * I, H)) * 0.3
    W2 = rng.standard_normal((E, H, I)) * 0.3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[3, 1] = -1                              # an entry not routed
    prob = rng.random((T, k)).astype(np.float32)
    dy = rng.standard_normal((T, H))
    off, dst, src, rprob = O.route(idx, prob, E, align)
    return x, W1, W2, idx, prob, dy, off, dst, src, rprob


def _autograd(x, W1, W2, idx, prob, dy):
    X = torch.tensor(x, requires_grad=True)
    A = torch.tensor(W1, requires_grad=True)
    Bw = torch.tensor(W2, requires_grad=True)
    P = torch.tensor(prob.astype(np.float64), requires_grad=True)
    T, k = idx.shape
    I = W2.shape[2]
    y = torch.zeros_like(X)
    rows = []
    for t in range(T):
        acc = torch.zeros(X.shape[1], dtype=torch.float64)
        for j in range(k):
            e = int(idx[t, j])
            if e < 0:
                continue
            c = A[e] @ X[t]
            g, u = c[:I], c[I:]
            acc = acc + Bw[e] @ (torch.nn.functional.silu(g) * u * P[t, j])
        rows.append(acc)
    y = torch.stack(rows)
    (y * torch.tensor(dy)).sum().backward()
    return X.grad.numpy(), A.grad.numpy(), Bw.grad.numpy(), P.grad.numpy()


def _oracle(mod, x, W1, W2, prob, dy, off, dst, src, rprob):
    rows = int(off[-1])
    I = W2.shape[2]
    Xr = mod.gather_rows(x, src, rows)
    C = np.zeros((rows, 2 * I))
    D = np.zeros((rows, I))
    for e in range(len(off) - 1):
        r0, r1 = int(off[e]), int(off[e + 1])
        C[r0:r1] = Xr[r0:r1] @ W1[e].T
        g, u = C[r0:r1, :I], C[r0:r1, I:]
        D[r0:r1] = g / (1 + np.exp(-g)) * u * rprob[r0:r1, None]
    out, _ = mod.moe_backward(dy, x, C, D, src, rprob, off, dst, W1, W2)
    return out


def _check(out, ref):
    dx, dW1, dW2, dp = ref
    for got, want in ((out["dx"], dx), (out["dW1"], dW1), (out["dW2"], dW2), (out["dprob"], dp)):
        assert got.shape == want.shape
        assert np.allclose(got, want, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", [1, 2])
def test_backward_matches_torch_autograd(seed):
    x, W1, W2, idx, prob, dy, off, dst, src, rprob = _case(seed)
    ref = _autograd(x, W1, W2, idx, prob, dy)
    _check(_oracle(B, x, W1, W2, prob, dy, off, dst, src, rprob), ref)


def test_padding_rows_and_empty_experts_give_nothing():
    x, W1, W2, idx, prob, dy, off, dst, src, rprob = _case(3, E=5)
    idx[:, :] = np.where(idx == 4, 0, idx)     # expert 4 empty
    off, dst, src, rprob = O.route(idx, prob, 5, 8)
    out = _oracle(B, x, W1, np.concatenate([W2[:3], W2[:2]]), prob, dy, off, dst, src, rprob)
    assert np.all(out["dW1"][4] == 0) and np.all(out["dW2"][4] == 0)
    assert out["dprob"][3, 1] == 0


MUTANTS = [
    ("silu_derivative_is_sigmoid", "dsilu = s * (1.0 + g * (1.0 - s))", "dsilu = s"),
    ("du_drops_router_weight", "du = dD * silu * p", "du = dD * silu"),
    ("dp_drops_up", "dp = np.sum(dD * silu * u, axis=1)", "dp = np.sum(dD * silu, axis=1)"),
    ("dgrad_transposed_weight", "out[r0:r1] = a[r0:r1] @ w[e]", "out[r0:r1] = a[r0:r1] @ w[e].T[:w.shape[1], :w.shape[2]] if w.shape[1] == w.shape[2] else a[r0:r1] @ w[e][::-1]"),
    ("wgrad_swapped_operands", "out[e] = a[r0:r1].T @ b[r0:r1]", "out[e] = (b[r0:r1].T @ a[r0:r1]).T[::-1]"),
    ("gate_up_swapped", "g, u = C[:, :I], C[:, I:]", "u, g = C[:, :I], C[:, I:]"),
    ("combine_skips_slot_0", "for j in range(k):\n        ok = dst_row[:, j] >= 0\n        out[ok] += rows[dst_row[ok, j]]",
     "for j in range(1, k):\n        ok = dst_row[:, j] >= 0\n        out[ok] += rows[dst_row[ok, j]]"),
]


@pytest.mark.parametrize("name,orig,mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, orig, mutant):
    src_text = inspect.getsource(B)
    assert src_text.count(orig) == 1, name
    mod = types.ModuleType("backward_mutant")
    exec(compile(src_text.replace(orig, mutant), "backward_mutant", "exec"), mod.__dict__)
    x, W1, W2, idx, prob, dy, off, dst, src, rprob = _case(7)
    ref = _autograd(x, W1, W2, idx, prob, dy)
    with pytest.raises(AssertionError):
        _check(_oracle(mod, x, W1, W2, prob, dy, off, dst, src, rprob), ref)
