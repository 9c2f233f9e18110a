"""Seeded synthetic inputs for the NVFP4 W4A4 MoE expert path.

This module holds input synthesis only: random activations, router outputs and
bf16 weights with the shapes and distributions of the measured workloads.  It
contains none of the quantization, permutation or GEMM arithmetic, and both
the HIP path's tests and the oracle consume what it produces.

The shapes follow the Qwen3-30B-A3B expert layer that the miniTE Technical
Report times (§6.1: hidden 2048, 128 experts, top-8, expert intermediate 768,
sequence length 4096-8192), whose real data (DAPO text, trained weights) is
not available here; seeded Gaussian / Student-t activations, N(0, 0.02)
weights and router logits with a Zipf-like per-expert bias stand in for it.

Generation order per workload is fixed: logits -> x -> outlier channels ->
zero rows -> W1 -> W2, from numpy PCG64(1000 + workload id).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["MoeWorkload", "DenseWorkload", "MOE_WORKLOADS", "make_moe", "make_dense",
           "to_bf16_bits", "bf16_bits_to_f32", "route_topk", "random_bf16"]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even (finite input)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bits = bits + 0x7FFF + ((bits >> 16) & 1)
    return (bits >> 16).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def random_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def route_topk(logits: np.ndarray, topk: int):
    """Router stand-in: softmax over experts (fp32), top-k with ties to the lower
    expert id, probabilities renormalised to sum to one over the k picks."""
    z = logits.astype(np.float32)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :topk]
    pk = np.take_along_axis(p, order, axis=1)
    pk = pk / pk.sum(axis=1, keepdims=True)
    return order.astype(np.int32), pk.astype(np.float32)


@dataclass
class MoeWorkload:
    name: str
    wid: int
    tokens: int
    hidden: int
    inter: int
    experts: int
    topk: int
    x: np.ndarray            # bf16 bits [T, H]
    topk_idx: np.ndarray     # int32 [T, k]
    topk_prob: np.ndarray    # f32 [T, k]
    w1: np.ndarray | None    # bf16 bits [E, 2I, H]  (gate | up)
    w2: np.ndarray | None    # bf16 bits [E, H, I]
    meta: dict = field(default_factory=dict)

    @property
    def routed_rows(self) -> int:
        return int((self.topk_idx >= 0).sum())

    def flops(self) -> float:
        """Algorithmic FLOPs of FC1 + FC2 over the routed rows (padding excluded)."""
        r = self.routed_rows
        return 2.0 * r * (2 * self.inter) * self.hidden + 2.0 * r * self.hidden * self.inter


@dataclass
class DenseWorkload:
    name: str
    wid: int
    tokens: int
    # list of (name, x bf16 [T, K], w bf16 [N, K])
    projections: list


# id: (name, tokens, hidden, inter, experts, topk, zipf_s, activation kind)
MOE_WORKLOADS = {
    0: ("tiny_moe", 256, 256, 128, 4, 2, 0.0, "normal"),
    2: ("qwen3_30b_a3b_moe_t8192", 8192, 2048, 768, 128, 8, 1.1, "normal"),
    3: ("decode_moe_t256", 256, 2048, 768, 128, 8, 0.0, "normal"),
    4: ("long_heavytail_moe_t32768", 32768, 2048, 768, 128, 8, 1.3, "student_t3"),
}
DENSE_WORKLOAD_ID = 1
MOE_NAME_TO_ID = {v[0]: k for k, v in MOE_WORKLOADS.items()}


def make_moe(wid, with_weights: bool = True, tokens: int | None = None) -> MoeWorkload:
    """Builds MoE workload `wid` (int id or name).  `tokens` truncates the token
    count (same distributions, for bounded samples)."""
    if isinstance(wid, str):
        wid = MOE_NAME_TO_ID[wid]
    name, T, H, I, E, k, zipf_s, act = MOE_WORKLOADS[wid]
    rng = np.random.Generator(np.random.PCG64(1000 + wid))
    # router logits N(0,1) plus a Zipf-like per-expert bias -s*ln(e+1)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if zipf_s:
        logits += (-zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
    idx, prob = route_topk(logits, k)
    meta = {"zipf_s": zipf_s, "activations": act}
    if act == "normal":
        xf = rng.standard_normal((T, H), dtype=np.float32)
    else:
        xf = rng.standard_t(3, size=(T, H)).astype(np.float32)
        # 0.1% of channels scaled x100
        n_out = max(1, int(round(0.001 * H)))
        ch = rng.choice(H, size=n_out, replace=False)
        xf[:, ch] *= np.float32(100.0)
        meta["outlier_channels"] = sorted(int(c) for c in ch)
        # 0.5% of rows all zero (half +0.0, half -0.0): the amax = 0 path
        n_zero = max(2, int(round(0.005 * T)))
        zr = rng.choice(T, size=n_zero, replace=False)
        xf[zr[: n_zero // 2]] = np.float32(0.0)
        xf[zr[n_zero // 2:]] = np.float32(-0.0)
        meta["zero_rows"] = sorted(int(r) for r in zr)
    x = to_bf16_bits(xf)
    w1 = w2 = None
    if with_weights:
        w1 = random_bf16(rng, (E, 2 * I, H), 0.02)
        w2 = random_bf16(rng, (E, H, I), 0.02)
    if tokens is not None and tokens < T:
        x, idx, prob, T = x[:tokens].copy(), idx[:tokens].copy(), prob[:tokens].copy(), tokens
    counts = np.bincount(idx.reshape(-1), minlength=E)
    meta["active_experts"] = int((counts > 0).sum())
    meta["cv_rows_per_expert"] = float(counts.std() / max(counts.mean(), 1e-9))
    return MoeWorkload(name, wid, T, H, I, E, k, x, idx, prob, w1, w2, meta)


def make_dense(tokens: int | None = None) -> DenseWorkload:
    """Dense W4A4 attention projections of a Qwen3-30B-A3B-like layer:
    QKV (K=2048, N=5120 = 32 q heads + 2x4 kv heads of dim 128) and O-proj
    (K=4096, N=2048); inputs N(0,1) with 0.1% of channels x50, weights N(0,0.02)."""
    wid = DENSE_WORKLOAD_ID
    rng = np.random.Generator(np.random.PCG64(1000 + wid))
    T = 8192
    projs = []
    for pname, K, N in (("qkv", 2048, 5120), ("o_proj", 4096, 2048)):
        xf = rng.standard_normal((T, K), dtype=np.float32)
        n_out = max(1, int(round(0.001 * K)))
        ch = rng.choice(K, size=n_out, replace=False)
        xf[:, ch] *= np.float32(50.0)
        w = random_bf16(rng, (N, K), 0.02)
        x = to_bf16_bits(xf)
        if tokens is not None and tokens < T:
            x = x[:tokens].copy()
        projs.append((pname, x, w))
    return DenseWorkload("dense_attn_proj_t8192", wid, tokens or T, projs)
