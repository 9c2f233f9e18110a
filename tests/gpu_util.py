"""Helpers for the GPU parity tests: host<->device transfer of bf16 bit
patterns, the oracle's NVFP4 weight quantization, decoding for error bounds,
and the GEMM tolerance of the contract:
    |gpu - oracle| <= 2^-10 * sum_k |a_k b_k| + 1e-6."""
import functools
import sys

import numpy as np
import torch

from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32, make_moe
from oracle import oracle as O

GEMM_REL = 2.0 ** -10
GEMM_ABS = 1e-6


def say(*a):
    """Names the case before a GPU step (flushed, so it survives a crash)."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def dev_bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return host_bf16(t)
    return t.contiguous().cpu().numpy()


def oracle_weights(w_bf16: np.ndarray):
    """Oracle NVFP4 of expert weights [G, N, K] with one outer scale per expert."""
    G, N, K = w_bf16.shape
    c, s, g = O.quantize(w_bf16.reshape(G * N, K), domain=1,
                         group_offsets=np.arange(G + 1, dtype=np.int32) * N)
    return c.reshape(G, N, K // 2), s.reshape(G, N, K // 16), g


def gemm_tol(bound: np.ndarray) -> np.ndarray:
    return GEMM_REL * bound + GEMM_ABS


def assert_gemm_close(gpu: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str):
    err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    tol = gemm_tol(bound)
    bad = np.flatnonzero(~(err <= tol))
    assert bad.size == 0, (f"{what}: {bad.size} of {err.size} outside tolerance; first "
                           f"idx {bad[:4]}, gpu {gpu.reshape(-1)[bad[:4]]}, ref "
                           f"{ref.reshape(-1)[bad[:4]]}, tol {tol.reshape(-1)[bad[:4]]}")


@functools.lru_cache(maxsize=None)
def moe_case(wid, with_weights=True):
    """Workload + oracle-quantized weights (cached for the session)."""
    w = make_moe(wid, with_weights=with_weights)
    W1 = W2 = None
    if with_weights:
        W1 = oracle_weights(w.w1)
        W2 = oracle_weights(w.w2)
    return w, W1, W2


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (2^(e-7) for normal v)."""
    v = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return 2.0 ** (e - 7)
