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


def _row_slice(A, r0, r1):
    return tuple(np.ascontiguousarray(a[r0:r1]) for a in A)


def oracle_gemm_chunks(A, W, offs, chunk_rows=None):
    """The oracle grouped GEMM with its bound over rows [offs[0], offs[-1]),
    yielded as (r0, r1, ref, bound) slices of at most `chunk_rows` rows, so
    the host holds one slice of the fp32 result and its fp64 bound at a time.
    A slice is the same definition on the rows it covers: its group offsets
    are the full ones clipped to [r0, r1)."""
    offs = np.asarray(offs, np.int64)
    n = W[0].shape[1]
    if chunk_rows is None:
        chunk_rows = max(1024, (256 << 20) // (12 * n))      # ~256 MB of result + bound
    start, end = int(offs[0]), int(offs[-1])
    for r0 in range(start, end, chunk_rows):
        r1 = min(end, r0 + chunk_rows)
        lo = (np.clip(offs, r0, r1) - r0).astype(np.int32)
        ref, bound = O.grouped_gemm(*_row_slice(A, r0, r1), *W, lo, with_bound=True)
        yield r0, r1, ref, bound


def oracle_single_pass_chunks(A2, gs, tile, W, offs, chunk_rows=None):
    """The oracle's single-pass FC2 (O12b) with its bound over rows
    [offs[0], offs[-1]), in row slices like oracle_gemm_chunks."""
    offs = np.asarray(offs, np.int64)
    n = W[0].shape[1]
    if chunk_rows is None:
        chunk_rows = max(1024, (256 << 20) // (12 * n))
    start, end = int(offs[0]), int(offs[-1])
    for r0 in range(start, end, chunk_rows):
        r1 = min(end, r0 + chunk_rows)
        lo = (np.clip(offs, r0, r1) - r0).astype(np.int32)
        c, sc = _row_slice(A2, r0, r1)
        ref, bound = O.single_pass_gemm(c, sc, np.ascontiguousarray(gs[r0:r1]), tile, *W, lo,
                                        with_bound=True)
        yield r0, r1, ref, bound


def assert_gemm_full(gpu: np.ndarray, A, W, offs, what: str, bf16_out: bool = False,
                     chunks=None):
    """Every output element of the rows [offs[0], offs[-1]) against the oracle:
    fp32 output within 2^-10 * sum|a_k b_k| + 1e-6; bf16 output (uint16 bit
    patterns) the round-to-nearest-even of a value within that tolerance,
    i.e. within it plus half a bf16 ulp of the oracle value.  `chunks` may be
    a list of precomputed oracle_gemm_chunks slices of the same problem.
    Returns the number of elements compared."""
    count = 0
    for r0, r1, ref, bound in (chunks if chunks is not None else oracle_gemm_chunks(A, W, offs)):
        g = gpu[r0:r1]
        if bf16_out:
            got = bf16_bits_to_f32(g).astype(np.float64)
            err = np.abs(got - ref.astype(np.float64))
            tol = gemm_tol(bound) + bf16_ulp(ref) * 0.5 * 1.0001
            bad = np.flatnonzero(~(err <= tol))
            assert bad.size == 0, (f"{what} rows [{r0},{r1}): {bad.size} of {err.size} "
                                   f"outside tolerance; first flat idx {bad[:4]}")
        else:
            assert_gemm_close(g, ref, bound, f"{what} rows [{r0},{r1})")
        count += ref.size
        say(f"{what}: rows [{r0}, {r1}) of [{int(offs[0])}, {int(offs[-1])}) within tolerance")
    return count


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


@functools.lru_cache(maxsize=None)
def moe_permute_ref(wid):
    """The oracle's routing + quantize-scatter of workload `wid` (cached)."""
    w, _, _ = moe_case(wid)
    return O.moe_permute(w.x, w.topk_idx, w.topk_prob, w.experts)


@functools.lru_cache(maxsize=None)
def fc1_oracle_chunks(wid):
    """The oracle FC1 (pre-activation C and its bound) of workload `wid` on
    the oracle's own A1, as a list of row slices.  Several tests compare GPU
    FC1 outputs on A1 bit-identical to the oracle's against it; the slices
    are computed once per session."""
    w, W1, _ = moe_case(wid)
    p = moe_permute_ref(wid)
    A1 = (p["codes"], p["scales"], p["gscale"])
    return list(oracle_gemm_chunks(A1, W1, p["offsets"]))

