"""GPU parity of moe_combine (through the C ABI).  The oracle sums a token's
k expert rows in binary64 and rounds once to bf16; the kernel accumulates in
binary32 in j order, so the two agree within the binary32 accumulation
bound plus one bf16 ulp.  The kernel's own arithmetic (binary32 adds in j
order, then round-to-nearest-even to bf16) is also checked bit for bit
against that recurrence written out with numpy.  Dropped entries
(dst_row < 0) add nothing."""
import numpy as np
import pytest
import torch

from gpu_util import dev, host, say
from gpu_util import bf16_ulp
from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32, random_bf16, to_bf16_bits
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("topk", [1, 8, 12, 20])
def test_combine_bit_exact(rows_dtype, topk):
    from nvfp4_w4a4_quantized_amd.ops import moe_combine
    rng = np.random.default_rng(topk * 7 + len(rows_dtype))
    T, H = 300, 2048 if topk <= 8 else 512
    R = T * topk + 37
    dst = rng.permutation(T * topk).reshape(T, topk).astype(np.int32)
    dst[rng.random((T, topk)) < 0.1] = -1              # dropped entries
    dst[5, :] = -1                                     # a token with no rows
    if rows_dtype == "bf16":
        yb = random_bf16(rng, (R, H), 3.0)
        yb[dst[7, 0]] = 0x8000                         # -0.0 row
        rows_t = torch.from_numpy(yb.view(np.int16)).cuda().view(torch.bfloat16)
        yr = bf16_bits_to_f32(yb)
    else:
        yr = (rng.standard_normal((R, H)) * 3).astype(np.float32)
        yr[dst[7, 0]] = -0.0
        rows_t = dev(yr)
    say("moe_combine", rows_dtype, "topk", topk, "H", H)
    y = moe_combine(rows_t, dev(dst))
    torch.cuda.synchronize()
    got = host(y)
    # the oracle: within the binary32 accumulation bound and one bf16 ulp
    ref = bf16_bits_to_f32(O.combine(yr, dst)).astype(np.float64)
    absum = np.zeros((T, H))
    s32 = np.zeros((T, H), np.float32)
    for j in range(topk):
        ok = dst[:, j] >= 0
        absum[ok] += np.abs(yr[dst[ok, j]])
        s32[ok] += yr[dst[ok, j]]                      # binary32, j order
    gv = bf16_bits_to_f32(got).astype(np.float64)
    tol = absum * topk * 2.0 ** -24 + bf16_ulp(ref) * 1.0001 + 1e-30
    assert np.all(np.abs(gv - ref) <= tol), "outside the accumulation bound"
    # the kernel's recurrence, bit for bit
    exp = to_bf16_bits(s32)
    assert np.array_equal(got, exp), f"{int((got != exp).sum())} elements differ from the j-order sum"
