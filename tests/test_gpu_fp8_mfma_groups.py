"""Characterisation of the gfx950 fp8 matrix core's summation, on normal
in-bounds inputs through the C ABI (float32 output, no scales, so the output
is the fp32 accumulator itself).

The operands are OCP fp8 e4m3 and the accumulation is fp32 ("[Kernel] Add
w8a8 CUTLASS kernels", PR description), in an order the pages leave open. The
matrix core adds each group of 8 consecutive products after aligning them to
the largest one, keeping 13 fraction bits below its leading bit: a product
2^-13 below the group's largest is kept, one 2^-14 below is dropped, a small
product alone in its group is exact, and the add of group sums into the fp32
accumulator rounds as fp32 does. These cases pin that reading, on which the
fp8 output tolerance of the parity tests rests (FP8_GROUP_REL in
tests/gpu_util.py, derived on the CPU in tests/test_fp8_group_model.py).
Both MFMA shapes the library uses are covered: 16x16x128 (decode kernel,
M <= 64) and 32x32x64 (tile kernel, M > 64).
"""
import numpy as np
import pytest
import torch

import int8_scaled_gemm_amd as w8
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu

ONE, P6, P7 = 0x38, 0x08, 0x04   # e4m3 codes of 1.0, 2^-6 (least normal), 2^-7 (subnormal)
K = 128

# (a codes by k, b codes by k, expected fp32 sum)
CASES = [
    # 1 + 2^-13 in one group: kept
    ({0: ONE, 1: P7}, {0: ONE, 1: P6}, 1.0 + 2.0 ** -13),
    # 1 + 2^-14 in one group: dropped
    ({0: ONE, 1: P7}, {0: ONE, 1: P7}, 1.0),
    # the same two products in different groups of 8: both kept
    ({0: ONE, 8: P7}, {0: ONE, 8: P7}, 1.0 + 2.0 ** -14),
    # 2^-14 alone: exact
    ({5: P7}, {5: P7}, 2.0 ** -14),
    # 2^-14 below the largest at the group's far end (k = 7 of k = 0..7)
    ({0: ONE, 7: P7}, {0: ONE, 7: P7}, 1.0),
    # group boundary at k = 64 (the second half of a 128-deep slice)
    ({63: ONE, 64: P7}, {63: ONE, 64: P7}, 1.0 + 2.0 ** -14),
]


def _operands(M):
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((len(CASES), K), np.uint8)
    for i, (ca, cb, _) in enumerate(CASES):
        for k, c in ca.items():
            a[i, k] = c
        for k, c in cb.items():
            b[i, k] = c
    return a, b


@pytest.mark.parametrize("M", [len(CASES), 96])  # decode kernel, then the tile kernel
def test_fp8_group_alignment(M):
    kernel = w8.w8a8_scaled_mm_kernel(M, len(CASES), K)
    print(f"fp8 MFMA groups M={M} kernel {kernel}", flush=True)
    a, b = _operands(M)
    ad = torch.from_numpy(a).to(DEV).view(torch.float8_e4m3fn)
    bd = torch.from_numpy(b).to(DEV).view(torch.float8_e4m3fn)
    out = w8.w8a8_scaled_mm(ad, bd.t(), None, None, torch.float32)
    torch.cuda.synchronize()
    d = out.cpu().numpy().astype(np.float64)
    for i, (_, _, want) in enumerate(CASES):
        assert d[i, i] == want, (i, d[i, i], want)
    assert (d[len(CASES):] == 0).all()
