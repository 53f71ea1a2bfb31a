"""Pins for the oracle's scaled matrix multiply.

D = a_scale (x) b_scale * (A_q . B_q) ("[Kernel] Add w8a8 CUTLASS kernels",
PR description list) is checked against exact rational brute force (integer
matmul of the codes, exact scale products, nearest bf16/fp16 by exhaustive
comparison), closed forms and invariants that a dropped term, a wrong index
or a transposed operand would break.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from tests.exact import e4m3_int512, nearest_bf16, nearest_fp16

NEAREST = {"bf16": nearest_bf16, "fp16": nearest_fp16}


def _exact_acc(a, b, qtype):
    """Exact accumulator as (integer numerator, power-of-two denominator)."""
    if qtype == "int8":
        ai = a.view(np.int8).astype(np.int64)
        bi = b.view(np.int8).astype(np.int64)
        return ai @ bi.T, 1
    return e4m3_int512(a) @ e4m3_int512(b).T, 2 ** 18


def _brute(a, b, qtype, sa, sb, otype):
    acc, den = _exact_acc(a, b, qtype)
    M, N = acc.shape
    sa = np.broadcast_to(np.asarray(sa, np.float32).reshape(-1), (M,))
    sb = np.broadcast_to(np.asarray(sb, np.float32).reshape(-1), (N,))
    out = np.empty((M, N), np.uint16)
    for m in range(M):
        fa = Fraction(float(sa[m]))
        for n in range(N):
            out[m, n] = NEAREST[otype](Fraction(int(acc[m, n]), den) * fa * Fraction(float(sb[n])))
    return out


def _codes(shape, qtype, seed):
    return workloads.random_codes(shape, qtype, seed=seed).numpy()


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("otype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K", [(16, 64, 128), (3, 5, 48), (1, 17, 16), (9, 33, 272)])
def test_scaled_mm_brute_force(orc, qtype, otype, M, N, K):
    a = _codes((M, K), qtype, 1)
    b = _codes((N, K), qtype, 2)
    rng = np.random.default_rng(M * 1000 + N)
    # per-token activation scales, per-channel weight scales, of the sizes
    # absmax/448 or absmax/127 produce for N(0,1) and N(0,0.02) data
    sa = (rng.uniform(0.5, 2.0, M) / (448 if qtype == "fp8" else 127) * 4).astype(np.float32)
    sb = (rng.uniform(0.5, 2.0, N) * 0.08 / (448 if qtype == "fp8" else 127)).astype(np.float32)
    if otype == "fp16" and qtype == "int8":
        sb *= 4  # keep fp16 results in the normal range
    got = orc.scaled_mm(a, b, qtype, sa, sb, otype)
    assert np.array_equal(got, _brute(a, b, qtype, sa, sb, otype))
    # per-tensor on both sides
    got1 = orc.scaled_mm(a, b, qtype, sa[:1], sb[:1], otype)
    assert np.array_equal(got1, _brute(a, b, qtype, sa[:1], sb[:1], otype))


def test_tiny_int8_case_brute_force(orc):
    """The tiny int8 case end to end: per-tensor int8 of A and W, int32 acc, bf16 out."""
    a, w = workloads.tiny_int8_inputs()
    ab, wb = workloads.as_u16(a), workloads.as_u16(w)
    qa, sa = orc.quant_per_tensor(ab, "int8", dynamic=True, xtype="bf16")
    qw, sw = orc.quant_per_tensor(wb, "int8", dynamic=True, xtype="bf16")
    # the scales are absmax/127 of the bf16 data (absmax is exact)
    assert sa == np.float32(np.abs(orc.bf16_bits_to_f64(ab)).max()) / np.float32(127)
    assert sw == np.float32(np.abs(orc.bf16_bits_to_f64(wb)).max()) / np.float32(127)
    got = orc.scaled_mm(qa, qw, "int8", [sa], [sw], "bf16")
    assert np.array_equal(got, _brute(qa, qw, "int8", [sa], [sw], "bf16"))
    raw = orc.scaled_mm(qa, qw, "int8", None, None, "i32")
    assert np.array_equal(raw, qa.view(np.int8).astype(np.int64) @ qw.view(np.int8).astype(np.int64).T)


def test_raw_accumulators(orc):
    a = _codes((7, 320), "fp8", 3)
    b = _codes((11, 320), "fp8", 4)
    acc, den = _exact_acc(a, b, "fp8")
    f32 = orc.scaled_mm(a, b, "fp8", None, None, "f32")
    assert np.array_equal(f32, np.array([[np.float32(float(Fraction(int(x), den))) for x in r] for r in acc]))
    ai = _codes((7, 320), "int8", 5)
    bi = _codes((11, 320), "int8", 6)
    assert np.array_equal(orc.scaled_mm(ai, bi, "int8", None, None, "i32"), _exact_acc(ai, bi, "int8")[0])


def test_int8_extreme_accumulator(orc):
    """All-127 times all -127 over the longest K in the workloads (28672):
    acc = -127*127*28672 = -462,450,688, inside int32."""
    K = 28672
    a = np.full((1, K), 127, np.int8).view(np.uint8)
    b = np.full((2, K), -127, np.int8).view(np.uint8)
    raw = orc.scaled_mm(a, b, "int8", None, None, "i32")
    assert raw.tolist() == [[-462450688, -462450688]]


def test_fp8_extreme_accumulator_is_exact(orc):
    """All 448 times all -448 over K = 28672: -448^2 * 28672 exactly, and the
    smallest subnormal squared (2^-18) survives next to it."""
    K = 28672
    a = np.full((1, K), 0x7E, np.uint8)
    b = np.full((1, K), 0xFE, np.uint8)
    a[0, 0] = 0x01
    b[0, 0] = 0x01
    f = orc.scaled_mm(a, b, "fp8", None, None, "f32")
    want = np.float32(-448.0 * 448.0 * (K - 1) + 2.0 ** -18)
    assert f[0, 0] == want


def test_per_tensor_equals_per_token_with_equal_scales(orc):
    a = _codes((13, 128), "fp8", 8)
    b = _codes((40, 128), "fp8", 9)
    s = np.float32(0.0123)
    t = np.float32(0.00041)
    d1 = orc.scaled_mm(a, b, "fp8", [s], [t], "bf16")
    d2 = orc.scaled_mm(a, b, "fp8", np.full(13, s), np.full(40, t), "bf16")
    assert np.array_equal(d1, d2)


def test_power_of_two_scale_is_exact(orc):
    a = _codes((6, 256), "int8", 10)
    b = _codes((24, 256), "int8", 11)
    sa = np.linspace(0.001, 0.01, 6).astype(np.float32)
    sb = np.linspace(0.0001, 0.0003, 24).astype(np.float32)
    d1 = orc.bf16_bits_to_f64(orc.scaled_mm(a, b, "int8", sa, sb, "bf16"))
    d2 = orc.bf16_bits_to_f64(orc.scaled_mm(a, b, "int8", sa * 4, sb, "bf16"))
    assert np.array_equal(d1 * 4, d2)


def test_identity_weight_reproduces_scaled_activation(orc):
    K = 64
    a = _codes((5, K), "fp8", 12)
    b = np.zeros((K, K), np.uint8)
    np.fill_diagonal(b, 0x38)  # e4m3 1.0
    sa = np.float32(0.25)
    sb = np.float32(3.0)
    d = orc.scaled_mm(a, b, "fp8", [sa], [sb], "f32")
    want = (e4m3_int512(a) / 512.0 * 0.75).astype(np.float32)
    assert np.array_equal(d, want)


def test_transpose_symmetry(orc):
    """D(A, B)^T with swapped scales equals D(B, A): catches a transposed operand."""
    a = _codes((9, 192), "fp8", 13)
    b = _codes((21, 192), "fp8", 14)
    sa = np.linspace(0.01, 0.02, 9).astype(np.float32)
    sb = np.linspace(0.001, 0.002, 21).astype(np.float32)
    d = orc.scaled_mm(a, b, "fp8", sa, sb, "bf16")
    dt = orc.scaled_mm(b, a, "fp8", sb, sa, "bf16")
    assert np.array_equal(d.T, dt)
    assert not np.array_equal(d[:, :9], d[:, :9].T)  # the data is not symmetric


def test_rows_variant_matches_full(orc):
    a = _codes((37, 128), "int8", 15)
    b = _codes((50, 128), "int8", 16)
    sa = np.linspace(0.01, 0.02, 37).astype(np.float32)
    sb = np.linspace(0.001, 0.002, 50).astype(np.float32)
    full = orc.scaled_mm(a, b, "int8", sa, sb, "bf16")
    rows = [0, 5, 36, 17]
    assert np.array_equal(orc.scaled_mm_rows(rows, a, b, "int8", sa, sb, "bf16"), full[rows])


def test_f64_output_is_exact_product_of_scales(orc):
    a = _codes((4, 96), "fp8", 17)
    b = _codes((6, 96), "fp8", 18)
    sa = np.array([0.5, 0.25, 2.0, 1.0], np.float32)
    sb = np.array([1, 2, 4, 8, 0.5, 0.125], np.float32)  # powers of two: products exact
    acc, den = _exact_acc(a, b, "fp8")
    want = acc / den * sa[:, None].astype(np.float64) * sb[None, :].astype(np.float64)
    assert np.array_equal(orc.scaled_mm(a, b, "fp8", sa, sb, "f64"), want)
