"""Pins of the oracle's asymmetric int8 functions (the asymmetric int8 case
of "[Kernel] Add w8a8 CUTLASS kernels": zero points per token and small
operations fused onto the GEMM; the pages give no formula, the textbook
scheme x ~ (q - z) * s over the row's range with 0 included is taken).

The pins do not retype the oracle: closed forms (0 maps to the zero point,
the row's negative extreme to -128, an all-zero row to scale 1 and codes
-128), the rounding-error bound of every element, and the product against
exact Python integers and against numpy's float64 matrix product of the
dequantised operands.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def _rows(seed, M=6, K=96):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32) * rng.uniform(0.1, 10, (M, 1)).astype(np.float32)
    x[1] = np.abs(x[1])            # all non-negative: lo = 0
    x[2] = -np.abs(x[2])           # all non-positive: hi = 0
    x[3] = 0.0                     # all zero
    x[4, :] = 0.0
    x[4, 7] = -3.0                 # a single negative value
    return x


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_azp_quant_closed_forms(seed):
    x = _rows(seed)
    q, s, z = oracle.quant_per_token_azp(x, "f32")
    qi = q.view(np.int8).astype(np.int64)
    for m in range(x.shape[0]):
        lo, hi = min(0.0, float(x[m].min())), max(0.0, float(x[m].max()))
        if hi == lo:
            assert s[m] == np.float32(1.0) and z[m] == -128 and (qi[m] == -128).all()
            continue
        assert s[m] == np.float32(np.float32(hi - lo) / np.float32(255.0))
        assert -128 <= z[m] <= 127
        if lo < 0:
            assert qi[m, int(np.argmin(x[m]))] == -128   # the negative extreme is the lowest code
        else:
            assert z[m] == -128                           # lo = 0 sits on the lowest code
        zero = x[m] == 0
        assert (qi[m][zero] == z[m]).all()                # 0 is exactly representable


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_azp_quant_error_bound(seed):
    """(q - z) * s is within half a step s of x for every element."""
    x = _rows(seed, M=8, K=512)
    q, s, z = oracle.quant_per_token_azp(x, "f32")
    deq = (q.view(np.int8).astype(np.float64) - z[:, None]) * s[:, None].astype(np.float64)
    err = np.abs(deq - x.astype(np.float64))
    assert (err <= 0.5 * s[:, None] * (1 + 2.0 ** -12)).all()


def test_azp_quant_bf16_input_matches_f32():
    x = workloads.activations(5, 272, seed=4)
    xh = workloads.as_u16(x)
    q1, s1, z1 = oracle.quant_per_token_azp(xh, "bf16")
    q2, s2, z2 = oracle.quant_per_token_azp(x.float().numpy(), "f32")
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2) and np.array_equal(z1, z2)


def test_colsum_is_the_row_sum():
    b = workloads.random_codes((37, 160), "int8", seed=3).numpy()
    assert np.array_equal(oracle.colsum(b), b.view(np.int8).astype(np.int64).sum(axis=1))


def test_scaled_mm_azp_against_python_integers():
    """I32 output = sum_k (a - z) b exactly; f64 output = that times the
    scales, within two binary64 roundings; per-tensor and per-token zero
    points."""
    rng = np.random.default_rng(5)
    M, N, K = 3, 5, 48
    a = workloads.random_codes((M, K), "int8", seed=6).numpy()
    b = workloads.random_codes((N, K), "int8", seed=7).numpy()
    ai, bi = a.view(np.int8).astype(int), b.view(np.int8).astype(int)
    sa = rng.uniform(0.001, 0.1, M).astype(np.float32)
    sb = rng.uniform(0.001, 0.1, N).astype(np.float32)
    for z in (np.array([17], np.int32), np.array([-128, 0, 127], np.int32)):
        acc = oracle.scaled_mm_azp(a, b, None, z, None, "i32")
        d = oracle.scaled_mm_azp(a, b, sa, z, sb, "f64")
        for m in range(M):
            zm = int(z[0] if z.size == 1 else z[m])
            for n in range(N):
                exact = sum((int(ai[m, k]) - zm) * int(bi[n, k]) for k in range(K))
                assert acc[m, n] == exact
                want = Fraction(exact) * Fraction(float(sa[m])) * Fraction(float(sb[n]))
                assert abs(Fraction(float(d[m, n])) - want) <= abs(want) * Fraction(1, 2 ** 51)


def test_scaled_mm_azp_is_the_dequantised_product():
    """D = ((a - z) s_a) . (b s_b)^T, numpy float64 matmul as the reference;
    zero points of 0 reduce to the symmetric product."""
    x = workloads.activations(4, 256, seed=8)
    a, sa, z = oracle.quant_per_token_azp(workloads.as_u16(x), "bf16")
    w = workloads.weights(24, 256, seed=9)
    b, sb = oracle.quant_per_token(workloads.as_u16(w), "int8", xtype="bf16")
    d = oracle.scaled_mm_azp(a, b, sa, z, sb, "f64")
    ref = ((a.view(np.int8).astype(np.float64) - z[:, None]) * sa[:, None]) @ \
          (b.view(np.int8).astype(np.float64) * sb[:, None]).T
    assert np.allclose(d, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    sym = oracle.scaled_mm(a, b, "int8", sa, sb, "f64")
    assert np.array_equal(oracle.scaled_mm_azp(a, b, sa, None, sb, "f64"), sym)


# Rows whose range hi - lo is 255 * 2^j make the scale the power of two 2^j
# exactly, so x / s and -128 - lo / s are exact and can be placed on a tie
# (a value half-way between two integers). The codes below are worked out by
# hand with round-half-to-even at each tie; rounding half away from zero
# gives a different zero point or code in every row.
TIE_ROWS = [
    # (row values, scale, zero point, codes)
    # lo = -127.5, hi = 127.5: s = 1, -128 - lo / s = -0.5 -> z = 0 (away: -1)
    ([-127.5, 127.5, 2.5, -0.5, 1.5, 3.5, 0.5, -2.5],
     1.0, 0, [-128, 127, 2, 0, 2, 4, 0, -2]),
    # lo = -64, hi = 191: s = 1, z = -64 exactly; ties in x / s only
    ([-64.0, 191.0, 2.5, -0.5, 0.5, 1.5, -1.5, 0.0],
     1.0, -64, [-128, 127, -62, -64, -64, -62, -66, -64]),
    # lo = -255, hi = 255: s = 2, -128 - lo / s = -0.5 -> z = 0; x / s ties
    ([-255.0, 255.0, 5.0, 3.0, -1.0, 1.0, -3.0, 7.0],
     2.0, 0, [-128, 127, 2, 2, 0, 0, -2, 4]),
    # lo = -31.875, hi = 0: s = 0.125, -128 - lo / s = -128 + 255 = 127 -> z = 127;
    # x / s = -0.5 -> 0 -> code 127, -1.5 -> -2 -> 125, -126.5 -> -126 -> 1
    ([-31.875, 0.0, -0.0625, -0.1875, -0.3125, -15.8125, -0.125, -8.0625],
     0.125, 127, [-128, 127, 127, 125, 125, 1, 126, 63]),
]


@pytest.mark.parametrize("row", range(len(TIE_ROWS)))
@pytest.mark.parametrize("xtype", ["f32", "bf16"])
def test_azp_quant_ties_round_half_even(row, xtype):
    vals, s, z, codes = TIE_ROWS[row]
    x = np.array([vals], np.float32)
    if xtype == "bf16":
        # every value above has at most 8 significant bits: bf16 holds it exactly
        h = (x.view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal((h.astype(np.uint32) << 16).view(np.float32), x)
        q, sc, zp = oracle.quant_per_token_azp(h, "bf16")
    else:
        q, sc, zp = oracle.quant_per_token_azp(x, "f32")
    assert sc[0] == np.float32(s)
    assert zp[0] == z
    assert q.view(np.int8)[0].tolist() == codes


def test_colsum_closed_forms():
    """Rows with a closed-form sum: a constant row c sums to c * K, the ramp
    -64..63 repeated sums to -K / 2 (each 128-code period sums to -64), a row
    and its negation sum to 0, and the extremes -128 and 127 do not wrap."""
    K = 4096
    rows = np.zeros((6, K), np.int8)
    rows[0] = 7
    rows[1] = -128
    rows[2] = 127
    rows[3] = (np.arange(K) % 128 - 64).astype(np.int8)
    rows[4] = workloads.random_codes((1, K), "int8", seed=11).numpy().view(np.int8)[0]
    rows[4][rows[4] == -128] = -127
    rows[5] = -rows[4]
    cs = oracle.colsum(rows.view(np.uint8))
    assert cs[0] == 7 * K and cs[1] == -128 * K and cs[2] == 127 * K
    assert cs[3] == -(K // 2)
    assert cs[4] + cs[5] == 0


def test_colsum_brute_force_tiny():
    """Small weights summed one code at a time in Python integers."""
    b = workloads.random_codes((5, 48), "int8", seed=12).numpy()
    cs = oracle.colsum(b)
    for n in range(5):
        total = 0
        for k in range(48):
            c = int(b[n, k])
            total += c - 256 if c >= 128 else c
        assert cs[n] == total


# ---------------------------------------------------------------- per tensor
# One scale and zero point for the whole tensor ("[Kernel] Add w8a8 CUTLASS
# kernels": zero points per tensor or per token): the per-token scheme over
# all elements at once (dynamic), or with a calibrated scale and zero point
# (static).

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_azp_per_tensor_dynamic_is_one_long_row(seed):
    """The dynamic per-tensor result equals the per-token one of the tensor
    laid out as a single row (itself pinned by the closed forms and ties above)."""
    x = _rows(seed, M=6, K=96)
    q, s, z = oracle.quant_per_tensor_azp(x, "f32")
    q1, s1, z1 = oracle.quant_per_token_azp(x.reshape(1, -1), "f32")
    assert s == s1[0] and z == z1[0]
    assert np.array_equal(q.reshape(1, -1), q1)


def test_azp_per_tensor_closed_forms():
    x = _rows(3, M=5, K=64)
    q, s, z = oracle.quant_per_tensor_azp(x, "f32")
    lo, hi = min(0.0, float(x.min())), max(0.0, float(x.max()))
    assert s == np.float32(np.float32(hi - lo) / np.float32(255.0))
    qi = q.view(np.int8)
    assert qi.reshape(-1)[int(np.argmin(x))] == -128
    assert (qi[x == 0] == z).all()
    deq = (qi.astype(np.float64) - z) * np.float64(s)
    assert (np.abs(deq - x) <= 0.5 * np.float64(s) * (1 + 2.0 ** -12)).all()
    zq, zs, zz = oracle.quant_per_tensor_azp(np.zeros((3, 32), np.float32), "f32")
    assert zs == np.float32(1.0) and zz == -128 and (zq.view(np.int8) == -128).all()


@pytest.mark.parametrize("scale,azp", [(0.05, 3), (1.0, -128), (0.37, 127), (2.0, 0)])
def test_azp_per_tensor_static_brute_force(scale, azp):
    """Static: q = clamp(round_half_even(fl32(x / s)) + z, -128, 127), element
    by element with numpy's binary32 division and Python's round (ties to even)."""
    x = _rows(4, M=6, K=48) * np.float32(3.0)
    x[0, :8] = np.float32(scale) * np.array([0.5, 1.5, 2.5, -0.5, -1.5, 100.5, -300.0, 1e6], np.float32)
    q, s, z = oracle.quant_per_tensor_azp(x, "f32", scale=scale, azp=azp, dynamic=False)
    assert s == np.float32(scale) and z == azp
    qi = q.view(np.int8)
    for m in range(x.shape[0]):
        for k in range(x.shape[1]):
            t = float(np.float32(x[m, k]) / np.float32(scale))
            want = min(127, max(-128, round(t) + azp))
            assert qi[m, k] == want, (m, k, x[m, k], t)


def test_azp_per_tensor_static_null_means_one_and_zero():
    x = _rows(5, M=6, K=32)
    q, s, z = oracle.quant_per_tensor_azp(x, "f32", dynamic=False)
    q2, _, _ = oracle.quant_per_tensor_azp(x, "f32", scale=1.0, azp=0, dynamic=False)
    assert s == np.float32(1.0) and z == 0 and np.array_equal(q, q2)
