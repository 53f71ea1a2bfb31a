"""Pins for the oracle's codecs (e4m3fn, int8, bf16, fp16).

Each check compares the oracle with something that is not the oracle: the
hand-derived OCP code points in tests/golden, torch's CPU float8_e4m3fn cast
run through the pages' own clamp-then-cast recipe ("[Kernel] Add w8a8
CUTLASS kernels", per_tensor_quantize snippet), numpy's rint and float16
conversion, and exact rational brute force.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_recipe_e4m3(v: np.ndarray) -> np.ndarray:
    """The pages' recipe: clamp to finfo(e4m3fn) range, then cast (torch CPU)."""
    fi = torch.finfo(torch.float8_e4m3fn)
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.clamp(min=fi.min, max=fi.max).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _all_finite_codes():
    return np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def test_golden_points(orc):
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_ocp_points.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, val = line.split()[:2]
            rows.append((int(code, 16), val))
    assert len(rows) >= 15
    dec = orc.e4m3_decode(np.array([c for c, _ in rows], np.uint8))
    for (code, val), got in zip(rows, dec):
        if val == "nan":
            assert math.isnan(got), hex(code)
        else:
            want = float(val)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), hex(code)


def test_decode_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert np.nanmax(ours) == 448.0  # the max-norm the KV-cache page states


def test_encode_roundtrip_every_code(orc):
    c = _all_finite_codes()
    assert np.array_equal(orc.e4m3_encode(orc.e4m3_decode(c).astype(np.float32)), c)


def _midpoints_and_neighbours(orc):
    vals = np.sort(np.unique(orc.e4m3_decode(_all_finite_codes())))
    mids = (vals[:-1] + vals[1:]) / 2  # exact in fp32: e4m3 midpoints need 5 bits
    m32 = mids.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mids)
    up = np.nextafter(m32, np.float32(np.inf))
    dn = np.nextafter(m32, np.float32(-np.inf))
    beyond = np.array([448, 456, 464, 464.0001, 480, 1e4, 3e38, np.inf], np.float32)
    out = np.concatenate([m32, up, dn, beyond, -beyond])
    return out


def test_encode_matches_pages_recipe_on_ties_and_boundaries(orc):
    v = _midpoints_and_neighbours(orc)
    assert np.array_equal(orc.e4m3_encode(v), _torch_recipe_e4m3(v))


def test_encode_matches_pages_recipe_on_all_bf16_values(orc):
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(orc.e4m3_encode(v), _torch_recipe_e4m3(v))


def test_encode_matches_pages_recipe_on_fp32_sweep(orc):
    # Every 1021st fp32 bit pattern (about 4.2M values across all binades).
    bits = np.arange(0, 2**32, 1021, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(orc.e4m3_encode(v), _torch_recipe_e4m3(v))


def test_encode_nan(orc):
    assert orc.e4m3_encode(np.array([np.nan, -np.nan], np.float32)).tolist() == [0x7F, 0x7F]


def test_encode_is_nearest_by_brute_force(orc):
    """Nearest finite code by exhaustive search in exact rationals, ties to the
    code with even mantissa, sign of zero kept."""
    codes = _all_finite_codes()
    exact = [(int(c), Fraction(float(x))) for c, x in zip(codes, orc.e4m3_decode(codes))
             if not (c == 0x80)]
    rng = np.random.default_rng(7)
    mags = np.concatenate([rng.uniform(0, 2**-8, 300), rng.uniform(0, 1, 300),
                           rng.uniform(0, 500, 300), 2.0 ** rng.uniform(-12, 9, 300)])
    v = (mags * rng.choice([-1, 1], mags.size)).astype(np.float32)
    got = orc.e4m3_encode(v)
    for x, g in zip(v, got):
        fx = Fraction(float(max(min(x, 448), -448)))
        best = min(abs(fx - val) for _, val in exact)
        cands = [c for c, val in exact if abs(fx - val) == best]
        if len(cands) > 1:
            cands = [c for c in cands if (c & 1) == 0]
        want = cands[0]
        if want == 0 and np.signbit(x):
            want = 0x80
        assert g == want, (x, hex(g), hex(want))


def test_encode_monotone(orc):
    v = np.sort(np.random.default_rng(3).uniform(-500, 500, 200000).astype(np.float32))
    d = orc.e4m3_decode(orc.e4m3_encode(v))
    assert np.all(np.diff(d) >= 0)


def test_int8_encode_matches_numpy(orc):
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.uniform(-300, 300, 100000), np.arange(-200, 200.5, 0.5),
                        [np.inf, -np.inf, 127.5, -127.5, 126.5, 0.5, -0.5, 1.5, 2.5]]).astype(np.float32)
    want = np.clip(np.rint(v.astype(np.float64)), -127, 127).astype(np.int8)
    assert np.array_equal(orc.int8_encode(v), want)
    assert orc.int8_encode(np.array([0.5, 1.5, 2.5, -2.5, 300, -300], np.float32)).tolist() == \
        [0, 2, 2, -2, 127, -127]


def _nearest_bf16_bits(x: float) -> int:
    """Nearest bf16 to the double x by exact comparison of its fp32-derived
    neighbours; ties to even; overflow by IEEE's rule (round with unbounded
    exponent, then compare with the largest finite value)."""
    fx = Fraction(x)
    f = np.float32(x)
    if np.isinf(f):
        base = 0x7F7F if x > 0 else 0xFF7F
    else:
        base = int(np.array(f).view(np.uint32)) >> 16
    cands = set()
    for d in (-2, -1, 0, 1, 2):
        b = (base & 0x8000) | max(0, min(0x7F80, (base & 0x7FFF) + d))
        cands.add(b)

    def val(b):
        if (b & 0x7FFF) == 0x7F80:
            return None
        return Fraction(float(np.array(b << 16, np.uint32).view(np.float32)))
    finite = [(abs(fx - val(b)), b) for b in cands if val(b) is not None]
    best = min(d for d, _ in finite)
    win = [b for d, b in finite if d == best]
    if len(win) > 1:
        win = [b for b in win if (b & 1) == 0]
    b = win[0]
    # IEEE overflow: beyond max + half an ulp (the tie goes to the even "2^128").
    maxf = Fraction(float(np.array(0x7F7F0000, np.uint32).view(np.float32)))
    half_ulp = Fraction(2) ** (127 - 8)
    if abs(fx) >= maxf + half_ulp:
        b = 0x7F80 if x > 0 else 0xFF80
    return b


def test_bf16_from_double_brute_force(orc):
    rng = np.random.default_rng(5)
    base = rng.standard_normal(3000) * 2.0 ** rng.integers(-140, 128, 3000)
    # exact ties between adjacent bf16 values, and values one double-ulp off them
    lo = rng.integers(0x0001, 0x7F7E, 1000).astype(np.uint32)
    a = (lo << 16).view(np.float32).astype(np.float64)
    b = ((lo + 1) << 16).view(np.float32).astype(np.float64)
    ties = (a + b) / 2
    vals = np.concatenate([base, ties, np.nextafter(ties, np.inf), np.nextafter(ties, -np.inf),
                           -ties, [3.3961e38, 3.40e38, -3.40e38, 1e-45, -1e-45, 0.0, -0.0]])
    got = orc.bf16_from_f64(vals)
    for x, g in zip(vals, got):
        assert g == _nearest_bf16_bits(float(x)), (x, hex(g))


def test_fp16_from_double_matches_numpy(orc):
    rng = np.random.default_rng(6)
    v = np.concatenate([rng.standard_normal(20000) * 2.0 ** rng.integers(-30, 17, 20000),
                        [65504.0, 65519.99, 65520.0, -65520.0, 2.0**-25, 2.0**-24, 3 * 2.0**-26]])
    # ties between adjacent halves and their neighbours
    h = rng.integers(1, 0x7BFF, 2000).astype(np.uint16)
    a = h.view(np.float16).astype(np.float64)
    b = (h + 1).view(np.float16).astype(np.float64)
    t = (a + b) / 2
    v = np.concatenate([v, t, np.nextafter(t, np.inf), np.nextafter(t, -np.inf)])
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.fp16_from_f64(v), want)
