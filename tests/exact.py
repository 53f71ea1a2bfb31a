"""Exact-rational helpers for the tests: nearest bf16 / fp16 of a rational.

Independent of the oracle: candidates come from numpy's own conversions and
the winner is chosen by exact comparison, ties to the even bit pattern, with
IEEE overflow (round as if the exponent were unbounded, then compare with the
largest finite value).
"""
from fractions import Fraction

import numpy as np

_BF16_MAX = Fraction(float(np.array(0x7F7F0000, np.uint32).view(np.float32)))
_FP16_MAX = Fraction(65504)


def _bf16_val(b: int) -> Fraction:
    return Fraction(float(np.array(b << 16, np.uint32).view(np.float32)))


def _fp16_val(b: int) -> Fraction:
    return Fraction(float(np.array(b, np.uint16).view(np.float16)))


def _pick(fx, cands, val):
    best = min(abs(fx - val(b)) for b in cands)
    win = sorted(b for b in cands if abs(fx - val(b)) == best)
    if len(win) > 1:
        win = [b for b in win if (b & 1) == 0]
    return win[0]


def nearest_bf16(x) -> int:
    fx = Fraction(x)
    neg = fx < 0 or (fx == 0 and np.signbit(float(x)))
    a = abs(fx)
    if a >= _BF16_MAX + Fraction(2) ** 119:
        return 0xFF80 if neg else 0x7F80
    f = np.float32(float(a)) if a <= Fraction(float(np.finfo(np.float32).max)) else np.float32(np.finfo(np.float32).max)
    base = int(np.array(f).view(np.uint32)) >> 16
    cands = {max(0, min(0x7F7F, base + d)) for d in (-2, -1, 0, 1, 2)}
    b = _pick(a, cands, _bf16_val)
    return b | (0x8000 if neg else 0)


def nearest_fp16(x) -> int:
    fx = Fraction(x)
    neg = fx < 0 or (fx == 0 and np.signbit(float(x)))
    a = abs(fx)
    if a >= _FP16_MAX + Fraction(2) ** 4:
        return 0xFC00 if neg else 0x7C00
    with np.errstate(over="ignore"):
        base = int(np.array(np.float16(min(float(a), 65504.0))).view(np.uint16))
    cands = {max(0, min(0x7BFF, base + d)) for d in (-2, -1, 0, 1, 2)}
    b = _pick(a, cands, _fp16_val)
    return b | (0x8000 if neg else 0)


def e4m3_int512(codes) -> np.ndarray:
    """512 * value of e4m3 codes as exact int64, decoded by torch's float8 type."""
    import torch
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    v = c.view(torch.float8_e4m3fn).double().numpy() * 512.0
    assert np.all(v == np.round(v))
    return v.astype(np.int64)
