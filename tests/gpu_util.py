"""Helpers for the GPU parity tests: moving bit patterns between numpy (the
oracle's side) and torch device tensors (the HIP library's side), and the
output tolerance of the scaled matrix multiply."""
from __future__ import annotations

import numpy as np
import torch

import oracle

DEV = "cuda"
TORCH_OF = {"bf16": torch.bfloat16, "fp16": torch.float16, "f32": torch.float32,
            "i32": torch.int32}
CODE_TORCH = {"int8": torch.int8, "fp8": torch.float8_e4m3fn}


def to_dev_bits(u16: np.ndarray, dtype: str) -> torch.Tensor:
    """uint16 bit patterns -> bf16/fp16 device tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(TORCH_OF[dtype])
    return t.to(DEV)


def codes_to_dev(q: np.ndarray, qtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(q).view(np.uint8)).view(CODE_TORCH[qtype])
    return t.to(DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a device tensor's bit patterns (uint8 / uint16 / uint32)."""
    t = t.detach().cpu().contiguous()
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, np.float32)).view(np.uint32)


def out_value(t: torch.Tensor) -> np.ndarray:
    """Device output -> float64 values on the host."""
    return t.detach().cpu().double().numpy()


def ulp(x: np.ndarray, otype: str) -> np.ndarray:
    """Spacing of the output format at |x| (subnormal spacing below the normal range)."""
    p, emin = {"bf16": (8, -126), "fp16": (11, -14), "f32": (24, -126)}[otype]
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - (p - 1)).astype(np.int64))


def fp8_group_bound(a: np.ndarray, b: np.ndarray, group: int = 8) -> np.ndarray:
    """Upper bound of sum over k-groups of max_group |a_k| * max_group |b_k|.

    Computed as a matmul of per-group maxima (groups of `group` consecutive k).
    """
    da = np.abs(oracle.e4m3_decode(a.view(np.uint8)))
    db = np.abs(oracle.e4m3_decode(b.view(np.uint8)))
    M, K = da.shape
    ga = da.reshape(M, K // group, group).max(axis=2)
    gb = db.reshape(db.shape[0], K // group, group).max(axis=2)
    return ga @ gb.T


# The fp8 matrix cores (v_mfma_f32_16x16x128_f8f6f4, _32x32x64_) add each
# group of 8 consecutive products (k = 8j .. 8j+7) after aligning them to the
# group's largest product: every other product is truncated toward zero to a
# multiple of 2^(E-13), 2^E the leading bit of the largest (characterised on
# the device in tests/test_gpu_fp8_mfma_groups.py: 2^-13 below the largest is
# kept, 2^-14 and 0.75 * 2^-13 are dropped, 1.25 * 2^-13 keeps 2^-13, negative
# products lose their low bits toward zero, seven products of 2^-14 are all
# dropped). The at most 7 truncated products lose less than 7 * 2^-13 < 2^-10
# of the group's max |a| * max |b| (derived in tests/test_fp8_group_model.py).
FP8_GROUP_REL = 2.0 ** -10


def min_exact_frac(qtype: str, otype: str) -> float:
    """Least fraction of outputs that must equal the oracle's own rounding.
    int8 accumulators are exact, so only the fp32 epilogue (a few 2^-24)
    separates the two roundings. fp8 sums carry the matrix core's group
    truncation, biased toward zero by up to ~2^-10 of a group's largest
    product: bf16 (7 fraction bits) hides most of it, fp16 (10 bits) shows
    8 times more of it in its last bit (measured 0.85 - 0.86 equal and
    0.95 - 0.96 within one fp16 ulp at the Llama-3-8B prefill shapes)."""
    if qtype == "int8":
        return 0.97
    return 0.9 if otype == "bf16" else 0.75


def assert_close_fraction(info: dict, qtype: str, otype: str) -> None:
    """exact_frac above min_exact_frac and, for fp8, 90% within one ulp."""
    assert info.get("exact_frac", 1.0) > min_exact_frac(qtype, otype), info
    if qtype == "fp8" and "within_1ulp" in info:
        assert info["within_1ulp"] > 0.9, info


def check_scaled_mm_rows(got: torch.Tensor, rows, a: np.ndarray, b: np.ndarray, qtype: str,
                         sa, sb, otype: str) -> dict:
    """check_scaled_mm on a sample of output rows (for sizes where the full
    oracle product would take too long)."""
    rows = np.asarray(sorted(set(int(r) for r in rows)), np.int64)
    sa_rows = sa if (sa is None or np.size(sa) == 1) else np.asarray(sa)[rows]
    return check_scaled_mm(got[torch.from_numpy(rows).to(got.device)], a[rows], b, qtype,
                           sa_rows, sb, otype)


def check_scaled_mm(got: torch.Tensor, a: np.ndarray, b: np.ndarray, qtype: str, sa, sb,
                    otype: str, max_abs_rel: float = 1e-2) -> dict:
    """Compare a HIP scaled_mm output with the oracle.

    int8, i32 output: bit-exact raw accumulator.
    int8, bf16/fp16: |D - D_exact| <= 1 ulp of the output format (the
      accumulator is exact; the fp32 epilogue adds < 3 * 2^-24 relative,
      then one rounding to nearest). f32 output: 3 float32 ulps (three
      roundings: int -> float, * a_scale, * b_scale).
    fp8: on top of that, the accumulation error: any fp32 summation order
      (K * 2^-24 * sum_k |a_k b_k|) plus the matrix core's in-group alignment
      (2^-10 * sum over groups of max|a| * max|b|), times |a_scale * b_scale|.
    Overall max|D - D_exact| / max|D_exact| <= 1e-2. Reported: the fraction
    of elements equal to the oracle's own rounding, and within 1 ulp.
    """
    M, K = a.shape
    if otype == "i32":
        ref = oracle.scaled_mm(a, b, qtype, None, None, "i32")
        assert np.array_equal(got.cpu().numpy(), ref), "raw int32 accumulator differs"
        return {"exact_frac": 1.0}
    exact = oracle.scaled_mm(a, b, qtype, sa, sb, "f64")
    g = out_value(got)
    u = ulp(exact, otype)
    tol = 3 * u if otype == "f32" else u.copy()
    if qtype == "fp8" and K > 0:
        absa = np.ascontiguousarray(a.view(np.uint8) & 0x7F)
        absb = np.ascontiguousarray(b.view(np.uint8) & 0x7F)
        mag = oracle.scaled_mm(absa, absb, "fp8", None, None, "f64")
        sab = np.abs(np.asarray(1.0 if sa is None else sa, np.float64).reshape(-1, 1)) * \
            np.abs(np.asarray(1.0 if sb is None else sb, np.float64).reshape(1, -1))
        tol = tol + sab * (mag * K * 2.0 ** -24 + FP8_GROUP_REL * fp8_group_bound(a, b))
    err = np.abs(g - exact)
    bad = ~(err <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{bad.sum()} of {bad.size} elements out of tolerance; first at "
                             f"{i}: got {g[i]!r}, exact {exact[i]!r}, tol {tol[i]!r}")
    denom = np.abs(exact).max() if exact.size else 0.0
    rel = err.max() / denom if denom > 0 else (err.max() if err.size else 0.0)
    assert rel <= max_abs_rel, rel
    ref_bits = oracle.scaled_mm(a, b, qtype, sa, sb, otype)
    gb = bits(got)
    if otype == "f32":
        ref_bits = ref_bits.view(np.uint32)
    return {"exact_frac": float(np.mean(gb == ref_bits)),
            "within_1ulp": float(np.mean(err <= u)), "max_abs_rel": float(rel)}
