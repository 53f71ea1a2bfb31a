"""Pins for the oracle's quantizers.

Closed forms from the pages: scale = absmax / 448 and q = fp8(x / scale),
x' = dequant(q) * scale ("Enable scaled FP8 (e4m3fn) KV cache on ROCm",
"Scaling semantics"); divide, clamp to the e4m3 range, cast ("[Kernel] Add
w8a8 CUTLASS kernels", per_tensor_quantize snippet); no scale means 1.0
(KV-cache page, review answers). Checked against torch's CPU arithmetic and
float8 cast, numpy's rint, and error bounds that hold for any correct
rounding.
"""
import numpy as np
import pytest
import torch

import workloads

FI = torch.finfo(torch.float8_e4m3fn)


def _bf16_f32(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _torch_fp8_recipe(x32: np.ndarray, s) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32))
    st = torch.from_numpy(np.ascontiguousarray(np.asarray(s, np.float32)))
    return (t / st).clamp(min=FI.min, max=FI.max).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_int8_recipe(x32: np.ndarray, s) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32))
    st = torch.from_numpy(np.ascontiguousarray(np.asarray(s, np.float32)))
    return torch.round(t / st).clamp(-127, 127).to(torch.int8).view(torch.uint8).numpy()


def _row_absmax_scale(x32, qmax):
    amax = torch.from_numpy(np.abs(x32)).amax(dim=-1)
    s = amax / torch.tensor(qmax, dtype=torch.float32)
    s[amax == 0] = 1.0
    return s.numpy()


@pytest.mark.parametrize("qtype,qmax", [("fp8", 448.0), ("int8", 127.0)])
@pytest.mark.parametrize("M,K", [(1, 4096), (16, 4096), (64, 14336), (37, 200)])
def test_per_token_matches_pages_recipe(orc, qtype, qmax, M, K):
    x = workloads.activations(M, K, seed=M + K)
    xb = workloads.as_u16(x)
    q, s = orc.quant_per_token(xb, qtype, xtype="bf16")
    x32 = _bf16_f32(xb)
    s_ref = _row_absmax_scale(x32, qmax)
    assert np.array_equal(s, s_ref)
    recipe = _torch_fp8_recipe if qtype == "fp8" else _torch_int8_recipe
    assert np.array_equal(q, recipe(x32, s_ref[:, None]))
    # every row's largest magnitude lands on the top code
    top = q[np.arange(M), np.abs(x32).argmax(axis=1)]
    if qtype == "fp8":
        assert set(top.tolist()) <= {0x7E, 0xFE}
    else:
        assert set(top.view(np.int8).tolist()) <= {127, -127}


def test_per_token_round_trip_error_bound(orc):
    """|dequant(q) * s - x| <= half an e4m3 spacing at x/s, times s (plus the
    division's own rounding): holds for any correct nearest rounding and
    fails for a wrong scale, index or truncation."""
    x = workloads.activations(32, 4096, seed=3)
    xb = workloads.as_u16(x)
    q, s = orc.quant_per_token(xb, "fp8", xtype="bf16")
    x64 = _bf16_f32(xb).astype(np.float64)
    y = orc.e4m3_decode(q) * s[:, None].astype(np.float64)
    t = np.abs(x64 / s[:, None])
    e = np.floor(np.log2(np.maximum(t, 2.0 ** -6)))
    half_spacing = 2.0 ** (e - 3) / 2
    bound = (half_spacing + t * 2.0 ** -23) * s[:, None]
    assert np.all(np.abs(y - x64) <= bound)


def test_all_bf16_values_against_recipe(orc):
    """Exhaustive over the 65,536 bf16 inputs (NaN excluded) for a set of static scales."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = _bf16_f32(bits)
    bits = bits[~np.isnan(v)]
    v = v[~np.isnan(v)]
    for s in [1.0, 1.0 / 448, 0.0123, 3.7, 2.0 ** -20, 1e10]:
        s32 = np.float32(s)
        q, s_out = orc.quant_per_tensor(bits.reshape(1, -1), "fp8", scale=s32, xtype="bf16")
        assert s_out == s32
        assert np.array_equal(q.reshape(-1), _torch_fp8_recipe(v, s32)), s
        qi, _ = orc.quant_per_tensor(bits.reshape(1, -1), "int8", scale=s32, xtype="bf16")
        fin = np.isfinite(v)
        assert np.array_equal(qi.reshape(-1)[fin], _torch_int8_recipe(v[fin], s32)), s


def test_per_tensor_dynamic_scale_is_absmax_over_448(orc):
    x = workloads.activations(50, 300, seed=4)
    xb = workloads.as_u16(x)
    q, s = orc.quant_per_tensor(xb, "fp8", dynamic=True, xtype="bf16")
    amax = np.abs(_bf16_f32(xb)).max()
    assert s == np.float32(amax) / np.float32(448.0)
    assert np.array_equal(q, _torch_fp8_recipe(_bf16_f32(xb), s))
    assert np.sum((q & 0x7F) == 0x7E) >= 1


def test_null_static_scale_means_one(orc):
    x = workloads.activations(4, 64, seed=5)
    xb = workloads.as_u16(x)
    q0, s0 = orc.quant_per_tensor(xb, "fp8", scale=None, xtype="bf16")
    q1, s1 = orc.quant_per_tensor(xb, "fp8", scale=np.float32(1.0), xtype="bf16")
    assert s0 == 1.0 and np.array_equal(q0, q1)
    assert np.array_equal(q0, _torch_fp8_recipe(_bf16_f32(xb), np.float32(1.0)))


def test_zero_rows_get_scale_one(orc):
    x = np.zeros((3, 128), np.uint16)
    x[1, 5] = 0x3F80  # 1.0 in bf16
    q, s = orc.quant_per_token(x, "fp8", xtype="bf16")
    assert s.tolist() == [1.0, np.float32(1.0) / np.float32(448.0), 1.0]
    assert q[1, 5] == 0x7E and q.sum() == 0x7E


def test_static_scale_saturates(orc):
    """A calibrated scale smaller than the runtime absmax saturates at +-448."""
    x = np.array([[1000.0, -1000.0, 1.0, -0.0]], np.float32)
    q, _ = orc.quant_per_tensor(x, "fp8", scale=np.float32(1.0))
    assert q.tolist() == [[0x7E, 0xFE, 0x38, 0x80]]
    qi, _ = orc.quant_per_tensor(x, "int8", scale=np.float32(1.0))
    assert qi.view(np.int8).tolist() == [[127, -127, 1, 0]]


def test_fp16_and_f32_inputs_agree_with_bf16(orc):
    x = workloads.activations(8, 256, seed=6)
    xb = workloads.as_u16(x)
    x32 = _bf16_f32(xb)
    qa, sa = orc.quant_per_token(xb, "fp8", xtype="bf16")
    qb, sb = orc.quant_per_token(x32, "fp8")
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb)
    h = torch.from_numpy(x32).to(torch.float16)
    hb = h.view(torch.int16).numpy().view(np.uint16)
    qc, sc = orc.quant_per_token(hb, "fp8", xtype="fp16")
    h32 = h.float().numpy()
    assert np.array_equal(sc, _row_absmax_scale(h32, 448.0))
    assert np.array_equal(qc, _torch_fp8_recipe(h32, sc[:, None]))


def test_kv_round_trip(orc):
    """KV cache: scale = absmax/448; the absmax element comes back exactly;
    every element comes back within half an e4m3 spacing (scaled) plus half a
    bf16 ulp; and quantising the dequantised tensor again with the same scale
    reproduces the codes."""
    x = workloads.kv_tensor(0, "k", shape=(256, 8, 128))
    xb = workloads.as_u16(x).reshape(-1)
    q, s = orc.kv_quant(xb, xtype="bf16")
    x32 = _bf16_f32(xb)
    amax = np.abs(x32).max()
    assert s == np.float32(amax) / np.float32(448.0)
    assert np.array_equal(q, _torch_fp8_recipe(x32, s))
    y = orc.kv_dequant(q, s, "bf16")
    y32 = _bf16_f32(y)
    i = np.abs(x32).argmax()
    assert y32[i] == x32[i]
    # dequant itself: RNE_bf16(fl32(dec(q) * s)) via torch arithmetic
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).float()
    want = (dec * torch.tensor(s)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, want)
    t = np.abs(x32.astype(np.float64) / s)
    e = np.floor(np.log2(np.maximum(t, 2.0 ** -6)))
    bound = (2.0 ** (e - 3) / 2 + t * 2.0 ** -23) * s + np.abs(y32) * 2.0 ** -8
    assert np.all(np.abs(y32.astype(np.float64) - x32) <= bound)
    q2, _ = orc.kv_quant(y, scale=s, dynamic=False, xtype="bf16")
    assert np.array_equal(q2, q)


def test_kv_dequant_null_scale_means_one(orc):
    q = np.arange(256, dtype=np.uint8)
    q = q[(q & 0x7F) != 0x7F]
    y = orc.kv_dequant(q, None, "f32")
    assert np.array_equal(y, orc.e4m3_decode(q).astype(np.float32))
