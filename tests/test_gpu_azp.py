"""GPU parity of the asymmetric int8 path (the asymmetric int8 case of
"[Kernel] Add w8a8 CUTLASS kernels": zero points and the small operations
fused onto the GEMM) against the oracle: the per-token quantizer's codes,
scales and zero points and the weights' code sums bit for bit; the product's
corrected int32 accumulator bit for bit and its bf16 output within one
rounding of the exact value, on every kernel configuration.
"""
import numpy as np
import pytest
import torch

import int8_scaled_gemm_amd as w8
import oracle
import workloads
from tests.gpu_util import DEV, bits, codes_to_dev, f32_bits, ulp

pytestmark = pytest.mark.gpu


def _x(M, K, seed, xtype="bf16"):
    x = workloads.activations(M, K, seed=seed)
    if M >= 4:
        x[1] = x[1].abs()        # non-negative row: lo = 0
        x[2] = -x[2].abs()       # non-positive row: hi = 0
        x[3] = 0                 # all-zero row: scale 1, codes -128
    if xtype == "fp16":
        x = x.to(torch.float16)
    elif xtype == "f32":
        x = x.float()
    return x


def _host(x):
    if x.dtype == torch.float32:
        return x.numpy(), "f32"
    return x.view(torch.int16).numpy().view(np.uint16), ("bf16" if x.dtype == torch.bfloat16 else "fp16")


@pytest.mark.parametrize("xtype", ["bf16", "fp16", "f32"])
@pytest.mark.parametrize("M,K", [(1, 4096), (16, 14336), (64, 4096), (300, 272), (5, 8192 + 16)])
def test_quant_per_token_azp_parity(M, K, xtype):
    x = _x(M, K, M + K, xtype)
    xh, xt = _host(x)
    q_ref, s_ref, z_ref = oracle.quant_per_token_azp(xh, xt)
    q, s, z = w8.w8a8_quant_per_token_azp(x.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(s.cpu().numpy()), f32_bits(s_ref))
    assert np.array_equal(z.cpu().numpy(), z_ref)
    assert np.array_equal(bits(q), q_ref)


@pytest.mark.parametrize("N,K", [(10240, 8192), (37, 160), (1000, 16)])
def test_colsum_parity(N, K):
    w = workloads.random_codes((N, K), "int8", seed=N).numpy()
    got = w8.w8a8_colsum(codes_to_dev(w, "int8"))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.colsum(w))


def test_colsum_strided():
    wbig = workloads.random_codes((40, 256 + 64), "int8", seed=3).numpy()
    w = np.ascontiguousarray(wbig[:, 32:32 + 256])
    got = w8.w8a8_colsum(codes_to_dev(wbig, "int8")[:, 32:32 + 256])
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.colsum(w))


SHAPES = [(1, 4096, 4096), (16, 28672, 1024), (64, 4096, 4096 + 16), (33, 1000, 1040),
          (64, 28672, 512), (300, 520, 272), (1024, 768, 2048), (65, 130, 128),
          (400 + 7, 3072 + 16, 1040), (1024 - 3, 4096, 144)]


@pytest.mark.parametrize("per_token", [True, False])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_scaled_mm_azp_parity(M, N, K, per_token):
    x = _x(M, K, 3 * M + N)
    if per_token:
        a, sa, z = oracle.quant_per_token_azp(_host(x)[0], "bf16")
    else:  # one scale and zero point for the tensor
        a, s1, z1 = oracle.quant_per_tensor_azp(_host(x)[0], "bf16")
        sa, z = np.array([s1], np.float32), np.array([z1], np.int32)
    w = workloads.weights(N, K, seed=N + K)
    b, sb = oracle.quant_per_token(w.view(torch.int16).numpy().view(np.uint16), "int8", xtype="bf16")
    ad, bd = codes_to_dev(a, "int8"), codes_to_dev(b, "int8")
    zd = torch.from_numpy(z).to(DEV)
    cs = w8.w8a8_colsum(bd)
    acc = w8.w8a8_scaled_mm_azp(ad, bd.t(), None, zd, cs, None, torch.int32)
    d = w8.w8a8_scaled_mm_azp(ad, bd.t(), torch.from_numpy(sa).to(DEV), zd, cs,
                              torch.from_numpy(sb).to(DEV), torch.bfloat16)
    torch.cuda.synchronize()
    print(f"M={M} N={N} K={K} {w8.w8a8_scaled_mm_kernel(M, N, K)}", flush=True)
    assert np.array_equal(acc.cpu().numpy(), oracle.scaled_mm_azp(a, b, None, z, None, "i32"))
    ref = oracle.scaled_mm_azp(a, b, sa, z, sb, "f64")
    got = d.float().cpu().numpy().astype(np.float64)
    assert (np.abs(got - ref) <= ulp(ref, "bf16")).all()
    exact = np.mean(bits(d) == oracle.scaled_mm_azp(a, b, sa, z, sb, "bf16"))
    assert exact > 0.99, exact


def test_scaled_mm_azp_without_zero_points_is_the_symmetric_product():
    M, N, K = 48, 640, 1024
    a = workloads.random_codes((M, K), "int8", seed=1).numpy()
    b = workloads.random_codes((N, K), "int8", seed=2).numpy()
    ad, bd = codes_to_dev(a, "int8"), codes_to_dev(b, "int8")
    sa = torch.full((M,), 0.01, device=DEV)
    sb = torch.full((N,), 0.002, device=DEV)
    d1 = w8.w8a8_scaled_mm_azp(ad, bd.t(), sa, None, None, sb, torch.bfloat16)
    d2 = w8.w8a8_scaled_mm(ad, bd.t(), sa, sb, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))


# ---------------------------------------------------------------- per tensor
@pytest.mark.parametrize("xtype", ["bf16", "fp16", "f32"])
@pytest.mark.parametrize("M,K", [(1, 16), (5, 272), (300, 1040), (64, 28672), (2048, 4096)])
def test_quant_per_tensor_azp_dynamic_parity(M, K, xtype):
    """Scale, zero point and codes bit for bit; (300, 1040) and up go through
    the three-kernel path whose partial ranges sit in the tail of the codes."""
    x = _x(M, K, 7 * M + K, xtype)
    xh, xt = _host(x)
    q_ref, s_ref, z_ref = oracle.quant_per_tensor_azp(xh, xt)
    q, s, z = w8.w8a8_quant_per_tensor_azp(x.to(DEV))
    torch.cuda.synchronize()
    assert f32_bits(s.cpu().numpy())[0] == f32_bits([s_ref])[0]
    assert int(z.item()) == z_ref
    assert np.array_equal(bits(q), q_ref)


@pytest.mark.parametrize("scale,azp", [(0.05, 3), (0.37, 127), (2.0, -128)])
def test_quant_per_tensor_azp_static_parity(scale, azp):
    M, K = 300, 1040
    x = _x(M, K, 11)
    xh, xt = _host(x)
    q_ref, _, _ = oracle.quant_per_tensor_azp(xh, xt, scale=scale, azp=azp, dynamic=False)
    sd = torch.tensor([scale], dtype=torch.float32, device=DEV)
    zd = torch.tensor([azp], dtype=torch.int32, device=DEV)
    q, _, _ = w8.w8a8_quant_per_tensor_azp(x.to(DEV), sd, zd, dynamic=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits(q), q_ref)
    q0, _, _ = w8.w8a8_quant_per_tensor_azp(x.to(DEV), dynamic=False)   # NULL: 1.0 and 0
    torch.cuda.synchronize()
    assert np.array_equal(bits(q0), oracle.quant_per_tensor_azp(xh, xt, dynamic=False)[0])


def test_quant_per_tensor_azp_strided_zero_and_empty():
    big = _x(400, 2048, 13)
    x = big[:, 512:512 + 1040]                      # a strided view, 416000 elements
    xh = np.ascontiguousarray(_host(big)[0][:, 512:512 + 1040])
    q_ref, s_ref, z_ref = oracle.quant_per_tensor_azp(xh, "bf16")
    qd = torch.zeros(400, 2048, dtype=torch.int8, device=DEV)
    q, s, z = w8.w8a8_quant_per_tensor_azp(x.to(DEV), q=qd[:, 16:16 + 1040])
    torch.cuda.synchronize()
    assert f32_bits(s.cpu().numpy())[0] == f32_bits([s_ref])[0] and int(z.item()) == z_ref
    assert np.array_equal(bits(q), q_ref)
    assert (qd[:, :16] == 0).all() and (qd[:, 16 + 1040:] == 0).all()   # nothing outside the view
    zero = torch.zeros(70, 1024, dtype=torch.bfloat16, device=DEV)
    q, s, z = w8.w8a8_quant_per_tensor_azp(zero)
    torch.cuda.synchronize()
    assert float(s.item()) == 1.0 and int(z.item()) == -128 and (q == -128).all()
    q, s, z = w8.w8a8_quant_per_tensor_azp(torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert float(s.item()) == 1.0 and int(z.item()) == -128
