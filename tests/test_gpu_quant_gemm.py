"""GPU parity of w8a8_quant_scaled_mm: dynamic per-token quantisation of the
activations followed by the scaled product ("[Kernel] Add w8a8 CUTLASS
kernels": per-token activation and per-channel weight scales; "[Kernel]
Support Fp8 Checkpoints (Dynamic + Static)": dynamic activation scales).

The codes and per-token scales it writes must equal the oracle's per-token
quantisation bit for bit, and the output must meet the scaled-product
tolerance against the oracle applied to those codes. One-token problems
(M == 1, K <= 15360, N < 16321) take the fused kernel; the others run the two
kernels.
"""
import numpy as np
import pytest
import torch

import int8_scaled_gemm_amd as w8
import oracle
import workloads
from tests.gpu_util import DEV, TORCH_OF, bits, check_scaled_mm, codes_to_dev, f32_bits

pytestmark = pytest.mark.gpu


def _x(M, K, seed, xtype):
    x = workloads.activations(M, K, seed=seed)
    if xtype == "fp16":
        x = x.to(torch.float16)
    elif xtype == "f32":
        x = x.float()
    return x


def _host(x):
    if x.dtype == torch.float32:
        return x.numpy(), None
    return x.view(torch.int16).numpy().view(np.uint16), ("bf16" if x.dtype == torch.bfloat16 else "fp16")


def _weights(N, K, qtype, seed):
    w = workloads.weights(N, K, seed=seed)
    return oracle.quant_per_token(w.view(torch.int16).numpy().view(np.uint16), qtype, xtype="bf16")


def _check(M, N, K, qtype, xtype="bf16", otype="bf16", gran="channel", seed=0, x_mul=1.0):
    x = _x(M, K, seed + 11, xtype) * x_mul  # a power of two: exact in every input type
    b, sb = _weights(N, K, qtype, seed + 12)
    if gran == "tensor":
        sb = sb[:1]
    elif gran == "none":
        sb = None
    xh, xt = _host(x)
    q_ref, sa_ref = oracle.quant_per_token(xh, qtype, xtype=xt)
    sbd = None if sb is None else torch.from_numpy(np.asarray(sb, np.float32)).to(DEV)
    q = torch.empty((M, K), dtype=w8.CODE_DTYPE[w8.QTYPE_OF[qtype]], device=DEV)
    sa = torch.empty(M, dtype=torch.float32, device=DEV)
    out = w8.w8a8_quant_scaled_mm(x.to(DEV), codes_to_dev(b, qtype).t(), sbd, qtype,
                                  TORCH_OF[otype], q=q, a_scales=sa)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(sa.cpu().numpy()), f32_bits(sa_ref)), "per-token scales differ"
    assert np.array_equal(bits(q), q_ref), "codes differ"
    info = check_scaled_mm(out, q_ref, b, qtype, sa_ref, sb, otype)
    if otype == "bf16":  # finer outputs show more of the fp8 summation order
        assert info.get("exact_frac", 1.0) > 0.9, info
    return info


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (1, 6144, 4096), (1, 100, 272), (1, 48, 16),
                                   (1, 4096, 14336), (1, 64, 15360), (1, 64, 15376),
                                   (1, 16400, 1040), (2, 300, 528), (16, 1000, 4096),
                                   (64, 640, 1024), (1, 28672 // 4, 4096), (1, 16320, 1024),
                                   (1, 16336, 1024)])
def test_quant_scaled_mm_parity(qtype, M, N, K):
    _check(M, N, K, qtype, seed=M + N + K)


@pytest.mark.parametrize("xtype", ["bf16", "fp16", "f32"])
@pytest.mark.parametrize("otype", ["bf16", "fp16", "f32"])
@pytest.mark.parametrize("gran", ["channel", "tensor", "none"])
def test_quant_scaled_mm_types_and_granularities(xtype, otype, gran):
    qtype = "fp8"
    # Without weight scales the output is sum_k x_k * b_k with weight codes up
    # to 448: N(0,1) activations with outliers reach past the fp16 range, so
    # that case takes activations 2^-8 as large (same codes, scale / 256).
    x_mul = 2.0 ** -8 if (otype == "fp16" and gran == "none") else 1.0
    _check(1, 272, 2048, qtype, xtype=xtype, otype=otype, gran=gran, seed=5, x_mul=x_mul)


def test_quant_scaled_mm_zero_row_and_saturation():
    """An all-zero token gets scale 1.0 and zero codes; a token with one huge
    value saturates nowhere (its scale follows the absmax)."""
    K, N = 4096, 256
    b, sb = _weights(N, K, "fp8", 3)
    sbd = torch.from_numpy(sb).to(DEV)
    bd = codes_to_dev(b, "fp8").t()
    x = torch.zeros(1, K, dtype=torch.bfloat16, device=DEV)
    q = torch.empty(1, K, dtype=torch.float8_e4m3fn, device=DEV)
    sa = torch.empty(1, dtype=torch.float32, device=DEV)
    out = w8.w8a8_quant_scaled_mm(x, bd, sbd, "fp8", q=q, a_scales=sa)
    torch.cuda.synchronize()
    assert float(sa[0]) == 1.0 and int(q.view(torch.uint8).sum()) == 0
    assert (out.float() == 0).all()
    x[0, 17] = 3.0e4
    _ = w8.w8a8_quant_scaled_mm(x, bd, sbd, "fp8", q=q, a_scales=sa)
    torch.cuda.synchronize()
    xh = x.cpu().view(torch.int16).numpy().view(np.uint16)
    q_ref, sa_ref = oracle.quant_per_token(xh, "fp8", xtype="bf16")
    assert np.array_equal(bits(q), q_ref)
    assert np.array_equal(f32_bits(sa.cpu().numpy()), f32_bits(sa_ref))


def test_quant_scaled_mm_empty_row():
    """K == 0 at one token (the fused kernel's shape, which would read the
    row's first elements): nothing is read, the scale is 1.0 and the output
    zero. The host-side choice is the two-call path."""
    assert w8.w8a8_quant_scaled_mm_kernel(1, 64, 0) == "quant_rows_kernel+scaled_mm"
    x = torch.empty(1, 0, dtype=torch.bfloat16, device=DEV)
    bd = torch.empty(64, 0, dtype=torch.float8_e4m3fn, device=DEV).t()
    q = torch.empty(1, 0, dtype=torch.float8_e4m3fn, device=DEV)
    sa = torch.full((1,), 7.0, dtype=torch.float32, device=DEV)
    out = torch.full((1, 64), 5.0, dtype=torch.bfloat16, device=DEV)
    w8.w8a8_quant_scaled_mm(x, bd, None, "fp8", out=out, q=q, a_scales=sa)
    torch.cuda.synchronize()
    assert float(sa[0]) == 1.0
    assert (out.float() == 0).all()


def test_quant_scaled_mm_graph_replay():
    """The fused call captures into a HIP graph; every replay matches eager."""
    M, N, K = 1, 4096, 4096
    x = _x(M, K, 41, "bf16").to(DEV)
    b, sb = _weights(N, K, "fp8", 42)
    bd = codes_to_dev(b, "fp8").t()
    sbd = torch.from_numpy(sb).to(DEV)
    ref = w8.w8a8_quant_scaled_mm(x, bd, sbd, "fp8")
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    q = torch.empty(M, K, dtype=torch.float8_e4m3fn, device=DEV)
    sa = torch.empty(M, dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            w8.w8a8_quant_scaled_mm(x, bd, sbd, "fp8", out=out, q=q, a_scales=sa)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
