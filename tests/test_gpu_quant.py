"""GPU parity of the quantizers: bit-exact codes and scales against the oracle.

Definitions: "Enable scaled FP8 (e4m3fn) KV cache on ROCm", "Scaling
semantics"; "[Kernel] Add w8a8 CUTLASS kernels", per-token / per-tensor
scales and the per_tensor_quantize recipe; "[Kernel] Support Fp8 Checkpoints
(Dynamic + Static)", static vs dynamic activation scales.
"""
import numpy as np
import pytest
import torch

import int8_scaled_gemm_amd as w8
import oracle
import workloads
from tests.gpu_util import DEV, bits, codes_to_dev, f32_bits, to_dev_bits

pytestmark = pytest.mark.gpu


def _x(M, K, seed, xtype="bf16"):
    x = workloads.activations(M, K, seed=seed)
    if xtype == "fp16":
        x = x.to(torch.float16)
    elif xtype == "f32":
        x = x.float()
    return x


def _host(x: torch.Tensor):
    """Oracle-side view of an input tensor: uint16 bits or float32."""
    if x.dtype == torch.float32:
        return x.numpy(), None
    return x.view(torch.int16).numpy().view(np.uint16), ("bf16" if x.dtype == torch.bfloat16 else "fp16")


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
@pytest.mark.parametrize("M,K", [(1, 4096), (16, 4096), (64, 14336), (37, 208), (3, 28672),
                                 (5, 40960), (200, 1024), (2, 16), (9, 8192), (4, 20000 - 20000 % 16)])
def test_per_token_bit_exact(qtype, M, K):
    x = _x(M, K, seed=M * 7 + K)
    xh, xt = _host(x)
    q_ref, s_ref = oracle.quant_per_token(xh, qtype, xtype=xt)
    q, s = w8.w8a8_quant_per_token(x.to(DEV), qtype)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(s.cpu().numpy()), f32_bits(s_ref))
    assert np.array_equal(bits(q), q_ref)


@pytest.mark.parametrize("xtype", ["fp16", "f32"])
@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_per_token_other_input_types(xtype, qtype):
    x = _x(24, 4096, seed=3, xtype=xtype)
    xh, xt = _host(x)
    q_ref, s_ref = oracle.quant_per_token(xh, qtype, xtype=xt)
    q, s = w8.w8a8_quant_per_token(x.to(DEV), qtype)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(s.cpu().numpy()), f32_bits(s_ref))
    assert np.array_equal(bits(q), q_ref)


def test_per_token_standalone_8192x4096():
    """The standalone dynamic per-token quantisation of [8192, 4096] bf16."""
    M, K = workloads.PER_TOKEN_STANDALONE
    x = workloads.activations(M, K, seed=0)
    xh, _ = _host(x)
    for qtype in ("fp8", "int8"):
        q_ref, s_ref = oracle.quant_per_token(xh, qtype, xtype="bf16")
        q, s = w8.w8a8_quant_per_token(x.to(DEV), qtype)
        torch.cuda.synchronize()
        assert np.array_equal(f32_bits(s.cpu().numpy()), f32_bits(s_ref))
        assert np.array_equal(bits(q), q_ref)


def test_per_token_submatrix_and_padding():
    """Strided input (a column window of a wider tensor) and strided output:
    the codes land in the window and the padding is untouched."""
    big = workloads.activations(40, 4096 + 64, seed=9).to(DEV)
    x = big[:, 32:32 + 4096]
    qbuf = torch.full((40, 4096 + 32), 0x55, dtype=torch.uint8, device=DEV)
    q = qbuf[:, 16:16 + 4096].view(torch.float8_e4m3fn)
    w8.w8a8_quant_per_token(x, "fp8", q=q)
    torch.cuda.synchronize()
    xh = x.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    q_ref, _ = oracle.quant_per_token(xh, "fp8", xtype="bf16")
    qb = qbuf.cpu().numpy()
    assert np.array_equal(qb[:, 16:16 + 4096], q_ref)
    assert (qb[:, :16] == 0x55).all() and (qb[:, 16 + 4096:] == 0x55).all()


def test_per_token_edges():
    # zero rows get scale 1.0 and code 0; K == 0 writes scales of 1.0
    x = torch.zeros(3, 256, dtype=torch.bfloat16, device=DEV)
    x[1, 7] = -2.5
    q, s = w8.w8a8_quant_per_token(x, "fp8")
    torch.cuda.synchronize()
    assert s.cpu().tolist() == [1.0, np.float32(2.5) / np.float32(448.0), 1.0]
    qb = bits(q)
    assert qb[1, 7] == 0xFE and int(qb.sum()) == 0xFE
    q0, s0 = w8.w8a8_quant_per_token(torch.empty(5, 0, dtype=torch.bfloat16, device=DEV), "int8")
    torch.cuda.synchronize()
    assert s0.cpu().tolist() == [1.0] * 5
    qe, se = w8.w8a8_quant_per_token(torch.empty(0, 64, dtype=torch.bfloat16, device=DEV), "fp8")
    assert qe.shape == (0, 64) and se.shape == (0,)


def _exhaustive_bf16():
    b = np.arange(65536, dtype=np.uint32)
    v = (b << 16).view(np.float32)
    keep = ~np.isnan(v)
    return b[keep].astype(np.uint16)


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_static_per_tensor_exhaustive_bf16(qtype):
    """Every non-NaN bf16 value, quantised with a set of static scales (some
    push results into e4m3 subnormals, some saturate everything)."""
    vals = _exhaustive_bf16()
    n = vals.size - vals.size % 256
    xh = vals[:n].reshape(-1, 256)
    x = to_dev_bits(xh, "bf16")
    for s in [1.0, 1.0 / 448, 0.0123, 3.7, 2.0 ** -20, 1e10, 7.0e-45, 0.3333333]:
        s32 = np.float32(s)
        q_ref, _ = oracle.quant_per_tensor(xh, qtype, scale=s32, xtype="bf16")
        st = torch.tensor([s32], dtype=torch.float32, device=DEV)
        q, _ = w8.w8a8_quant_per_tensor(x, qtype, scale=st, dynamic=False)
        torch.cuda.synchronize()
        assert np.array_equal(bits(q), q_ref), s


def test_static_per_tensor_random_scales():
    """Random scales over many binades: exercises the division for each."""
    x = workloads.activations(8, 4096, seed=11)
    xh, _ = _host(x)
    xd = x.to(DEV)
    rng = np.random.default_rng(1)
    for s in (2.0 ** rng.uniform(-40, 40, 24)).astype(np.float32):
        for qtype in ("fp8", "int8"):
            q_ref, _ = oracle.quant_per_tensor(xh, qtype, scale=s, xtype="bf16")
            q, _ = w8.w8a8_quant_per_tensor(xd, qtype, scale=torch.tensor([s], device=DEV))
            torch.cuda.synchronize()
            assert np.array_equal(bits(q), q_ref), (s, qtype)


def test_static_null_scale_means_one():
    x = workloads.activations(4, 512, seed=12)
    xh, _ = _host(x)
    q_ref, _ = oracle.quant_per_tensor(xh, "fp8", scale=None, xtype="bf16")
    q, s = w8.w8a8_quant_per_tensor(x.to(DEV), "fp8", scale=None, dynamic=False)
    torch.cuda.synchronize()
    assert s is None and np.array_equal(bits(q), q_ref)


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
@pytest.mark.parametrize("M,K", [(16, 128), (512, 4096), (513, 14336), (1, 16), (3000, 48)])
def test_dynamic_per_tensor_bit_exact(qtype, M, K):
    x = workloads.activations(M, K, seed=M + 3 * K)
    xh, _ = _host(x)
    q_ref, s_ref = oracle.quant_per_tensor(xh, qtype, dynamic=True, xtype="bf16")
    q, s = w8.w8a8_quant_per_tensor(x.to(DEV), qtype, dynamic=True)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(s.cpu().numpy()), f32_bits([s_ref]))
    assert np.array_equal(bits(q), q_ref)


def test_dynamic_per_tensor_reuses_scale_slot():
    """The scale slot is reset on every call: a second, smaller tensor gets
    its own absmax, not the first one's."""
    s = torch.empty(1, dtype=torch.float32, device=DEV)
    big = workloads.activations(64, 1024, seed=21).to(DEV) * 4
    small = workloads.activations(64, 1024, seed=22).to(DEV)
    w8.w8a8_quant_per_tensor(big, "fp8", scale=s, dynamic=True)
    q, _ = w8.w8a8_quant_per_tensor(small, "fp8", scale=s, dynamic=True)
    torch.cuda.synchronize()
    xh = small.cpu().view(torch.int16).numpy().view(np.uint16)
    q_ref, s_ref = oracle.quant_per_tensor(xh, "fp8", dynamic=True, xtype="bf16")
    assert f32_bits(s.cpu().numpy())[0] == f32_bits([s_ref])[0]
    assert np.array_equal(bits(q), q_ref)


@pytest.mark.parametrize("shape", [(32768, 8, 128), (100, 8, 128), (1, 1, 16)])
def test_kv_quant_dequant_bit_exact(shape):
    """Scaled fp8 KV cache, one layer's K tensor: dynamic per-tensor scale,
    codes, and the dequantised bf16 values, all bit-exact."""
    x = workloads.kv_tensor(0, "k", shape=shape)
    xh = x.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    q_ref, s_ref = oracle.kv_quant(xh, xtype="bf16")
    y_ref = oracle.kv_dequant(q_ref, s_ref, "bf16")
    q, s = w8.kv_fp8_scaled_quant(x.to(DEV))
    y = w8.kv_fp8_scaled_dequant(q, s, torch.bfloat16)
    torch.cuda.synchronize()
    assert f32_bits(s.cpu().numpy())[0] == f32_bits([s_ref])[0]
    assert np.array_equal(bits(q).reshape(-1), q_ref)
    assert np.array_equal(bits(y).reshape(-1), y_ref)


@pytest.mark.parametrize("otype", ["bf16", "fp16", "f32"])
def test_kv_dequant_all_codes(otype):
    """Every code (NaN included) through dequant with several scales."""
    codes = np.tile(np.arange(256, dtype=np.uint8), 4)
    qd = torch.from_numpy(codes).to(DEV).view(torch.float8_e4m3fn)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "f32": torch.float32}[otype]
    for s in [None, 1.0, 0.0123, 1e-3, 3.5e4, 2.0 ** -130]:
        st = None if s is None else torch.tensor([s], dtype=torch.float32, device=DEV)
        y = w8.kv_fp8_scaled_dequant(qd, st, tdt)
        torch.cuda.synchronize()
        y_ref = oracle.kv_dequant(codes, None if s is None else np.float32(s), otype)
        yb = bits(y)
        if otype == "f32":
            y_ref = y_ref.view(np.uint32)
        nan = (codes & 0x7F) == 0x7F
        assert np.array_equal(yb[~nan], y_ref[~nan]), s
        assert np.isnan(y.float().cpu().numpy()[nan]).all()


@pytest.mark.parametrize("otype", ["bf16", "fp16", "f32"])
def test_kv_dequant_ragged_length(otype):
    """Random valid codes, a length that ends part-way through a workgroup
    step (16 x 12347 codes), every output type: bit-exact."""
    n = 16 * 12347
    codes = workloads.random_codes((n,), "fp8", seed=31).numpy()
    qd = torch.from_numpy(codes).to(DEV).view(torch.float8_e4m3fn)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "f32": torch.float32}[otype]
    st = torch.tensor([0.0371], dtype=torch.float32, device=DEV)
    y = w8.kv_fp8_scaled_dequant(qd, st, tdt)
    torch.cuda.synchronize()
    y_ref = oracle.kv_dequant(codes, np.float32(0.0371), otype)
    if otype == "f32":
        y_ref = y_ref.view(np.uint32)
    assert np.array_equal(bits(y), y_ref)


def test_kv_static_scale_and_fp16_input():
    x = workloads.kv_tensor(3, "v", shape=(64, 8, 128)).to(torch.float16)
    xh = x.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    s = np.float32(0.01)
    q_ref, _ = oracle.kv_quant(xh, scale=s, dynamic=False, xtype="fp16")
    q, _ = w8.kv_fp8_scaled_quant(x.to(DEV), scale=torch.tensor([s], device=DEV), dynamic=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits(q).reshape(-1), q_ref)


def test_nan_inputs_follow_the_oracle():
    x = torch.tensor([[np.nan, 1.0, -np.nan, -3.0] * 4], dtype=torch.float32)
    for qtype in ("fp8", "int8"):
        q_ref, s_ref = oracle.quant_per_token(x.numpy(), qtype)
        q, s = w8.w8a8_quant_per_token(x.to(DEV), qtype)
        torch.cuda.synchronize()
        assert np.array_equal(bits(q), q_ref)
        assert f32_bits(s.cpu().numpy())[0] == f32_bits(s_ref)[0]
