"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (graph-free here, same library calls: the fused one-token kernel and the
split-K workspace where bench.py uses them), on sampled output rows the oracle
computes one by one.

Workloads: fp8 decode and prefill GEMMs at the Llama-3-8B layer shapes
(QKV 6144x4096, O 4096x4096, gate_up 28672x4096, down 4096x14336), the
int8 Llama-3-70B layer shapes (QKV 10240x8192, O 8192x8192, gate_up
57344x8192, down 8192x28672), with the quantizers that feed them, as the
"[Kernel] Add w8a8 CUTLASS kernels" PR lists (per-token / per-tensor
activations, per-channel weights) and "[Kernel] Support Fp8 Checkpoints"
describes (static calibrated vs dynamic activation scales). Inputs are drawn
on the device by torch's seeded generator and copied to the host for the
oracle; the weights' quantisation on the device is itself checked bit-exact
on sampled rows.
"""
import numpy as np
import pytest
import torch

import int8_scaled_gemm_amd as w8
import oracle
import workloads
from tests.gpu_util import DEV, TORCH_OF, assert_close_fraction, bits, check_scaled_mm_rows, f32_bits, ulp

pytestmark = pytest.mark.gpu


def _u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _sample_rows(M, seed, n=12):
    rng = np.random.default_rng(seed)
    return sorted(set([0, M - 1] + [int(r) for r in rng.integers(0, M, n)]))


def _weights_checked(N, K, qtype, seed):
    """Device weights, quantised per channel on the device; sampled rows of
    the codes and all scales checked against the oracle."""
    w = workloads.weights(N, K, seed=seed, device=DEV)
    wq, ws = w8.w8a8_quant_per_token(w, qtype)
    rows = _sample_rows(N, seed, 8)
    wh = _u16(w[rows])
    q_ref, s_ref = oracle.quant_per_token(wh, qtype, xtype="bf16")
    wq_h = bits(wq)
    assert np.array_equal(wq_h[rows], q_ref)
    assert np.array_equal(f32_bits(ws.cpu().numpy()[rows]), f32_bits(s_ref))
    return w, wq, ws, wq_h, ws.cpu().numpy()


def _check_layer(M, N, K, qtype, act, seed, otype="bf16"):
    w, wq, ws, wq_h, ws_h = _weights_checked(N, K, qtype, seed)
    del w
    x = workloads.activations(M, K, seed=seed + 500, device=DEV)
    # the route bench.py times: the fused one-token kernel where the library
    # fuses, else the quantizer and the product with a split-K workspace
    ws_bytes = w8.w8a8_scaled_mm_workspace_size(M, N, K)
    workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    if act == "per_token" and w8.w8a8_quant_scaled_mm_kernel(M, N, K) == "gemm_dynq_kernel":
        xq = torch.empty((M, K), dtype=wq.dtype, device=DEV)
        xs = torch.empty(M, dtype=torch.float32, device=DEV)
        out = w8.w8a8_quant_scaled_mm(x, wq.t(), ws, qtype, TORCH_OF[otype], q=xq, a_scales=xs)
    else:
        if act == "per_token":
            xq, xs = w8.w8a8_quant_per_token(x, qtype)
        else:
            calib = workloads.activations(workloads.CALIBRATION_ROWS, K,
                                          seed=workloads.CALIBRATION_SEED, device=DEV)
            _, xs = w8.w8a8_quant_per_tensor(calib, qtype, dynamic=True)
            xq, _ = w8.w8a8_quant_per_tensor(x, qtype, scale=xs)
        out = w8.w8a8_scaled_mm(xq, wq.t(), xs, ws, TORCH_OF[otype], workspace=workspace)
    torch.cuda.synchronize()
    rows = _sample_rows(M, seed + 1, 16 if M > 64 else M)
    # activation codes on the sampled rows against the oracle
    xh = _u16(x[rows])
    if act == "per_token":
        q_ref, s_ref = oracle.quant_per_token(xh, qtype, xtype="bf16")
        assert np.array_equal(f32_bits(xs.cpu().numpy()[rows]), f32_bits(s_ref))
    else:
        q_ref, _ = oracle.quant_per_tensor(xh, qtype, scale=np.float32(xs.item()), xtype="bf16")
    xq_h = bits(xq)
    assert np.array_equal(xq_h[rows], q_ref)
    sa = xs.cpu().numpy()
    info = check_scaled_mm_rows(out, rows, xq_h, wq_h, qtype, sa if sa.size > 1 else sa[:1], ws_h,
                                otype)
    assert_close_fraction(info, qtype, otype)
    return info


@pytest.mark.parametrize("name,N,K", workloads.LLAMA3_8B_LAYERS)
@pytest.mark.parametrize("M", workloads.FP8_DECODE_M)
def test_fp8_decode_full(M, name, N, K):
    print(f"fp8 decode M={M} {name} {N}x{K}", flush=True)
    _check_layer(M, N, K, "fp8", "per_token", seed=10 * M + N % 97)


@pytest.mark.parametrize("otype", ["bf16", "fp16"])
@pytest.mark.parametrize("name,N,K", workloads.LLAMA3_8B_LAYERS)
@pytest.mark.parametrize("M", workloads.FP8_PREFILL_M)
def test_fp8_prefill_full(M, name, N, K, otype):
    """The prefill configuration with both of its output types, bf16 and fp16."""
    print(f"fp8 prefill M={M} {name} {N}x{K} {otype}", flush=True)
    _check_layer(M, N, K, "fp8", "per_tensor_static", seed=11 * M + N % 89, otype=otype)


@pytest.mark.parametrize("name,N,K", workloads.LLAMA3_70B_LAYERS)
@pytest.mark.parametrize("M", workloads.INT8_70B_M)
def test_int8_70b_full(M, name, N, K):
    print(f"int8 70B M={M} {name} {N}x{K}", flush=True)
    _check_layer(M, N, K, "int8", "per_token", seed=13 * M + N % 83)


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("name,N,K", workloads.LLAMA3_70B_TP8_LAYERS)
@pytest.mark.parametrize("M", workloads.INT8_70B_M)
def test_70b_tp8_shard_full(M, name, N, K, qtype):
    """One GPU's share of the Llama-3-70B layers under 8-way tensor
    parallelism (QKV and gate_up split along N, O and down along K, the
    sharding of "Add async tensor parallelism for scaled mm"): the same calls
    at the shard's shapes, where narrow weights take the split-K plans."""
    print(f"{qtype} 70B TP8 shard M={M} {name} {N}x{K} "
          f"{w8.w8a8_scaled_mm_kernel(M, N, K, workspace=True)}", flush=True)
    _check_layer(M, N, K, qtype, "per_token", seed=17 * M + N % 79)


@pytest.mark.parametrize("name,N,K", workloads.LLAMA3_70B_LAYERS)
@pytest.mark.parametrize("M", workloads.INT8_70B_M)
def test_int8_azp_70b_full(M, name, N, K):
    """The int8_azp workload's route at its sizes: per-token asymmetric
    activations (scale and zero point per row), per-channel int8 weights and
    their code sums, the product with the zero-point term in the epilogue.
    Sampled rows of every step against the oracle: codes, scales, zero points
    and code sums bit for bit, the int32 sums exactly, the bf16 output within
    one ulp of the exact value and equal to its rounding almost everywhere."""
    print(f"int8 azp 70B M={M} {name} {N}x{K}", flush=True)
    seed = 17 * M + N % 89
    w, wq, ws, wq_h, ws_h = _weights_checked(N, K, "int8", seed)
    del w
    cs = w8.w8a8_colsum(wq)
    x = workloads.activations(M, K, seed=seed + 500, device=DEV)
    q, sa, z = w8.w8a8_quant_per_token_azp(x)
    out = w8.w8a8_scaled_mm_azp(q, wq.t(), sa, z, cs, ws, torch.bfloat16)
    acc = w8.w8a8_scaled_mm_azp(q, wq.t(), None, z, cs, None, torch.int32)
    torch.cuda.synchronize()
    wrows = _sample_rows(N, seed + 2, 8)
    assert np.array_equal(cs.cpu().numpy()[wrows], oracle.colsum(wq_h[wrows]))
    rows = _sample_rows(M, seed + 1, 16 if M > 64 else M)
    ri = torch.tensor(rows, device=DEV)
    q_ref, s_ref, z_ref = oracle.quant_per_token_azp(_u16(x[ri]), "bf16")
    q_h = bits(q[ri])
    sa_h, z_h = sa[ri].cpu().numpy(), z[ri].cpu().numpy()
    assert np.array_equal(q_h, q_ref)
    assert np.array_equal(f32_bits(sa_h), f32_bits(s_ref)) and np.array_equal(z_h, z_ref)
    assert np.array_equal(acc[ri].cpu().numpy(), oracle.scaled_mm_azp(q_h, wq_h, None, z_h, None, "i32"))
    ref = oracle.scaled_mm_azp(q_h, wq_h, sa_h, z_h, ws_h, "f64")
    got = out[ri].float().cpu().numpy().astype(np.float64)
    assert (np.abs(got - ref) <= ulp(ref, "bf16")).all()
    exact = np.mean(bits(out[ri]) == oracle.scaled_mm_azp(q_h, wq_h, sa_h, z_h, ws_h, "bf16"))
    assert exact > 0.99, exact


def test_kv_cache_layer_full_sampled():
    """One full 32-layer pass is what the bench times; every layer's K and V go
    through the same kernels, so two layers are checked in full."""
    for layer, which in [(0, "v"), (31, "k")]:
        x = workloads.kv_tensor(layer, which, device=DEV)
        q, s = w8.kv_fp8_scaled_quant(x)
        y = w8.kv_fp8_scaled_dequant(q, s, torch.bfloat16)
        torch.cuda.synchronize()
        xh = _u16(x).reshape(-1)
        q_ref, s_ref = oracle.kv_quant(xh, xtype="bf16")
        assert f32_bits(s.cpu().numpy())[0] == f32_bits([s_ref])[0]
        assert np.array_equal(bits(q).reshape(-1), q_ref)
        assert np.array_equal(bits(y).reshape(-1), oracle.kv_dequant(q_ref, s_ref, "bf16"))
