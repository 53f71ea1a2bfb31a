"""GPU parity of the merged-layer calls ("[Kernel] Support Fp8 Checkpoints
(Dynamic + Static)": merged QKV / gate_up layers whose shards carry their own
weight scales) against the oracle: the per-channel expansion and the shared-
scale requantisation bit for bit, and one merged product with expanded scales
against the shards' separate per-tensor products.
"""
import numpy as np
import pytest
import torch

import int8_scaled_gemm_amd as w8
import oracle
import workloads
from tests.gpu_util import DEV, bits, check_scaled_mm, codes_to_dev, f32_bits

pytestmark = pytest.mark.gpu

LLAMA3_8B_QKV = [4096, 1024, 1024]      # q, k, v rows of the merged QKV weight
LLAMA3_8B_GATE_UP = [14336, 14336]


def _scales(S, seed):
    rng = np.random.default_rng(seed)
    return rng.uniform(2e-4, 4e-3, S).astype(np.float32)


@pytest.mark.parametrize("rows", [[100, 0, 37, 4096], [1], LLAMA3_8B_QKV, [0, 3]])
def test_expand_shard_scales_parity(rows):
    s = _scales(len(rows), sum(rows))
    got = w8.w8a8_expand_shard_scales(torch.from_numpy(s).to(DEV), rows)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(got.cpu().numpy()), f32_bits(oracle.expand_shard_scales(s, rows)))


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
@pytest.mark.parametrize("rows,K", [(LLAMA3_8B_QKV, 4096), ([5, 0, 300, 17], 272), ([64], 16),
                                    ([7, 9], 4096 + 16)])
def test_requant_shared_scale_parity(qtype, rows, K):
    N = sum(rows)
    w = workloads.random_codes((N, K), qtype, seed=N + K).numpy()
    s = _scales(len(rows), N)
    want, want_s = oracle.requant_shared_scale(w, qtype, rows, s)
    out, shared = w8.w8a8_requant_shared_scale(codes_to_dev(w, qtype), rows, torch.from_numpy(s).to(DEV))
    torch.cuda.synchronize()
    assert f32_bits(shared.cpu().numpy())[0] == f32_bits([want_s])[0]
    assert np.array_equal(bits(out), want)


def test_requant_gate_up_full_size_in_place():
    """Llama-3-8B gate_up (two 14336 x 4096 shards), rescaled in place."""
    rows, K = LLAMA3_8B_GATE_UP, 4096
    w = workloads.random_codes((sum(rows), K), "fp8", seed=11).numpy()
    s = _scales(2, 12)
    want, want_s = oracle.requant_shared_scale(w, "fp8", rows, s)
    wd = codes_to_dev(w, "fp8")
    out, shared = w8.w8a8_requant_shared_scale(wd, rows, torch.from_numpy(s).to(DEV), out=wd)
    torch.cuda.synchronize()
    assert out.data_ptr() == wd.data_ptr()
    assert f32_bits(shared.cpu().numpy())[0] == f32_bits([want_s])[0]
    assert np.array_equal(bits(wd), want)


def test_requant_strided_and_empty():
    """Row strides wider than K; no rows or K == 0 still write the shared scale."""
    rows, K = [40, 24], 256
    wbig = workloads.random_codes((64, K + 96), "fp8", seed=5).numpy()
    w = np.ascontiguousarray(wbig[:, 32:32 + K])
    s = _scales(2, 6)
    want, want_s = oracle.requant_shared_scale(w, "fp8", rows, s)
    wd = codes_to_dev(wbig, "fp8")[:, 32:32 + K]
    obig = torch.zeros(64, K + 48, dtype=torch.float8_e4m3fn, device=DEV)
    out = obig[:, 16:16 + K]
    w8.w8a8_requant_shared_scale(wd, rows, torch.from_numpy(s).to(DEV), out=out)
    torch.cuda.synchronize()
    ob = bits(obig)
    assert np.array_equal(ob[:, 16:16 + K], want)
    assert (ob[:, :16] == 0).all() and (ob[:, 16 + K:] == 0).all()
    for shape, r in (((0, 64), [0, 0]), ((32, 0), [16, 16])):
        e = torch.empty(shape, dtype=torch.float8_e4m3fn, device=DEV)
        _, sh = w8.w8a8_requant_shared_scale(e, r, torch.from_numpy(s).to(DEV))
        torch.cuda.synchronize()
        assert float(sh[0]) == float(np.max(s))


@pytest.mark.parametrize("M", [1, 16, 300])
def test_merged_product_equals_the_shards_products(M):
    """int8 (exact accumulation): one product over the merged QKV weight with
    expanded per-channel scales equals the three per-tensor products bit for
    bit; fp8: the merged product meets the scaled-product tolerance."""
    rows, K = [512, 128, 128], 1024
    for qtype in ("int8", "fp8"):
        a = workloads.random_codes((M, K), qtype, seed=M).numpy()
        w = workloads.random_codes((sum(rows), K), qtype, seed=M + 1).numpy()
        sa = np.float32(0.011)
        s = _scales(3, M + 2)
        sad = torch.tensor([sa], device=DEV)
        ad, wd = codes_to_dev(a, qtype), codes_to_dev(w, qtype)
        sb = w8.w8a8_expand_shard_scales(torch.from_numpy(s).to(DEV), rows)
        merged = w8.w8a8_scaled_mm(ad, wd.t(), sad, sb, torch.bfloat16)
        torch.cuda.synchronize()
        if qtype == "int8":
            n0 = 0
            for r, si in zip(rows, s):
                part = w8.w8a8_scaled_mm(ad, wd[n0:n0 + r].t(), sad, torch.tensor([si], device=DEV),
                                         torch.bfloat16)
                torch.cuda.synchronize()
                assert np.array_equal(bits(merged[:, n0:n0 + r]), bits(part))
                n0 += r
        check_scaled_mm(merged, a, w, qtype, [sa], oracle.expand_shard_scales(s, rows), "bf16")


def test_requantised_weight_in_the_product():
    """The shared-scale weight runs as a per-tensor product; its output meets
    the scaled-product tolerance against the oracle on the rescaled codes."""
    rows, K, M = LLAMA3_8B_QKV, 4096, 16
    w = workloads.random_codes((sum(rows), K), "fp8", seed=21).numpy()
    a = workloads.random_codes((M, K), "fp8", seed=22).numpy()
    s = _scales(3, 23)
    wq, ws = oracle.requant_shared_scale(w, "fp8", rows, s)
    out, shared = w8.w8a8_requant_shared_scale(codes_to_dev(w, "fp8"), rows, torch.from_numpy(s).to(DEV))
    d = w8.w8a8_scaled_mm(codes_to_dev(a, "fp8"), out.t(), torch.tensor([0.02], device=DEV), shared,
                          torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), wq)
    check_scaled_mm(d, a, wq, "fp8", [np.float32(0.02)], [ws], "bf16")
