"""The Python binding checks every caller-supplied buffer (outputs, codes,
scales, zero points, code sums, workspaces) for shape, element count, dtype
and layout before its pointer reaches the C ABI, which sees bare pointers
and cannot tell an undersized buffer from a good one. Each mistake below is
refused with a ValueError naming the argument; host tensors of the right
shape are refused too (GPU tensors only), so no call here reaches a kernel.
"""
import pytest
import torch

import int8_scaled_gemm_amd as w8

E4, I8, BF, F32, I32 = torch.float8_e4m3fn, torch.int8, torch.bfloat16, torch.float32, torch.int32
M, N, K = 4, 8, 128


def _raises(fn, *names):
    with pytest.raises(ValueError) as e:
        fn()
    msg = str(e.value)
    assert any(n in msg for n in names), msg


def _gpu_only(fn):
    _raises(fn, "GPU tensors only")


def test_scaled_mm_buffers():
    a = torch.zeros(M, K, dtype=E4)
    b = torch.zeros(N, K, dtype=E4).t()
    _raises(lambda: w8.w8a8_scaled_mm(a, b, None, None, out=torch.empty(M, N - 1, dtype=BF)), "out")
    _raises(lambda: w8.w8a8_scaled_mm(a, b, None, None, out=torch.empty(M - 1, N, dtype=BF)), "out")
    _raises(lambda: w8.w8a8_scaled_mm(a, b, None, None, out=torch.empty(M, N, dtype=torch.float64)), "out")
    _raises(lambda: w8.w8a8_scaled_mm(a, b, torch.ones(M + 1), None), "a_scales")
    _raises(lambda: w8.w8a8_scaled_mm(a, b, None, torch.ones(N - 1)), "b_scales")
    _raises(lambda: w8.w8a8_scaled_mm(a, b, None, None,
                                      workspace=torch.empty(64, 2, dtype=torch.uint8).t()), "workspace")
    _gpu_only(lambda: w8.w8a8_scaled_mm(a, b, torch.ones(M), torch.ones(N),
                                        out=torch.empty(M, N, dtype=BF)))
    _gpu_only(lambda: w8.scaled_mm(a, b, torch.ones(1), torch.ones(1)))


def test_quant_scaled_mm_buffers():
    x = torch.zeros(M, K, dtype=BF)
    b = torch.zeros(N, K, dtype=E4).t()
    _raises(lambda: w8.w8a8_quant_scaled_mm(x, b, None, out=torch.empty(M, N + 1, dtype=BF)), "out")
    _raises(lambda: w8.w8a8_quant_scaled_mm(x, b, None, q=torch.empty(M, K - 16, dtype=E4)), "q")
    _raises(lambda: w8.w8a8_quant_scaled_mm(x, b, None, q=torch.empty(M, K, dtype=I8)), "q")
    _raises(lambda: w8.w8a8_quant_scaled_mm(x, b, None, a_scales=torch.empty(M - 1)), "a_scales")
    _raises(lambda: w8.w8a8_quant_scaled_mm(x, b, None, a_scales=torch.empty(M, dtype=torch.float64)),
            "a_scales")
    _raises(lambda: w8.w8a8_quant_scaled_mm(x, b, torch.ones(N + 1)), "b_scales")
    _gpu_only(lambda: w8.w8a8_quant_scaled_mm(x, b, torch.ones(N)))


def test_quantizer_buffers():
    x = torch.zeros(M, K, dtype=BF)
    _raises(lambda: w8.w8a8_quant_per_token(x, "fp8", q=torch.empty(M, K - 16, dtype=E4)), "q")
    _raises(lambda: w8.w8a8_quant_per_token(x, "fp8", q=torch.empty(M, K, dtype=I8)), "q")
    _raises(lambda: w8.w8a8_quant_per_token(x, "int8", scales=torch.empty(M - 1)), "scales")
    _raises(lambda: w8.w8a8_quant_per_token(x, "int8", scales=torch.empty(2 * M)[::2]), "scales")
    _raises(lambda: w8.w8a8_quant_per_tensor(x, "fp8", q=torch.empty(M + 1, K, dtype=E4)), "q")
    _raises(lambda: w8.w8a8_quant_per_tensor(x, "fp8", scale=torch.empty(2), dynamic=True), "scale")
    _raises(lambda: w8.w8a8_quant_per_tensor(x, "fp8", scale=torch.empty(1, dtype=torch.float16)), "scale")
    _raises(lambda: w8.w8a8_quant_per_token(torch.zeros(M, K, dtype=I32), "fp8"), "x")
    _gpu_only(lambda: w8.w8a8_quant_per_token(x, "fp8"))
    _gpu_only(lambda: w8.quant_per_token(x, "int8"))
    _gpu_only(lambda: w8.quant_per_tensor(x, "fp8", dynamic=True))


def test_kv_buffers():
    x = torch.zeros(64, 8, 128, dtype=BF)
    q = torch.zeros(64, 8, 128, dtype=E4)
    _raises(lambda: w8.kv_fp8_scaled_quant(x, q=torch.empty(63, 8, 128, dtype=E4)), "q")
    _raises(lambda: w8.kv_fp8_scaled_quant(x, q=torch.empty(64, 8, 128, dtype=I8)), "q")
    _raises(lambda: w8.kv_fp8_scaled_quant(x, scale=torch.empty(2)), "scale")
    _raises(lambda: w8.kv_fp8_scaled_dequant(q, None, out=torch.empty(64, 8, 127, dtype=BF)), "out")
    _raises(lambda: w8.kv_fp8_scaled_dequant(q, None, out=torch.empty(128, 8, 64, dtype=BF)[::2]),
            "out")
    _raises(lambda: w8.kv_fp8_scaled_dequant(q, None, out=torch.empty(64, 8, 128, dtype=I32)), "out")
    _raises(lambda: w8.kv_fp8_scaled_dequant(q, torch.ones(3)), "scale")
    _gpu_only(lambda: w8.kv_quant(x))
    _gpu_only(lambda: w8.kv_dequant(q, torch.ones(1)))


def test_attention_buffers():
    qh = torch.zeros(2, 8, 128, dtype=BF)
    kc = torch.zeros(64, 2, 128, dtype=E4)
    starts = torch.tensor([0, 30, 64], dtype=I32)
    _raises(lambda: w8.kv_fp8_decode_attention(qh, kc, kc, starts, 64,
                                               out=torch.empty(2, 8, 64, dtype=BF)), "out")
    _raises(lambda: w8.kv_fp8_decode_attention(qh, kc, kc, starts, 64,
                                               out=torch.empty(2, 8, 128, dtype=torch.float16)), "out")
    _raises(lambda: w8.kv_fp8_decode_attention(qh, kc.to(BF), kc.to(BF), starts, 64), "k_cache")
    _raises(lambda: w8.kv_fp8_decode_attention(qh, kc, kc, starts, 64, k_scale=torch.ones(2)),
            "k_scale")
    _gpu_only(lambda: w8.kv_fp8_decode_attention(qh, kc, kc, starts, 64,
                                                 workspace=torch.empty(1 << 20, dtype=torch.uint8)))


def test_azp_buffers():
    x = torch.zeros(M, K, dtype=BF)
    a = torch.zeros(M, K, dtype=I8)
    b = torch.zeros(N, K, dtype=I8).t()
    _raises(lambda: w8.w8a8_quant_per_token_azp(x, q=torch.empty(M, K, dtype=E4)), "q")
    _raises(lambda: w8.w8a8_quant_per_token_azp(x, scales=torch.empty(M + 1)), "scales")
    _raises(lambda: w8.w8a8_quant_per_token_azp(x, azp=torch.empty(M, dtype=torch.int64)), "azp")
    _raises(lambda: w8.w8a8_colsum(torch.zeros(N, K, dtype=I8), out=torch.empty(N - 1, dtype=I32)),
            "out")
    z = torch.zeros(M, dtype=I32)
    cs = torch.zeros(N, dtype=I32)
    _raises(lambda: w8.w8a8_scaled_mm_azp(a, b, None, z, torch.zeros(N - 1, dtype=I32), None), "colsum")
    _raises(lambda: w8.w8a8_scaled_mm_azp(a, b, None, torch.zeros(M + 1, dtype=I32), cs, None), "azp")
    _raises(lambda: w8.w8a8_scaled_mm_azp(a, b, None, z, cs, None,
                                          out=torch.empty(M, N - 1, dtype=BF)), "out")
    _gpu_only(lambda: w8.w8a8_scaled_mm_azp(a, b, None, z, cs, None))


def test_merged_layer_buffers():
    sc = torch.ones(3)
    _raises(lambda: w8.w8a8_expand_shard_scales(sc, [4, 2, 2], out=torch.empty(7)), "out")
    w = torch.zeros(8, K, dtype=E4)
    _raises(lambda: w8.w8a8_requant_shared_scale(w, [4, 2, 2], sc, shared_scale=torch.empty(2)),
            "shared_scale")
    _gpu_only(lambda: w8.w8a8_expand_shard_scales(sc, [4, 2, 2]))
