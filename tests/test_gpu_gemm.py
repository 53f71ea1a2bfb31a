"""GPU parity of the scaled matrix multiply against the oracle.

D = a_scale (x) b_scale * (A_q . B_q) with B column-major ("[Kernel] Add w8a8
CUTLASS kernels": PR description list, misaligned-address report, and the
review's unit test on submatrices of A and B). int8 accumulators are
compared bit for bit; outputs within the tolerance in tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import int8_scaled_gemm_amd as w8
import oracle
import workloads
from tests.gpu_util import (DEV, TORCH_OF, assert_close_fraction, bits, check_scaled_mm,
                            check_scaled_mm_rows, codes_to_dev)

pytestmark = pytest.mark.gpu


def _quantized(M, N, K, qtype, seed):
    """Llama-like data quantised by the oracle: activations per token,
    weights per output channel."""
    x = workloads.activations(M, K, seed=seed)
    w = workloads.weights(N, K, seed=seed + 1)
    a, sa = oracle.quant_per_token(x.view(torch.int16).numpy().view(np.uint16), qtype, xtype="bf16")
    b, sb = oracle.quant_per_token(w.view(torch.int16).numpy().view(np.uint16), qtype, xtype="bf16")
    return a, sa, b, sb


def _run(a, b, qtype, sa, sb, otype):
    ad = codes_to_dev(a, qtype)
    bd = codes_to_dev(b, qtype)  # [N, K] row-major: its transpose is K x N column-major
    sad = None if sa is None else torch.from_numpy(np.asarray(sa, np.float32)).to(DEV)
    sbd = None if sb is None else torch.from_numpy(np.asarray(sb, np.float32)).to(DEV)
    out = w8.w8a8_scaled_mm(ad, bd.t(), sad, sbd, TORCH_OF[otype])
    torch.cuda.synchronize()
    return out


SHAPES = [
    # decode path (M <= 64): ragged N, K with a 16-byte tail past a 128-byte slice
    (1, 48, 4096), (1, 4096, 4096), (5, 100, 272), (16, 64, 128), (17, 200, 1040),
    (33, 1000, 144), (64, 6144, 512), (2, 16, 16),
    # tiled path: several tiles and ragged tails in M, N, K
    (65, 130, 128), (200, 384, 1040), (256, 256, 4096), (300, 520, 272), (777, 1111, 528),
    (1024, 768, 2048),
]


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_scaled_mm_parity(qtype, M, N, K):
    a, sa, b, sb = _quantized(M, N, K, qtype, seed=M + N + K)
    info = check_scaled_mm(_run(a, b, qtype, sa, sb, "bf16"), a, b, qtype, sa, sb, "bf16")
    assert info["exact_frac"] > 0.9, info


# Shapes that select each block tile of the tiled kernel (256x256, 256x128,
# 128x128 with 2 and 3 ring stages, 128x64, 64x64), with ragged M, N and K
# tails; checked on sampled rows.
TILE_SHAPES = [(4096 + 37, 4096 + 48, 384 + 16), (2048, 4096 + 16, 272), (512 - 5, 8320 - 16, 144),
               (200, 300, 1040), (1024 - 3, 4096, 144), (512, 4352 - 16, 400), (512 + 3, 6144 + 16, 272),
               (400 + 7, 3072 + 16, 1040)]


def test_tile_configs_are_the_ones_named():
    """The shapes above cover every tile configuration."""
    names = {w8.w8a8_scaled_mm_kernel(M, N, K) for M, N, K in TILE_SHAPES}
    assert names == {"gemm_tile_kernel<256x256>", "gemm_tile_kernel<256x128>",
                     "gemm_tile_kernel<128x128>", "gemm_tile_kernel<128x128,3x128>",
                     "gemm_tile_kernel<128x64,4x128>", "gemm_tile_kernel<64x64,4x128>"}, names


@pytest.mark.parametrize("otype", ["bf16", "fp16"])
@pytest.mark.parametrize("qtype", ["fp8", "int8"])
@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
def test_tile_configs_sampled_rows(qtype, M, N, K, otype):
    """Both 2-byte outputs of the prefill configuration (bf16 and fp16, "[Kernel]
    Add w8a8 CUTLASS kernels", PR description) on every block tile, whose
    epilogue rounds into LDS and stores whole rows."""
    a, sa, b, sb = _quantized(M, N, K, qtype, seed=M + 2 * N + K)
    got = _run(a, b, qtype, sa, sb, otype)
    rng = np.random.default_rng(M)
    rows = [0, 1, 15, 16, 255, 256, M - 1, M - 2] + list(rng.integers(0, M, 40))
    rows = [r for r in rows if r < M]
    info = check_scaled_mm_rows(got, rows, a, b, qtype, sa, sb, otype)
    assert_close_fraction(info, qtype, otype)


@pytest.mark.parametrize("qtype,otype", [("fp8", "f32"), ("int8", "f32"), ("int8", "i32")])
@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
def test_tile_configs_wide_outputs_sampled_rows(qtype, otype, M, N, K):
    """The 4-byte outputs (float32, and int8's raw int32 accumulator) on
    every block tile: their epilogue stores the fragments directly instead of
    restaging the tile through LDS."""
    a, sa, b, sb = _quantized(M, N, K, qtype, seed=M + 3 * N + K)
    if otype == "i32":
        sa = sb = None
    got = _run(a, b, qtype, sa, sb, otype)
    rng = np.random.default_rng(M + 1)
    rows = [0, 1, 31, 32, 127, 128, M - 1, M - 2] + list(rng.integers(0, M, 24))
    rows = [r for r in rows if r < M]
    check_scaled_mm_rows(got, rows, a, b, qtype, sa, sb, otype)


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
@pytest.mark.parametrize("otype", ["bf16", "fp16", "f32"])
@pytest.mark.parametrize("gran", ["tensor-tensor", "token-tensor", "tensor-channel", "none"])
@pytest.mark.parametrize("M", [8, 160])
def test_scale_granularities_and_outputs(qtype, otype, gran, M):
    N, K = 272, 384
    a, sa, b, sb = _quantized(M, N, K, qtype, seed=7 * M)
    if gran == "tensor-tensor":
        sa, sb = sa[:1], sb[:1]
    elif gran == "token-tensor":
        sb = sb[:1]
    elif gran == "tensor-channel":
        sa = sa[:1]
    else:
        sa = sb = None
        if otype == "fp16":  # raw accumulators overflow fp16
            sa = np.array([2.0 ** -10], np.float32)
    check_scaled_mm(_run(a, b, qtype, sa, sb, otype), a, b, qtype, sa, sb, otype)


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (16, 64, 128), (40, 100, 4096), (300, 300, 1024),
                                   (64, 28672 // 8, 4096)])
def test_int8_raw_accumulator_bit_exact(M, N, K):
    a = workloads.random_codes((M, K), "int8", seed=1).numpy()
    b = workloads.random_codes((N, K), "int8", seed=2).numpy()
    check_scaled_mm(_run(a, b, "int8", None, None, "i32"), a, b, "int8", None, None, "i32")


def test_int8_extreme_accumulator():
    """All 127 x all -127 over K = 28672: -462,450,688 in every element."""
    K = 28672
    a = np.full((3, K), 127, np.int8).view(np.uint8)
    b = np.full((20, K), -127, np.int8).view(np.uint8)
    out = _run(a, b, "int8", None, None, "i32").cpu().numpy()
    assert (out == -462450688).all()


def test_fp8_uniform_random_codes():
    """Every finite e4m3 code, including subnormals and +-448, in the operands."""
    M, N, K = 96, 160, 1024
    a = workloads.random_codes((M, K), "fp8", seed=3).numpy()
    b = workloads.random_codes((N, K), "fp8", seed=4).numpy()
    sa = np.float32(1e-4) * np.ones(M, np.float32)
    sb = np.linspace(1e-3, 2e-3, N).astype(np.float32)
    check_scaled_mm(_run(a, b, "fp8", sa, sb, "bf16"), a, b, "fp8", sa, sb, "bf16")
    a1 = a[:7]
    check_scaled_mm(_run(a1, b, "fp8", sa[:7], sb, "f32"), a1, b, "fp8", sa[:7], sb, "f32")


@pytest.mark.parametrize("M", [5, 100])
def test_fp8_codes_read_as_ocp_e4m3(M):
    """The matrix cores read the codes as OCP E4M3 (the e4m3fn of "Enable
    scaled FP8 (e4m3fn) KV cache on ROCm"), not as the FNUZ variant: against
    a weight code of 1.0 (0x38), 0x7E gives 448 (FNUZ: 224), 0x7F gives NaN
    (FNUZ: 240), a row of 0x80 gives 0 (FNUZ: NaN), 0x01 and 0x08 give 2^-9
    and 2^-6. M = 5 runs the decode kernel, M = 100 a tile kernel."""
    N, K = 64, 128
    a = np.zeros((M, K), np.uint8)
    a[0, 0] = 0x7E
    a[1, :] = 0x80
    a[2, 0] = 0x7F
    a[3, 0] = 0x01
    a[4, 0] = 0x08
    b = np.zeros((N, K), np.uint8)
    b[:, 0] = 0x38
    got = _run(a, b, "fp8", None, None, "f32").cpu().numpy()
    assert (got[0] == 448.0).all(), got[0, :4]
    assert (got[1] == 0.0).all(), got[1, :4]
    assert np.isnan(got[2]).all(), got[2, :4]
    assert (got[3] == 2.0 ** -9).all() and (got[4] == 2.0 ** -6).all()
    assert (got[5:] == 0.0).all()


def test_tiny_int8_case_end_to_end():
    """The tiny int8 case, every step on the GPU: per-tensor dynamic int8
    quantisation of A [16,128] and W [64,128], int32 accumulate, bf16 out."""
    x, w = workloads.tiny_int8_inputs()
    xh = x.view(torch.int16).numpy().view(np.uint16)
    wh = w.view(torch.int16).numpy().view(np.uint16)
    qa_ref, sa_ref = oracle.quant_per_tensor(xh, "int8", dynamic=True, xtype="bf16")
    qw_ref, sw_ref = oracle.quant_per_tensor(wh, "int8", dynamic=True, xtype="bf16")
    d_ref = oracle.scaled_mm(qa_ref, qw_ref, "int8", [sa_ref], [sw_ref], "bf16")
    qa, sa = w8.w8a8_quant_per_tensor(x.to(DEV), "int8", dynamic=True)
    qw, sw = w8.w8a8_quant_per_tensor(w.to(DEV), "int8", dynamic=True)
    d = w8.scaled_mm(qa, qw.t(), sa, sw, torch.bfloat16)
    raw = w8.w8a8_scaled_mm(qa, qw.t(), None, None, torch.int32)
    torch.cuda.synchronize()
    assert np.array_equal(bits(qa), qa_ref) and np.array_equal(bits(qw), qw_ref)
    assert np.array_equal(raw.cpu().numpy(), oracle.scaled_mm(qa_ref, qw_ref, "int8", None, None, "i32"))
    check_scaled_mm(d, qa_ref, qw_ref, "int8", [sa_ref], [sw_ref], "bf16")
    assert np.mean(bits(d) == d_ref) > 0.99


@pytest.mark.parametrize("col0", [24, 23])
@pytest.mark.parametrize("M,N", [(7, 96), (150, 96), (300, 4096 + 32), (3000, 4096)])
def test_submatrices_and_output_padding(M, N, col0):
    """A and B as column windows of wider matrices (leading dimensions larger
    than K), output into a window of a wider buffer: padding untouched. An
    odd first column leaves the output only 2-byte aligned (element stores).
    The shapes reach the decode kernel and the 64x64, 128x64 and 256x256
    tiles."""
    K = 256
    qtype = "fp8"
    abig = workloads.random_codes((M, K + 64), qtype, seed=5).numpy()
    bbig = workloads.random_codes((N + 8, K + 32), qtype, seed=6).numpy()
    a = np.ascontiguousarray(abig[:, 32:32 + K])
    b = np.ascontiguousarray(bbig[4:4 + N, 16:16 + K])
    sa = np.full(M, 1e-3, np.float32)
    sb = np.full(N, 2e-3, np.float32)
    ad = codes_to_dev(abig, qtype)[:, 32:32 + K]
    bd = codes_to_dev(bbig, qtype)[4:4 + N, 16:16 + K]
    obig = torch.full((M, N + 40), 7.0, dtype=torch.bfloat16, device=DEV)
    out = obig[:, col0:col0 + N]
    w8.w8a8_scaled_mm(ad, bd.t(), torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV),
                      torch.bfloat16, out=out)
    torch.cuda.synchronize()
    check_scaled_mm(out, a, b, qtype, sa, sb, "bf16")
    ob = obig.float().cpu().numpy()
    assert (ob[:, :col0] == 7.0).all() and (ob[:, col0 + N:] == 7.0).all()


def test_k_zero_writes_zeros_and_empty_is_noop():
    a = torch.empty(5, 0, dtype=torch.int8, device=DEV)
    b = torch.empty(0, 9, dtype=torch.int8, device=DEV)
    out = torch.full((5, 9), 3.0, dtype=torch.bfloat16, device=DEV)
    w8.w8a8_scaled_mm(a, b, None, None, torch.bfloat16, out=out)
    torch.cuda.synchronize()
    assert (out.float().cpu() == 0).all()
    e = w8.w8a8_scaled_mm(torch.empty(0, 64, dtype=torch.int8, device=DEV),
                          torch.empty(64, 32, dtype=torch.int8, device=DEV).t().contiguous().t(),
                          None, None)
    assert e.shape == (0, 32)


def test_wrong_b_layout_is_an_error_not_a_crash():
    """The misaligned-address report: B passed row-major K x N instead of
    column-major. Here it is refused before any launch."""
    a = torch.zeros(8, 4096, dtype=torch.float8_e4m3fn, device=DEV)
    b = torch.zeros(4096, 8192, dtype=torch.float8_e4m3fn, device=DEV)  # row-major K x N
    with pytest.raises(ValueError, match="column-major"):
        w8.w8a8_scaled_mm(a, b, None, None, torch.float16)
    lib = w8.load_library()
    st = lib.w8a8_scaled_mm(None, 0, 8192, a.data_ptr(), 4096, b.data_ptr(), 8192 - 8192, 1,
                            8, 8192, 4096, None, 1, None, 1, None)
    assert st == 3  # W8A8_ERR_LAYOUT


def test_graph_capture_and_replay():
    """The quantizers and the GEMM capture into a HIP graph (they allocate and
    synchronise nothing) and every replay matches the eager result."""
    M, N, K = 16, 512, 1024
    x = workloads.activations(M, K, seed=31).to(DEV)
    w = workloads.weights(N, K, seed=32).to(DEV)
    qw, sw = w8.w8a8_quant_per_token(w, "fp8")
    q_eager, s_eager = w8.w8a8_quant_per_token(x, "fp8")
    d_eager = w8.w8a8_scaled_mm(q_eager, qw.t(), s_eager, sw, torch.bfloat16)
    kv = workloads.kv_tensor(1, "k", shape=(64, 8, 128)).to(DEV)
    kq_eager, ks_eager = w8.kv_fp8_scaled_quant(kv)
    torch.cuda.synchronize()
    q = torch.empty_like(q_eager)
    s = torch.empty_like(s_eager)
    d = torch.empty_like(d_eager)
    kq = torch.empty_like(kq_eager)
    ks = torch.empty_like(ks_eager)
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            w8.w8a8_quant_per_token(x, "fp8", q=q, scales=s)
            w8.w8a8_scaled_mm(q, qw.t(), s, sw, torch.bfloat16, out=d)
            w8.kv_fp8_scaled_quant(kv, scale=ks, dynamic=True, q=kq)
    torch.cuda.synchronize()
    for i in range(3):
        d.zero_()
        kq.zero_()
        ks.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits_t(d), bits_t(d_eager)), i
        assert torch.equal(kq.view(torch.uint8), kq_eager.view(torch.uint8)), i
        assert torch.equal(ks, ks_eager), i
        # eager work between replays
        w8.w8a8_quant_per_token(kv.view(-1, 128)[:64], "int8")
        torch.cuda.synchronize()


def bits_t(t):
    return t.view(torch.int16)


# Shapes that select each decode configuration: 64-column blocks (N with at
# least 256 column tiles) and 16-column blocks, at M <= 16 and M <= 64, with
# ragged M, N and K tails and K past several ring stages.
DECODE_SHAPES = [(1, 4096, 4096), (5, 6144 + 16, 4096 + 16), (16, 4096, 14336), (17, 100, 272),
                 (33, 1000, 1040), (64, 4096, 4096), (64, 48, 144), (1, 16384 + 16, 1024 + 16),
                 (16, 16384, 2064), (17, 16384, 2048), (64, 16400, 272), (40, 20000, 512),
                 (3, 16336, 16), (64, 28672, 4096),
                 # long K on 129..256 sixteen-column workgroups: the long-stage variants
                 (64, 4096, 14336), (40, 3000 + 8, 8192 + 16),
                 # grids past one round of the deeper rings: the 2-stage variants
                 (1, 32768 + 16, 272), (48, 6144 + 16, 1040)]


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
@pytest.mark.parametrize("M,N,K", DECODE_SHAPES)
def test_decode_configs_parity(qtype, M, N, K):
    a, sa, b, sb = _quantized(M, N, K, qtype, seed=3 * M + N + K)
    got = _run(a, b, qtype, sa, sb, "bf16")
    info = check_scaled_mm(got, a, b, qtype, sa, sb, "bf16")
    assert info["exact_frac"] > 0.9, info
    if qtype == "int8":
        raw = _run(a, b, qtype, None, None, "i32")
        check_scaled_mm(raw, a, b, qtype, None, None, "i32")


def test_decode_configs_are_the_ones_named():
    """The shapes above cover every decode configuration."""
    names = {w8.w8a8_scaled_mm_kernel(M, N, K) for M, N, K in DECODE_SHAPES}
    assert names == {"gemm_decode_kernel<16x16>", "gemm_decode_kernel<16x16,4x512>",
                     "gemm_decode_kernel<16x64>", "gemm_decode_kernel<16x64,3x512>",
                     "gemm_decode_kernel<64x16>", "gemm_decode_kernel<64x16,4x256>",
                     "gemm_decode_kernel<64x64>", "gemm_decode_kernel<16x16,4x1K>",
                     "gemm_decode_kernel<16x64,1K>"}, names


# Split-K through a caller workspace: decode problems above 16 rows with a
# long K on weights too narrow to occupy the GPU. The 64-column kernel split
# (the Llama-3-8B down projection at 64 tokens, the widest N that still
# splits) and the 16-column ones on narrow weights (Llama-3-70B QKV on one of
# eight GPUs, 1280 rows; 2- and 3-slot rings; K of 4096 on at most 1024
# rows), with ragged N and K.
SPLITK_SHAPES = [(64, 4608, 14336), (40, 1000, 8192 + 16), (17, 300, 16384), (64, 16320, 8192),
                 (64, 10240, 8192), (64, 4096, 14336),
                 (33, 48, 9000 - 9000 % 16), (64, 1280, 8192), (33, 2000, 8192 + 16),
                 (64, 1024, 14336), (17, 768 + 16, 4096 + 16)]


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
@pytest.mark.parametrize("M,N,K", SPLITK_SHAPES)
def test_split_k_workspace_parity(qtype, M, N, K):
    need = w8.w8a8_scaled_mm_workspace_size(M, N, K)
    assert need > 0
    assert w8.w8a8_scaled_mm_kernel(M, N, K, workspace=True).endswith("splitk_reduce_kernel")
    a, sa, b, sb = _quantized(M, N, K, qtype, seed=5 * M + N + K)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ad, bd = codes_to_dev(a, qtype), codes_to_dev(b, qtype)
    sad = torch.from_numpy(np.asarray(sa, np.float32)).to(DEV)
    sbd = torch.from_numpy(np.asarray(sb, np.float32)).to(DEV)
    got = w8.w8a8_scaled_mm(ad, bd.t(), sad, sbd, torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    info = check_scaled_mm(got, a, b, qtype, sa, sb, "bf16")
    assert info["exact_frac"] > 0.9, info
    if qtype == "int8":  # the split sums are exact: raw accumulators bit for bit
        raw = w8.w8a8_scaled_mm(ad, bd.t(), None, None, torch.int32, workspace=ws)
        torch.cuda.synchronize()
        check_scaled_mm(raw, a, b, qtype, None, None, "i32")
        plain = w8.w8a8_scaled_mm(ad, bd.t(), sad, sbd, torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(plain.view(torch.int16), got.view(torch.int16))


def test_split_k_workspace_too_small_falls_back():
    """A workspace below the size needed is not used: the plain kernel runs."""
    M, N, K = 64, 4608, 14336
    a, sa, b, sb = _quantized(M, N, K, "int8", seed=9)
    need = w8.w8a8_scaled_mm_workspace_size(M, N, K)
    ad, bd = codes_to_dev(a, "int8"), codes_to_dev(b, "int8")
    small = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    raw = w8.w8a8_scaled_mm(ad, bd.t(), None, None, torch.int32, workspace=small)
    torch.cuda.synchronize()
    check_scaled_mm(raw, a, b, "int8", None, None, "i32")


def test_split_k_graph_replay():
    """The two split-K kernels capture into a HIP graph; replays match eager."""
    M, N, K = 64, 1024, 8192
    a, sa, b, sb = _quantized(M, N, K, "fp8", seed=21)
    ws = torch.empty(w8.w8a8_scaled_mm_workspace_size(M, N, K), dtype=torch.uint8, device=DEV)
    ad, bd = codes_to_dev(a, "fp8"), codes_to_dev(b, "fp8")
    sad = torch.from_numpy(sa).to(DEV)
    sbd = torch.from_numpy(sb).to(DEV)
    ref = w8.w8a8_scaled_mm(ad, bd.t(), sad, sbd, torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            w8.w8a8_scaled_mm(ad, bd.t(), sad, sbd, torch.bfloat16, out=out, workspace=ws)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
