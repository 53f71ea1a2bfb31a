"""The C ABI library: it loads, exports every function include/w8a8.h
declares, and rejects bad arguments on the host with a status (never a
crash), as the review on "[Kernel] Add w8a8 CUTLASS kernels" asks of input
validation. No call here reaches the GPU: each one fails validation first.
"""
import ctypes
import os
import re
import subprocess

import pytest

import int8_scaled_gemm_amd as w8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")

# status codes (include/w8a8.h)
OK, INVALID, SHAPE, LAYOUT, ALIGN, DTYPE, UNSUP = 0, 1, 2, 3, 4, 5, 6
FAKE = 0x10000  # a 16-byte-aligned non-NULL address; never dereferenced by failing calls


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_\w+|kv_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return w8.load_library()


def test_exports_every_declared_function(lib):
    names = _declared()
    assert set(names) >= {"w8a8_quant_per_token", "w8a8_quant_per_tensor", "w8a8_scaled_mm",
                          "kv_fp8_scaled_quant", "kv_fp8_scaled_dequant",
                          "w8a8_status_string", "w8a8_last_error"}
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", w8.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)", out))
    assert set(names) <= exported


def test_header_compiles_as_c(tmp_path):
    c = tmp_path / "t.c"
    c.write_text('#include "w8a8.h"\nint main(void){return (int)w8a8_status_string(W8A8_OK)[0];}\n')
    subprocess.run(["gcc", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.dirname(HEADER), str(c)], check=True)


def test_status_strings(lib):
    for code, name in w8.STATUS_NAMES.items():
        assert lib.w8a8_status_string(code).decode() == name
    assert lib.w8a8_version().decode().startswith("libw8a8")


def mm(lib, out=FAKE, ot=0, ldo=64, a=FAKE, lda=128, b=FAKE, ldb=128, qt=1, M=16, N=64, K=128,
       sa=None, n_a=1, sb=None, n_b=1):
    return lib.w8a8_scaled_mm(out, ot, ldo, a, lda, b, ldb, qt, M, N, K, sa, n_a, sb, n_b, None)


def test_scaled_mm_validation(lib):
    assert mm(lib, ldb=64) == LAYOUT          # B not column-major (ldb < K)
    assert "column-major" in lib.w8a8_last_error().decode()
    assert mm(lib, lda=100) == LAYOUT
    assert mm(lib, ldo=32) == LAYOUT
    assert mm(lib, M=-1) == SHAPE
    assert mm(lib, K=120, lda=128, ldb=128) == ALIGN   # K not a multiple of 16
    assert mm(lib, lda=136) == ALIGN
    assert mm(lib, a=FAKE + 8) == ALIGN
    assert mm(lib, out=FAKE + 1) == ALIGN              # bf16 out must be 2-byte aligned
    assert mm(lib, qt=7) == DTYPE
    assert mm(lib, ot=9) == DTYPE
    # any int is rejected, negative and extreme ones too (the enums span int)
    for bad in (-1, 2, -2147483648, 2147483647):
        assert mm(lib, qt=bad) == DTYPE, bad
        assert mm(lib, ot=bad if bad != 2 else 4) == DTYPE, bad
    assert mm(lib, ot=3, qt=1) == DTYPE                 # raw int32 only for int8
    assert mm(lib, ot=3, qt=0, sa=FAKE) == INVALID      # raw accumulator takes no scales
    assert mm(lib, sa=FAKE, n_a=5) == SHAPE             # neither 1 nor M
    assert mm(lib, sb=FAKE, n_b=63) == SHAPE
    assert mm(lib, out=None) == INVALID
    assert mm(lib, a=None) == INVALID
    assert mm(lib, qt=0, K=131088, lda=131088, ldb=131088) == UNSUP
    assert mm(lib, M=2**31) == UNSUP
    # empty problems are accepted without touching memory
    assert mm(lib, M=0, out=None, a=None, b=None) == OK
    assert mm(lib, N=0, out=None, a=None, b=None) == OK


def test_quant_validation(lib):
    f = lib.w8a8_quant_per_token
    assert f(FAKE, 0, 4, 100, 112, FAKE, 1, 112, FAKE, None) == ALIGN
    assert f(FAKE, 0, 4, 128, 64, FAKE, 1, 128, FAKE, None) == LAYOUT
    assert f(FAKE, 5, 4, 128, 128, FAKE, 1, 128, FAKE, None) == DTYPE
    assert f(FAKE, 0, 4, 128, 128, FAKE, 3, 128, FAKE, None) == DTYPE
    assert f(FAKE, 0, 4, 128, 128, FAKE, 1, 128, None, None) == INVALID
    assert f(None, 0, 4, 128, 128, FAKE, 1, 128, FAKE, None) == INVALID
    assert f(FAKE, 0, -4, 128, 128, FAKE, 1, 128, FAKE, None) == SHAPE
    assert f(None, 0, 0, 128, 128, None, 1, 128, None, None) == OK
    g = lib.w8a8_quant_per_tensor
    assert g(FAKE, 0, 4, 128, 128, FAKE, 1, 128, None, 1, None) == INVALID  # dynamic needs a slot
    assert g(FAKE, 0, 4, 128, 128, FAKE, 1, 128, FAKE, 2, None) == INVALID
    assert g(FAKE + 4, 0, 4, 128, 128, FAKE, 1, 128, None, 0, None) == ALIGN
    k = lib.kv_fp8_scaled_quant
    assert k(FAKE, 0, 100, FAKE, FAKE, 1, None) == ALIGN
    assert k(FAKE, 0, 128, FAKE, None, 1, None) == INVALID
    assert k(FAKE, 0, -16, FAKE, FAKE, 1, None) == SHAPE
    d = lib.kv_fp8_scaled_dequant
    assert d(FAKE, 100, FAKE, FAKE, 0, None) == ALIGN
    assert d(FAKE, 128, FAKE, FAKE, 3, None) == DTYPE
    assert d(None, 128, FAKE, FAKE, 0, None) == INVALID
    assert d(None, 0, None, None, 0, None) == OK


def test_attention_validation(lib):
    ws = lib.kv_fp8_attention_workspace_size(2, 32, 8, 1000)
    # 2 x 8 waves per split: the rows per wave drop from 256 to the floor of 64 (16 splits)
    assert ws == 2 * 32 * 16 * 130 * 4  # (o, m, l) per head and split

    def call(out=FAKE, q=FAKE, B=2, Hq=32, Hkv=8, D=128, k=FAKE, v=FAKE, rows=100, st=FAKE,
             max_len=1000, ks=None, vs=None, sm=0.0, w=FAKE, wb=ws):
        return lib.kv_fp8_decode_attention(out, q, B, Hq, Hkv, D, k, v, rows, st, max_len, ks, vs,
                                           sm, w, wb, None)
    assert call(D=64) == UNSUP
    assert call(Hq=24) == UNSUP        # 3 query heads per KV head
    assert call(Hq=30) == SHAPE        # not a multiple of Hkv
    assert call(B=-1) == SHAPE
    assert call(wb=ws - 1) == INVALID
    assert call(w=None) == INVALID
    assert call(st=None) == INVALID
    assert call(k=None) == INVALID
    assert call(out=FAKE + 2) == ALIGN
    assert call(st=FAKE + 2) == ALIGN
    assert call(B=0, out=None, q=None, w=None) == OK  # nothing to do
    assert lib.kv_fp8_attention_workspace_size(-1, 32, 8, 10) == 0
    assert lib.kv_fp8_attention_workspace_size(2**40, 2**40, 8, 10) == 0  # no overflow
    assert call(Hq=65536 * 8, Hkv=65536) == UNSUP


def test_binding_layout_errors_are_python_errors():
    import torch
    # the binding refuses host tensors and wrong layouts before calling the library
    a = torch.zeros(4, 128, dtype=torch.float8_e4m3fn)
    with pytest.raises(ValueError):
        w8.w8a8_scaled_mm(a, a.t(), None, None)


def test_kernel_configuration_names(lib):
    """Host-only query of the kernel configuration a GEMM problem runs with."""
    name = lambda M, N, K: lib.w8a8_scaled_mm_kernel(M, N, K).decode()
    # deeper rings where the grid fits one round of their resident workgroups
    assert name(1, 4096, 4096) == "gemm_decode_kernel<16x16,4x512>"      # 256 groups
    assert name(1, 6144, 4096) == "gemm_decode_kernel<16x16,4x512>"      # 384
    assert name(1, 8192, 4096) == "gemm_decode_kernel<16x16>"            # 512
    assert name(64, 4096, 4096) == "gemm_decode_kernel<16x64,3x512>"     # 256
    assert name(64, 6144, 4096) == "gemm_decode_kernel<16x64>"           # 384
    assert name(1, 28672, 4096) == "gemm_decode_kernel<64x16,4x256>"     # 448 blocks
    assert name(1, 57344, 8192) == "gemm_decode_kernel<64x16>"           # 896
    assert name(17, 28672, 4096) == "gemm_decode_kernel<64x64>"
    assert name(16, 4096, 14336) == "gemm_decode_kernel<16x16,4x1K>"
    assert name(16, 6144, 14336) == "gemm_decode_kernel<16x16,4x512>"  # more workgroups than CUs
    assert name(1, 1280, 8192) == "gemm_decode_kernel<16x16,4x1K>"     # 80 groups, long K
    assert name(16, 2048, 8192) == "gemm_decode_kernel<16x16,4x1K>"    # 128 groups
    assert name(1, 768, 4096) == "gemm_decode_kernel<16x16,4x512>"     # K < 8192
    assert name(64, 1280, 8192) == "gemm_decode_kernel<16x64,3x512>"   # above 16 rows: 80 groups keep it
    assert name(8192, 28672, 4096) == "gemm_tile_kernel<256x256>"
    assert name(2048, 4096, 4096) == "gemm_tile_kernel<256x128>"
    # 128 x 64 where 192 to 256 of them fill one round, else 64 x 64
    assert name(512, 4096, 4096) == "gemm_tile_kernel<128x64,4x128>"     # 256 tiles
    assert name(300, 4096, 4096) == "gemm_tile_kernel<128x64,4x128>"     # 192
    assert name(128, 16384, 4096) == "gemm_tile_kernel<128x64,4x128>"    # 256
    assert name(400, 2048, 8192) == "gemm_tile_kernel<64x64,4x128>"      # 128 of 128 x 64; 224
    assert name(512, 4352, 4096) == "gemm_tile_kernel<128x128,3x128>"    # 136 of 128 x 128; 272 of 128 x 64
    assert name(512, 6144, 4096) == "gemm_tile_kernel<128x128,3x128>"    # 192 of 128 x 128
    assert name(512, 5120, 4096) == "gemm_tile_kernel<128x128,3x128>"    # 160
    assert name(512, 4608, 4096) == "gemm_tile_kernel<128x128,3x128>"    # 144
    assert name(512, 7168, 4096) == "gemm_tile_kernel<128x128,3x128>"    # 224
    # the large tiles from 160 tiles: one round of them beats more of smaller ones
    assert name(2048, 6144, 4096) == "gemm_tile_kernel<256x256>"   # 8 x 24 = 192 tiles
    assert name(512, 28672, 4096) == "gemm_tile_kernel<256x256>"   # 2 x 112 = 224 tiles
    assert name(2048, 5888, 4096) == "gemm_tile_kernel<256x256>"   # 8 x 23 = 184 tiles
    assert name(8192, 1280, 8192) == "gemm_tile_kernel<256x256>"   # 32 x 5 = 160 tiles
    assert name(4096, 1280, 4096) == "gemm_tile_kernel<256x128>"   # 80 of 256 x 256; 160
    assert name(512, 10240, 8192) == "gemm_tile_kernel<256x128>"   # 2 x 80 = 160 tiles
    assert name(1024 + 128, 4096, 4096) == "gemm_tile_kernel<256x128>"   # 5 x 32 = 160
    assert name(1024, 4096, 4096) == "gemm_tile_kernel<128x128,3x128>"   # 128 of 256 x 128; 256
    assert name(3072, 1280, 8192) == "gemm_tile_kernel<128x128,3x128>"   # 120 of 256 x 128; 240
    assert name(640, 6656, 4096) == "gemm_tile_kernel<256x128>"    # 156 of 256 x 128; 260 of 128 x 128
    assert name(512, 8320, 4096) == "gemm_tile_kernel<128x128>"    # 130 of 256 x 128; 260 of 128 x 128
    assert name(-1, 4, 4) == ""


def test_quant_scaled_mm_validation(lib):
    def f(out=FAKE, ot=0, ldo=64, x=FAKE, xt=0, ldx=128, b=FAKE, ldb=128, qt=1, M=1, N=64, K=128,
          sb=None, n_b=1, q=FAKE, ldq=128, sa=FAKE):
        return lib.w8a8_quant_scaled_mm(out, ot, ldo, x, xt, ldx, b, ldb, qt, M, N, K, sb, n_b, q,
                                        ldq, sa, None)
    assert f(ot=3, qt=0) == DTYPE          # the output is scaled: no raw accumulator
    assert f(sa=None) == INVALID           # the per-token scales are an output
    assert f(ldb=64) == LAYOUT             # B not column-major
    assert f(xt=9) == DTYPE
    assert f(xt=-1) == DTYPE
    assert f(qt=-2147483648) == DTYPE
    assert f(ldx=100) == LAYOUT
    assert f(sb=FAKE, n_b=7) == SHAPE
    assert f(x=None) == INVALID
    assert f(M=0, out=None, x=None, b=None, q=None, sa=None) == OK
    name = lambda M, N, K: lib.w8a8_quant_scaled_mm_kernel(M, N, K).decode()
    assert name(1, 4096, 14336) == "gemm_dynq_kernel"
    assert name(1, 4096, 15376) == "quant_rows_kernel+scaled_mm"
    assert name(2, 4096, 4096) == "quant_rows_kernel+scaled_mm"
    assert name(1, 28672, 4096) == "quant_rows_kernel+scaled_mm"  # wide weights: two kernels


def test_split_k_workspace_plan(lib):
    """Which problems split K with a workspace, and how much they need."""
    size = lib.w8a8_scaled_mm_workspace_size
    assert size(64, 8192, 14336) == 4 * 64 * 8192 * 4     # 128 column blocks: 4 splits
    assert size(17, 8192, 8192) == 4 * 17 * 8192 * 4
    assert size(40, 1000, 8192) == 4 * 40 * 1000 * 4      # few column blocks: at most 4 splits
    assert size(64, 1280, 8192) == 4 * 64 * 1280 * 4      # narrow: 16-column blocks split 4 ways
    assert size(64, 768, 4096) == 4 * 64 * 768 * 4        # at most 1024 rows: from K = 4096
    assert size(64, 1280, 4096) == 0                       # 1280 rows at K = 4096: no split
    assert size(16, 1280, 8192) == 0                       # at most 16 rows: no split
    assert size(64, 10240, 8192) == 3 * 64 * 10240 * 4    # 160 column blocks: 3 splits fill 512
    assert size(64, 16320, 8192) == 2 * 64 * 16320 * 4    # 255 column blocks: 2 splits
    assert size(64, 4096, 14336) == 4 * 64 * 4096 * 4     # Llama-3-8B down
    assert size(16, 4096, 14336) == 0                      # M <= 16: no split
    assert size(64, 4096, 4096) == 0                       # short K
    assert size(64, 28672, 8192) == 0                      # wide N
    assert size(65, 4096, 14336) == 0                      # the tiled path
    assert size(-1, 4096, 14336) == 0
    name = lambda M, N, K: lib.w8a8_scaled_mm_ws_kernel(M, N, K).decode()
    assert name(64, 8192, 14336) == "gemm_decode_kernel<64x64>+splitk_reduce_kernel"
    assert name(64, 4096, 4096) == lib.w8a8_scaled_mm_kernel(64, 4096, 4096).decode()
    assert name(64, 4096, 14336) == "gemm_decode_kernel<64x64>+splitk_reduce_kernel"
    assert name(64, 1280, 8192) == "gemm_decode_kernel<16x64>+splitk_reduce_kernel"          # 4 stages each
    assert name(64, 1024, 14336) == "gemm_decode_kernel<16x64,3x512>+splitk_reduce_kernel"   # 7 stages each
    assert name(64, 768, 4096) == "gemm_decode_kernel<16x64,3x512>+splitk_reduce_kernel"
    assert lib.w8a8_scaled_mm_kernel(64, 4096, 14336).decode() == "gemm_decode_kernel<16x64,1K>"
    ws = lib.w8a8_scaled_mm_ws
    args = (FAKE, 0, 64, FAKE, 128, FAKE, 128, 1, 16, 64, 128, None, 1, None, 1)
    assert ws(*args, FAKE + 16, 1024, None) == ALIGN       # 256-byte aligned workspace
    assert ws(*args, None, 1024, None) == INVALID
    assert ws(*args, FAKE, -1, None) == INVALID


def test_merged_layer_validation(lib):
    """Shard tables are checked on the host: counts, sizes, layout."""
    I64 = ctypes.c_int64

    def rows(*r):
        return (I64 * len(r))(*r)

    ex = lib.w8a8_expand_shard_scales
    assert ex(FAKE, rows(4, -1), 2, FAKE, None) == SHAPE
    assert "shard 1" in lib.w8a8_last_error().decode()
    assert ex(FAKE, rows(4), 0, FAKE, None) == SHAPE
    assert ex(FAKE, rows(*([1] * 65)), 65, FAKE, None) == UNSUP
    assert ex(FAKE, None, 1, FAKE, None) == INVALID
    assert ex(None, rows(3), 1, FAKE, None) == INVALID
    assert ex(FAKE + 2, rows(3), 1, FAKE, None) == ALIGN
    assert ex(None, rows(0, 0), 2, None, None) == OK           # no rows: nothing to write
    rq = lib.w8a8_requant_shared_scale
    r = rows(64, 64)
    assert rq(FAKE, 128, 5, 128, r, 2, FAKE, FAKE, 128, FAKE, None) == DTYPE
    assert rq(FAKE, 64, 1, 128, r, 2, FAKE, FAKE, 128, FAKE, None) == LAYOUT
    assert rq(FAKE, 136, 1, 120, r, 2, FAKE, FAKE, 136, FAKE, None) == ALIGN
    assert rq(FAKE + 16, 128, 1, 128, r, 2, FAKE, FAKE + 8, 128, FAKE, None) == ALIGN
    assert rq(FAKE, 128, 1, 128, r, 2, FAKE, FAKE, 128, None, None) == INVALID  # the shared scale is an output
    assert rq(None, 128, 1, 128, r, 2, FAKE, FAKE, 128, FAKE, None) == INVALID
    assert rq(FAKE, 128, 1, -16, r, 2, FAKE, FAKE, 128, FAKE, None) == SHAPE
    assert rq(FAKE, 128, 1, 128, rows(1, -2), 2, FAKE, FAKE, 128, FAKE, None) == SHAPE


def test_azp_validation(lib):
    """Asymmetric int8 calls: host-side checks."""
    qa = lib.w8a8_quant_per_token_azp
    assert qa(FAKE, 0, 4, 128, 128, FAKE, 128, FAKE, None, None) == INVALID   # azp is an output
    assert qa(FAKE, 5, 4, 128, 128, FAKE, 128, FAKE, FAKE, None) == DTYPE
    assert qa(FAKE, 0, 4, 100, 112, FAKE, 112, FAKE, FAKE, None) == ALIGN
    assert qa(None, 0, 0, 128, 128, None, 128, None, None, None) == OK
    cs = lib.w8a8_colsum
    assert cs(FAKE, 64, 8, 128, FAKE, None) == LAYOUT
    assert cs(FAKE, 136, 8, 120, FAKE, None) == ALIGN
    assert cs(FAKE, 128, 8, 128, None, None) == INVALID
    assert cs(None, 128, 0, 128, None, None) == OK
    mz = lib.w8a8_scaled_mm_azp

    def f(out=FAKE, ot=0, ldo=64, a=FAKE, lda=128, b=FAKE, ldb=128, M=16, N=64, K=128, sa=None,
          n_a=1, z=FAKE, n_z=1, cs=FAKE, sb=None, n_b=1):
        return mz(out, ot, ldo, a, lda, b, ldb, M, N, K, sa, n_a, z, n_z, cs, sb, n_b, None)
    assert f(n_z=3) == SHAPE                      # neither 1 nor M
    assert f(cs=None) == INVALID                  # zero points need the code sums
    assert f(z=FAKE + 2) == ALIGN
    assert f(K=65552, lda=65552, ldb=65552) == UNSUP
    assert f(ldb=64) == LAYOUT
    assert f(M=0, out=None, a=None, b=None) == OK


def test_per_tensor_azp_validation(lib):
    """Asymmetric int8 per tensor: host-side checks."""
    qt = lib.w8a8_quant_per_tensor_azp
    assert qt(FAKE, 0, 4, 128, 128, FAKE, 128, FAKE, FAKE, 2, None) == INVALID    # dynamic 0 or 1
    assert qt(FAKE, 0, 4, 128, 128, FAKE, 128, None, FAKE, 1, None) == INVALID    # dynamic: outputs
    assert qt(FAKE, 0, 4, 128, 128, FAKE, 128, FAKE, None, 1, None) == INVALID
    assert qt(FAKE, 5, 4, 128, 128, FAKE, 128, FAKE, FAKE, 1, None) == DTYPE
    assert qt(FAKE, 0, 4, 100, 112, FAKE, 112, FAKE, FAKE, 1, None) == ALIGN
    assert qt(FAKE, 0, 4, 128, 128, FAKE, 128, FAKE + 2, FAKE, 1, None) == ALIGN
    assert qt(FAKE, 0, 4, 128, 64, FAKE, 128, FAKE, FAKE, 1, None) == LAYOUT      # ldx < K
    assert qt(None, 0, 0, 128, 128, None, 128, None, None, 0, None) == OK          # static, empty


def test_paged_attention_validation(lib):
    """Paged attention: host-side checks of the block layout."""
    f = lib.kv_fp8_paged_decode_attention

    def call(B=2, Hq=8, Hkv=2, D=128, nblk=4, bs=16, tables=FAKE, stride=4, lens=FAKE, max_len=64,
             ws=FAKE, ws_bytes=1 << 20):
        return f(FAKE, FAKE, B, Hq, Hkv, D, FAKE, FAKE, nblk, bs, tables, stride, lens, max_len,
                 None, None, 0.0, ws, ws_bytes, None)
    assert call(bs=12) == UNSUP                  # not a power of two
    assert call(bs=2048) == UNSUP
    assert call(bs=0) == UNSUP
    assert call(stride=3) == SHAPE               # 3 blocks of 16 rows cannot cover 64
    assert call(nblk=-1) == SHAPE
    assert call(tables=None) == INVALID
    assert call(lens=None) == INVALID
    assert call(tables=FAKE + 2) == ALIGN
    assert call(D=64) == UNSUP
    assert call(ws_bytes=16) == INVALID           # workspace too small
    assert call(B=0) == OK
