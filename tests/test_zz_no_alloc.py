"""w8a8_scaled_mm_noalloc, the scaled product for callers that cannot
allocate: split K through the library's static device scratch. Called
through the C ABI; its output must equal w8a8_scaled_mm_ws's (same kernels,
same split order: bit for bit) and meet the parity bar against the oracle,
on two calls in a row, the second smaller, so the scratch's leftover
contents from the first call must not leak into the second.
"""
import ctypes

import numpy as np
import pytest
import torch

import int8_scaled_gemm_amd as w8
import oracle
import workloads
from tests.gpu_util import DEV, bits, check_scaled_mm, codes_to_dev

pytestmark = pytest.mark.gpu

Q = {"fp8": w8.Q_FP8, "int8": w8.Q_INT8}


def _problem(M, N, K, qtype, seed):
    x = workloads.activations(M, K, seed=seed)
    w = workloads.weights(N, K, seed=seed + 1)
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    a, sa = oracle.quant_per_token(u16(x), qtype, xtype="bf16")
    b, sb = oracle.quant_per_token(u16(w), qtype, xtype="bf16")
    return a, sa, b, sb


def _abi_call(name, out, a, b, sa, sb, qtype, extra=()):
    lib = w8.load_library()
    M, K = a.shape
    N = b.shape[0]
    st = torch.cuda.current_stream().cuda_stream
    fn = getattr(lib, name)
    status = fn(ctypes.c_void_p(out.data_ptr()), w8.DTYPE_OF[out.dtype], out.stride(0),
                ctypes.c_void_p(a.data_ptr()), a.stride(0), ctypes.c_void_p(b.data_ptr()),
                b.stride(0), Q[qtype], M, N, K,
                None if sa is None else ctypes.c_void_p(sa.data_ptr()),
                0 if sa is None else sa.numel(),
                None if sb is None else ctypes.c_void_p(sb.data_ptr()),
                0 if sb is None else sb.numel(), *extra, st)
    assert status == 0, (name, status, lib.w8a8_last_error().decode())


def _both(M, N, K, qtype, otype, seed):
    a, sa, b, sb = _problem(M, N, K, qtype, seed)
    ad, bd = codes_to_dev(a, qtype), codes_to_dev(b, qtype)
    if otype == torch.int32:
        sa = sb = None
    sad = None if sa is None else torch.from_numpy(sa).to(DEV)
    sbd = None if sb is None else torch.from_numpy(sb).to(DEV)
    got = torch.full((M, N), 7, dtype=otype, device=DEV)
    _abi_call("w8a8_scaled_mm_noalloc", got, ad, bd, sad, sbd, qtype)
    need = w8.w8a8_scaled_mm_workspace_size(M, N, K)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    ref = torch.full((M, N), 9, dtype=otype, device=DEV)
    _abi_call("w8a8_scaled_mm_ws", ref, ad, bd, sad, sbd, qtype,
              extra=(ctypes.c_void_p(ws.data_ptr()), ws.numel()))
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), bits(ref)), "no-alloc output differs from the workspace call"
    tag = {torch.bfloat16: "bf16", torch.int32: "i32"}[otype]
    info = check_scaled_mm(got, a, b, qtype, sa, sb, tag)
    if tag == "bf16":
        assert info["exact_frac"] > 0.9, info
    return need


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_no_alloc_matches_workspace_call_twice(qtype):
    print(f"no-alloc scaled_mm {qtype}: 64x4608x14336 then 40x1000x8208", flush=True)
    # first call: a split-K decode problem (Llama-3-8B down at 64 tokens, N cut)
    assert _both(64, 4608, 14336, qtype, torch.bfloat16, seed=1) > 0
    # second call, smaller: the scratch still holds the first call's sums
    assert _both(40, 1000, 8192 + 16, qtype, torch.bfloat16, seed=2) > 0
    if qtype == "int8":  # the raw accumulators, bit for bit
        assert _both(17, 300, 16384, qtype, torch.int32, seed=3) > 0


def test_no_alloc_unsplit_problems():
    """Problems that do not split use no scratch and run as w8a8_scaled_mm."""
    print("no-alloc scaled_mm: unsplit decode and tile problems", flush=True)
    assert _both(16, 4096, 4096, "fp8", torch.bfloat16, seed=4) == 0
    assert _both(300, 520, 272, "fp8", torch.bfloat16, seed=5) == 0


def test_no_alloc_validation_and_empty():
    lib = w8.load_library()
    x = torch.zeros(4, 128, dtype=torch.float8_e4m3fn, device=DEV)
    out = torch.zeros(4, 4, dtype=torch.bfloat16, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    # ldb < K: B is not column-major
    s = lib.w8a8_scaled_mm_noalloc(out.data_ptr(), w8.D_BF16, 4, x.data_ptr(), 128, x.data_ptr(), 64,
                                   w8.Q_FP8, 4, 4, 128, None, 0, None, 0, st)
    assert s == 3  # W8A8_ERR_LAYOUT
    s = lib.w8a8_scaled_mm_noalloc(out.data_ptr(), w8.D_BF16, 4, x.data_ptr(), 128, x.data_ptr(), 128,
                                   w8.Q_FP8, 0, 4, 128, None, 0, None, 0, st)
    assert s == 0  # M = 0: no-op
