"""Python binding of libw8a8, the MI355X (gfx950) w8a8 scaled-GEMM library.

Argument marshalling only: every step runs in the HIP kernels of
``libw8a8.so`` through its C ABI (``include/w8a8.h``). PyTorch supplies
device memory and the current stream. There is no fallback: without the
built library every call raises.

Functions carry the C names:

* ``w8a8_quant_per_token(x, qtype)`` -> ``(q, scales)``
* ``w8a8_quant_per_tensor(x, qtype, scale=None, dynamic=False)`` -> ``(q, scale)``
* ``w8a8_scaled_mm(a, b, a_scales, b_scales, out_dtype)`` -> ``out``
* ``kv_fp8_scaled_quant(x, scale=None, dynamic=True)`` -> ``(q, scale)``
* ``kv_fp8_scaled_dequant(q, scale, out_dtype)`` -> ``x``
* ``kv_fp8_decode_attention(q, k_cache, v_cache, seq_starts, max_seq_len, k_scale, v_scale)``
  -> ``out`` (decode attention reading the fp8 cache)

plus the short names ``quant_per_token(x, qtype)``, ``quant_per_tensor(x,
qtype, scale, dynamic)``, ``kv_quant(x)``, ``kv_dequant(q, scale)`` and
``scaled_mm(a, b, scale_a, scale_b, out_dtype)``, the call shape of
``cutlass_scaled_mm_dq`` in "[Kernel] Add w8a8 CUTLASS kernels" (the usage
snippet of its misaligned-address report), where ``b`` is a K x N
column-major view such as ``weight.t()``.

Codes are torch.int8 (int8) or torch.float8_e4m3fn (fp8) tensors; scales are
float32 device tensors.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw8a8.so")

# Enum values of include/w8a8.h.
W8A8_OK = 0
STATUS_NAMES = {0: "W8A8_OK", 1: "W8A8_ERR_INVALID_ARG", 2: "W8A8_ERR_SHAPE",
                3: "W8A8_ERR_LAYOUT", 4: "W8A8_ERR_ALIGNMENT", 5: "W8A8_ERR_DTYPE",
                6: "W8A8_ERR_UNSUPPORTED", 7: "W8A8_ERR_HIP"}
Q_INT8, Q_FP8 = 0, 1
D_BF16, D_FP16, D_F32, D_I32 = 0, 1, 2, 3

QTYPE_OF = {"int8": Q_INT8, "fp8": Q_FP8, torch.int8: Q_INT8, torch.float8_e4m3fn: Q_FP8}
CODE_DTYPE = {Q_INT8: torch.int8, Q_FP8: torch.float8_e4m3fn}
DTYPE_OF = {torch.bfloat16: D_BF16, torch.float16: D_FP16, torch.float32: D_F32,
            torch.int32: D_I32}

# C ABI signatures (name -> argtypes); every function returns w8a8_status.
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "w8a8_quant_per_token": [_P, _I, _I64, _I64, _I64, _P, _I, _I64, _P, _P],
    "w8a8_quant_per_tensor": [_P, _I, _I64, _I64, _I64, _P, _I, _I64, _P, _I, _P],
    "w8a8_scaled_mm": [_P, _I, _I64, _P, _I64, _P, _I64, _I, _I64, _I64, _I64, _P, _I64, _P,
                       _I64, _P],
    "w8a8_scaled_mm_ws": [_P, _I, _I64, _P, _I64, _P, _I64, _I, _I64, _I64, _I64, _P, _I64, _P,
                          _I64, _P, _I64, _P],
    "w8a8_scaled_mm_noalloc": [_P, _I, _I64, _P, _I64, _P, _I64, _I, _I64, _I64, _I64, _P, _I64,
                               _P, _I64, _P],
    "w8a8_quant_scaled_mm": [_P, _I, _I64, _P, _I, _I64, _P, _I64, _I, _I64, _I64, _I64, _P, _I64,
                             _P, _I64, _P, _P],
    "kv_fp8_scaled_quant": [_P, _I, _I64, _P, _P, _I, _P],
    "kv_fp8_scaled_dequant": [_P, _I64, _P, _P, _I, _P],
    "w8a8_quant_per_token_azp": [_P, _I, _I64, _I64, _I64, _P, _I64, _P, _P, _P],
    "w8a8_quant_per_tensor_azp": [_P, _I, _I64, _I64, _I64, _P, _I64, _P, _P, _I, _P],
    "w8a8_colsum": [_P, _I64, _I64, _I64, _P, _P],
    "w8a8_scaled_mm_azp": [_P, _I, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _I64, _P, _I64,
                           _P, _P, _I64, _P],
    "w8a8_expand_shard_scales": [_P, _P, _I64, _P, _P],
    "w8a8_requant_shared_scale": [_P, _I64, _I, _I64, _P, _I64, _P, _P, _I64, _P, _P],
    "kv_fp8_decode_attention": [_P, _P, _I64, _I64, _I64, _I64, _P, _P, _I64, _P, _I64, _P, _P,
                                ctypes.c_float, _P, _I64, _P],
    "kv_fp8_paged_decode_attention": [_P, _P, _I64, _I64, _I64, _I64, _P, _P, _I64, _I64, _P, _I64,
                                      _P, _I64, _P, _P, ctypes.c_float, _P, _I64, _P],
}


class W8A8Error(RuntimeError):
    """A libw8a8 call returned an error status."""

    def __init__(self, fn: str, status: int, message: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{fn}: {self.status_name}: {message}")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libw8a8.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libw8a8 is not built ({path} missing): run "
                          f"`python -m int8_scaled_gemm_amd.build` first")
    lib = ctypes.CDLL(path)
    for name, argtypes in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int
    lib.w8a8_status_string.argtypes = [ctypes.c_int]
    lib.w8a8_status_string.restype = ctypes.c_char_p
    lib.w8a8_last_error.argtypes = []
    lib.w8a8_last_error.restype = ctypes.c_char_p
    lib.w8a8_version.argtypes = []
    lib.w8a8_version.restype = ctypes.c_char_p
    lib.w8a8_scaled_mm_kernel.argtypes = [_I64, _I64, _I64]
    lib.w8a8_scaled_mm_kernel.restype = ctypes.c_char_p
    lib.w8a8_quant_scaled_mm_kernel.argtypes = [_I64, _I64, _I64]
    lib.w8a8_quant_scaled_mm_kernel.restype = ctypes.c_char_p
    lib.w8a8_scaled_mm_ws_kernel.argtypes = [_I64, _I64, _I64]
    lib.w8a8_scaled_mm_ws_kernel.restype = ctypes.c_char_p
    lib.w8a8_scaled_mm_workspace_size.argtypes = [_I64, _I64, _I64]
    lib.w8a8_scaled_mm_workspace_size.restype = ctypes.c_int64
    lib.kv_fp8_attention_workspace_size.argtypes = [_I64, _I64, _I64, _I64]
    lib.kv_fp8_attention_workspace_size.restype = ctypes.c_int64
    _lib = lib
    return lib


def _call(name: str, *args) -> None:
    lib = load_library()
    st = getattr(lib, name)(*args)
    if st != W8A8_OK:
        raise W8A8Error(name, st, lib.w8a8_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libw8a8 operates on GPU tensors only")


def _same_device(ref: torch.Tensor, *ts):
    for t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"libw8a8: tensors on {ref.device} and {t.device}")


def _want(t, what: str, *, shape=None, numel=None, dtypes=None, contiguous: bool = False):
    """Check a caller-supplied tensor before its pointer goes to the C ABI,
    which cannot see its size: an undersized or mistyped buffer would be
    written past its end by the kernels."""
    if t is None:
        return
    if dtypes is not None and t.dtype not in dtypes:
        names = ", ".join(str(d) for d in dtypes)
        raise ValueError(f"{what} must have dtype {names}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() not in ((numel,) if isinstance(numel, int) else numel):
        raise ValueError(f"{what} must have {numel} elements, got {t.numel()}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


_F32, _I32 = (torch.float32,), (torch.int32,)
_OUT_DTYPES = (torch.bfloat16, torch.float16, torch.float32, torch.int32)
_X_DTYPES = (torch.bfloat16, torch.float16, torch.float32)


def _rows(t: torch.Tensor, what: str):
    """(rows, cols, leading dimension) of a 2-D tensor with unit column stride."""
    if t.dim() != 2:
        raise ValueError(f"{what} must be 2-D, got shape {tuple(t.shape)}")
    if t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError(f"{what} must have unit stride along its last dimension")
    ld = t.stride(0) if t.size(0) > 1 else max(t.size(1), t.stride(0))
    return t.size(0), t.size(1), ld


def _qtype(qtype) -> int:
    if isinstance(qtype, int) and qtype in (Q_INT8, Q_FP8):
        return qtype
    try:
        return QTYPE_OF[qtype]
    except KeyError:
        raise ValueError(f"qtype must be 'int8' or 'fp8', got {qtype!r}") from None


def _dtype(dt) -> int:
    try:
        return DTYPE_OF[dt]
    except KeyError:
        raise ValueError(f"unsupported dtype {dt}") from None


# ------------------------------------------------------------------ quantizers
def w8a8_quant_per_token(x: torch.Tensor, qtype="fp8", q: torch.Tensor | None = None,
                         scales: torch.Tensor | None = None):
    """Dynamic per-token quantisation of x [M, K] -> (codes [M, K], scales fp32 [M])."""
    qt = _qtype(qtype)
    M, K, ldx = _rows(x, "x")
    _want(x, "x", dtypes=_X_DTYPES)
    _want(q, "q", shape=(M, K), dtypes=(CODE_DTYPE[qt],))
    _want(scales, "scales", numel=M, dtypes=_F32, contiguous=True)
    _check_cuda(x, q, scales)
    _same_device(x, q, scales)
    if q is None:
        q = torch.empty((M, K), dtype=CODE_DTYPE[qt], device=x.device)
    if scales is None:
        scales = torch.empty(M, dtype=torch.float32, device=x.device)
    _, _, ldq = _rows(q, "q")
    _call("w8a8_quant_per_token", _ptr(x), _dtype(x.dtype), M, K, ldx, _ptr(q), qt, ldq,
          _ptr(scales), _stream(x))
    return q, scales


def w8a8_quant_per_tensor(x: torch.Tensor, qtype="fp8", scale: torch.Tensor | None = None,
                          dynamic: bool = False, q: torch.Tensor | None = None):
    """Per-tensor quantisation. Static (dynamic=False) uses ``scale`` (None means 1.0);
    dynamic computes absmax/Qmax into ``scale`` (allocated when None)."""
    qt = _qtype(qtype)
    M, K, ldx = _rows(x, "x")
    _want(x, "x", dtypes=_X_DTYPES)
    _want(q, "q", shape=(M, K), dtypes=(CODE_DTYPE[qt],))
    _want(scale, "scale", numel=1, dtypes=_F32)
    _check_cuda(x, q, scale)
    _same_device(x, q, scale)
    if q is None:
        q = torch.empty((M, K), dtype=CODE_DTYPE[qt], device=x.device)
    if dynamic and scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _, _, ldq = _rows(q, "q")
    _call("w8a8_quant_per_tensor", _ptr(x), _dtype(x.dtype), M, K, ldx, _ptr(q), qt, ldq,
          _ptr(scale), 1 if dynamic else 0, _stream(x))
    return q, scale


def kv_fp8_scaled_quant(x: torch.Tensor, scale: torch.Tensor | None = None,
                        dynamic: bool = True, q: torch.Tensor | None = None):
    """Scaled fp8 KV-cache quantisation of a contiguous tensor (any shape)."""
    if not x.is_contiguous():
        raise ValueError("kv_fp8_scaled_quant needs a contiguous tensor")
    _want(x, "x", dtypes=_X_DTYPES)
    _want(q, "q", numel=x.numel(), dtypes=(torch.float8_e4m3fn,), contiguous=True)
    _want(scale, "scale", numel=1, dtypes=_F32)
    _check_cuda(x, q, scale)
    _same_device(x, q, scale)
    if q is None:
        q = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    if dynamic and scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _call("kv_fp8_scaled_quant", _ptr(x), _dtype(x.dtype), x.numel(), _ptr(q), _ptr(scale),
          1 if dynamic else 0, _stream(x))
    return q, scale


def kv_fp8_scaled_dequant(q: torch.Tensor, scale: torch.Tensor | None,
                          out_dtype=torch.bfloat16, out: torch.Tensor | None = None):
    """x' = dequant(q) * scale, rounded into out_dtype."""
    if not q.is_contiguous():
        raise ValueError("kv_fp8_scaled_dequant needs a contiguous tensor")
    _want(q, "q", dtypes=(torch.float8_e4m3fn, torch.uint8))
    _want(scale, "scale", numel=1, dtypes=_F32)
    _want(out, "out", numel=q.numel(), dtypes=_X_DTYPES, contiguous=True)
    _check_cuda(q, scale, out)
    _same_device(q, scale, out)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _call("kv_fp8_scaled_dequant", _ptr(q), q.numel(), _ptr(scale), _ptr(out),
          _dtype(out.dtype), _stream(q))
    return out


def kv_fp8_attention_workspace_size(B: int, Hq: int, Hkv: int, max_seq_len: int) -> int:
    return load_library().kv_fp8_attention_workspace_size(B, Hq, Hkv, max_seq_len)


def kv_fp8_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            seq_starts: torch.Tensor, max_seq_len: int,
                            k_scale: torch.Tensor | None = None,
                            v_scale: torch.Tensor | None = None, sm_scale: float = 0.0,
                            out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention over an e4m3fn KV cache: q [B, Hq, D] bf16, caches
    [rows, Hkv, D] e4m3fn, seq_starts [B + 1] int32 (sequence b owns cache
    rows seq_starts[b] .. seq_starts[b+1]-1) -> out [B, Hq, D] bf16."""
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"kv_fp8_decode_attention: {name} must be a contiguous 3-d tensor")
    if q.dtype != torch.bfloat16 or seq_starts.dtype != torch.int32:
        raise ValueError("kv_fp8_decode_attention: q must be bfloat16 and seq_starts int32")
    if k_cache.shape != v_cache.shape:
        raise ValueError("kv_fp8_decode_attention: k_cache and v_cache shapes differ")
    B, Hq, D = q.shape
    rows, Hkv, Dk = k_cache.shape
    if Dk != D or seq_starts.numel() != B + 1:
        raise ValueError("kv_fp8_decode_attention: head dimension or seq_starts length mismatch")
    _want(k_cache, "k_cache", dtypes=(torch.float8_e4m3fn, torch.uint8))
    _want(v_cache, "v_cache", dtypes=(torch.float8_e4m3fn, torch.uint8))
    _want(seq_starts, "seq_starts", contiguous=True)
    _want(k_scale, "k_scale", numel=1, dtypes=_F32)
    _want(v_scale, "v_scale", numel=1, dtypes=_F32)
    _want(out, "out", shape=(B, Hq, D), dtypes=(torch.bfloat16,), contiguous=True)
    _want(workspace, "workspace", contiguous=True)
    _check_cuda(q, k_cache, v_cache, seq_starts, k_scale, v_scale, out, workspace)
    _same_device(q, k_cache, v_cache, seq_starts, k_scale, v_scale, out, workspace)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    need = kv_fp8_attention_workspace_size(B, Hq, Hkv, max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"the call needs {need}")
    _call("kv_fp8_decode_attention", _ptr(out), _ptr(q), B, Hq, Hkv, D, _ptr(k_cache),
          _ptr(v_cache), rows, _ptr(seq_starts), max_seq_len, _ptr(k_scale), _ptr(v_scale),
          float(sm_scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
          _stream(q))
    return out


def kv_fp8_paged_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                  block_tables: torch.Tensor, seq_lens: torch.Tensor,
                                  max_seq_len: int, k_scale: torch.Tensor | None = None,
                                  v_scale: torch.Tensor | None = None, sm_scale: float = 0.0,
                                  out: torch.Tensor | None = None,
                                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention over a paged e4m3fn KV cache: q [B, Hq, D] bf16,
    caches [num_blocks, block_size, Hkv, D] e4m3fn, block_tables [B, n] int32
    (logical row t of sequence b lives in block block_tables[b, t // block_size]),
    seq_lens [B] int32 -> out [B, Hq, D] bf16."""
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"kv_fp8_paged_decode_attention: {name} must be a contiguous "
                             f"[num_blocks, block_size, Hkv, D] tensor")
    if q.dim() != 3 or not q.is_contiguous() or q.dtype != torch.bfloat16:
        raise ValueError("kv_fp8_paged_decode_attention: q must be a contiguous bfloat16 [B, Hq, D] tensor")
    if k_cache.shape != v_cache.shape:
        raise ValueError("kv_fp8_paged_decode_attention: k_cache and v_cache shapes differ")
    B, Hq, D = q.shape
    nblk, bs, Hkv, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("kv_fp8_paged_decode_attention: head dimension mismatch")
    if block_tables.dim() != 2 or block_tables.size(0) != B or block_tables.dtype != torch.int32:
        raise ValueError("block_tables must be an int32 [B, n] tensor")
    if block_tables.size(1) > 1 and block_tables.stride(1) != 1:
        raise ValueError("block_tables must have unit stride along its last dimension")
    _want(k_cache, "k_cache", dtypes=(torch.float8_e4m3fn, torch.uint8))
    _want(v_cache, "v_cache", dtypes=(torch.float8_e4m3fn, torch.uint8))
    _want(seq_lens, "seq_lens", numel=B, dtypes=_I32, contiguous=True)
    _want(k_scale, "k_scale", numel=1, dtypes=_F32)
    _want(v_scale, "v_scale", numel=1, dtypes=_F32)
    _want(out, "out", shape=(B, Hq, D), dtypes=(torch.bfloat16,), contiguous=True)
    _want(workspace, "workspace", contiguous=True)
    _check_cuda(q, k_cache, v_cache, block_tables, seq_lens, k_scale, v_scale, out, workspace)
    _same_device(q, k_cache, v_cache, block_tables, seq_lens, k_scale, v_scale, out, workspace)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    need = kv_fp8_attention_workspace_size(B, Hq, Hkv, max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"the call needs {need}")
    stride = block_tables.stride(0) if B > 1 else block_tables.size(1)
    _call("kv_fp8_paged_decode_attention", _ptr(out), _ptr(q), B, Hq, Hkv, D, _ptr(k_cache),
          _ptr(v_cache), nblk, bs, _ptr(block_tables), stride, _ptr(seq_lens), max_seq_len,
          _ptr(k_scale), _ptr(v_scale), float(sm_scale), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(q))
    return out


# ------------------------------------------------------- asymmetric int8 (azp)
def w8a8_quant_per_token_azp(x: torch.Tensor, q: torch.Tensor | None = None,
                             scales: torch.Tensor | None = None, azp: torch.Tensor | None = None):
    """Asymmetric per-token int8 quantisation of x [M, K] -> (codes int8
    [M, K], scales fp32 [M], zero points int32 [M]), x ~ (q - z) * s."""
    M, K, ldx = _rows(x, "x")
    _want(x, "x", dtypes=_X_DTYPES)
    _want(q, "q", shape=(M, K), dtypes=(torch.int8,))
    _want(scales, "scales", numel=M, dtypes=_F32, contiguous=True)
    _want(azp, "azp", numel=M, dtypes=_I32, contiguous=True)
    _check_cuda(x, q, scales, azp)
    _same_device(x, q, scales, azp)
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty(M, dtype=torch.float32, device=x.device)
    if azp is None:
        azp = torch.empty(M, dtype=torch.int32, device=x.device)
    _, _, ldq = _rows(q, "q")
    _call("w8a8_quant_per_token_azp", _ptr(x), _dtype(x.dtype), M, K, ldx, _ptr(q), ldq,
          _ptr(scales), _ptr(azp), _stream(x))
    return q, scales, azp


def w8a8_quant_per_tensor_azp(x: torch.Tensor, scale: torch.Tensor | None = None,
                              azp: torch.Tensor | None = None, dynamic: bool = True,
                              q: torch.Tensor | None = None):
    """Asymmetric per-tensor int8 quantisation of x [M, K] -> (codes int8
    [M, K], scale fp32 [1], zero point int32 [1]). dynamic: both from the
    tensor's range (allocated when None); static: the given ones (None: 1.0, 0)."""
    M, K, ldx = _rows(x, "x")
    _want(x, "x", dtypes=_X_DTYPES)
    _want(q, "q", shape=(M, K), dtypes=(torch.int8,))
    _want(scale, "scale", numel=1, dtypes=_F32)
    _want(azp, "azp", numel=1, dtypes=_I32)
    _check_cuda(x, q, scale, azp)
    _same_device(x, q, scale, azp)
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if dynamic and scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    if dynamic and azp is None:
        azp = torch.empty(1, dtype=torch.int32, device=x.device)
    _, _, ldq = _rows(q, "q")
    _call("w8a8_quant_per_tensor_azp", _ptr(x), _dtype(x.dtype), M, K, ldx, _ptr(q), ldq,
          _ptr(scale), _ptr(azp), 1 if dynamic else 0, _stream(x))
    return q, scale, azp


def w8a8_colsum(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Per-row sums of int8 weight codes w [N, K] (int32 [N])."""
    if w.dtype != torch.int8:
        raise ValueError("w8a8_colsum takes int8 codes")
    N, K, ldw = _rows(w, "w")
    _want(out, "out", numel=N, dtypes=_I32, contiguous=True)
    _check_cuda(w, out)
    _same_device(w, out)
    if out is None:
        out = torch.empty(N, dtype=torch.int32, device=w.device)
    _call("w8a8_colsum", _ptr(w), ldw, N, K, _ptr(out), _stream(w))
    return out


def w8a8_scaled_mm_azp(a: torch.Tensor, b: torch.Tensor, a_scales: torch.Tensor | None,
                       azp: torch.Tensor | None, colsum: torch.Tensor | None,
                       b_scales: torch.Tensor | None, out_dtype=torch.bfloat16,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """D = a_scales (x) b_scales * ((a - azp) @ b) for int8 codes; b and the
    scales as in w8a8_scaled_mm, azp int32 [1] or [M], colsum =
    w8a8_colsum(weight) for b = weight.t()."""
    if a.dtype != torch.int8 or b.dtype != torch.int8:
        raise ValueError("w8a8_scaled_mm_azp takes int8 codes")
    M, K, lda = _rows(a, "a")
    if b.dim() != 2 or b.size(0) != K:
        raise ValueError(f"b must be K x N with K={K}, got shape {tuple(b.shape)}")
    N = b.size(1)
    if b.size(0) > 1 and b.stride(0) != 1:
        raise ValueError("b must be column-major (K x N with stride(0) == 1), e.g. weight.t()")
    ldb = b.stride(1) if N > 1 else max(K, b.stride(1))
    _want(out, "out", shape=(M, N), dtypes=_OUT_DTYPES)
    _want(a_scales, "a_scales", numel=(1, M))
    _want(b_scales, "b_scales", numel=(1, N))
    _want(azp, "azp", numel=(1, M))
    if azp is not None:
        _want(colsum, "colsum", numel=N, dtypes=_I32, contiguous=True)
    _check_cuda(a, b, a_scales, azp, colsum, b_scales, out)
    _same_device(a, b, a_scales, azp, colsum, b_scales, out)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _, _, ldo = _rows(out, "out")
    sa = None if a_scales is None else a_scales.reshape(-1)
    sb = None if b_scales is None else b_scales.reshape(-1)
    z = None if azp is None else azp.reshape(-1)
    for t, what, dt in ((sa, "a_scales", torch.float32), (sb, "b_scales", torch.float32),
                        (z, "azp", torch.int32), (colsum, "colsum", torch.int32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise ValueError(f"{what} must be a contiguous {dt} tensor")
    _call("w8a8_scaled_mm_azp", _ptr(out), _dtype(out.dtype), ldo, _ptr(a), lda, _ptr(b), ldb,
          M, N, K, _ptr(sa), 0 if sa is None else sa.numel(), _ptr(z), 0 if z is None else z.numel(),
          _ptr(colsum), _ptr(sb), 0 if sb is None else sb.numel(), _stream(a))
    return out


# -------------------------------------------------------------- merged layers
def _shard_rows(shard_rows):
    rows = (ctypes.c_int64 * max(len(shard_rows), 1))(*[int(r) for r in shard_rows])
    return rows, len(shard_rows), sum(int(r) for r in shard_rows)


def w8a8_expand_shard_scales(shard_scales: torch.Tensor, shard_rows,
                             out: torch.Tensor | None = None) -> torch.Tensor:
    """Per-channel weight scales of a merged layer: shard i's scale on each of
    its shard_rows[i] rows (float32 [N] on the device)."""
    rows, S, N = _shard_rows(shard_rows)
    if shard_scales.dtype != torch.float32 or not shard_scales.is_contiguous() or shard_scales.numel() != S:
        raise ValueError("shard_scales must be a contiguous float32 tensor with one entry per shard")
    _want(out, "out", numel=N, dtypes=_F32, contiguous=True)
    _check_cuda(shard_scales, out)
    _same_device(shard_scales, out)
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=shard_scales.device)
    _call("w8a8_expand_shard_scales", _ptr(shard_scales), rows, S, _ptr(out), _stream(shard_scales))
    return out


def w8a8_requant_shared_scale(w: torch.Tensor, shard_rows, shard_scales: torch.Tensor,
                              out: torch.Tensor | None = None,
                              shared_scale: torch.Tensor | None = None):
    """Codes of a merged weight [N, K] (float8_e4m3fn or int8) rescaled to one
    shared scale max(shard_scales). out may be w (in place). Returns
    (out, shared_scale) with shared_scale a float32 [1] device tensor."""
    qt = _qtype(w.dtype)
    N, K, ldw = _rows(w, "w")
    rows, S, n = _shard_rows(shard_rows)
    if n != N:
        raise ValueError(f"shard_rows add up to {n}, w has {N} rows")
    if shard_scales.dtype != torch.float32 or not shard_scales.is_contiguous() or shard_scales.numel() != S:
        raise ValueError("shard_scales must be a contiguous float32 tensor with one entry per shard")
    if out is None:
        out = torch.empty((N, K), dtype=w.dtype, device=w.device)
    if out.dtype != w.dtype or tuple(out.shape) != (N, K):
        raise ValueError("out must match w in dtype and shape")
    _want(shared_scale, "shared_scale", numel=1, dtypes=_F32)
    _check_cuda(w, shard_scales, out, shared_scale)
    _same_device(w, shard_scales, out, shared_scale)
    _, _, ldo = _rows(out, "out")
    if K == 0:
        ldw = ldo = 0  # no columns: the strides are never used
    if shared_scale is None:
        shared_scale = torch.empty(1, dtype=torch.float32, device=w.device)
    _call("w8a8_requant_shared_scale", _ptr(w), ldw, qt, K, rows, S, _ptr(shard_scales), _ptr(out),
          ldo, _ptr(shared_scale), _stream(w))
    return out, shared_scale


# ---------------------------------------------------------------------- GEMM
def w8a8_scaled_mm_workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of workspace with which w8a8_scaled_mm_ws splits K (0: none)."""
    return int(load_library().w8a8_scaled_mm_workspace_size(M, N, K))


def w8a8_scaled_mm(a: torch.Tensor, b: torch.Tensor, a_scales: torch.Tensor | None,
                   b_scales: torch.Tensor | None, out_dtype=torch.bfloat16,
                   out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """D = a_scales (x) b_scales * (a @ b).

    a: codes [M, K] with unit column stride. b: codes K x N, COLUMN-major
    (b.stride(0) == 1), e.g. ``weight.t()`` for a row-major [N, K] weight.
    a_scales: fp32 [1] or [M] (or [M, 1]); b_scales: fp32 [1] or [N] (or [1, N]).
    None means 1.0. out_dtype: bfloat16, float16, float32, or int32 (the raw
    int8 accumulator, scales must be None).
    workspace: optional uint8 device tensor; with at least
    w8a8_scaled_mm_workspace_size(M, N, K) bytes the call goes through
    w8a8_scaled_mm_ws and may split K. "static": w8a8_scaled_mm_noalloc
    (split K through the library's static device scratch).
    """
    qt = _qtype(a.dtype)
    if b.dtype != a.dtype:
        raise ValueError(f"a and b must share a code type, got {a.dtype} and {b.dtype}")
    M, K, lda = _rows(a, "a")
    if b.dim() != 2 or b.size(0) != K:
        raise ValueError(f"b must be K x N with K={K}, got shape {tuple(b.shape)}")
    N = b.size(1)
    if b.size(0) > 1 and b.stride(0) != 1:
        raise ValueError("b must be column-major (K x N with stride(0) == 1), e.g. weight.t()")
    ldb = b.stride(1) if N > 1 else max(K, b.stride(1))
    _want(out, "out", shape=(M, N), dtypes=_OUT_DTYPES)
    _want(a_scales, "a_scales", numel=(1, M))
    _want(b_scales, "b_scales", numel=(1, N))
    ws_t = workspace if isinstance(workspace, torch.Tensor) else None
    if workspace is not None and ws_t is None and workspace != "static":
        raise ValueError("workspace must be a device tensor, None, or 'static'")
    _want(ws_t, "workspace", contiguous=True)
    _check_cuda(a, b, a_scales, b_scales, out, ws_t)
    _same_device(a, b, a_scales, b_scales, out, ws_t)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _, _, ldo = _rows(out, "out")
    sa = None if a_scales is None else a_scales.reshape(-1)
    sb = None if b_scales is None else b_scales.reshape(-1)
    for s, what in ((sa, "a_scales"), (sb, "b_scales")):
        if s is not None and (s.dtype != torch.float32 or not s.is_contiguous()):
            raise ValueError(f"{what} must be a contiguous float32 tensor")
    args = (_ptr(out), _dtype(out.dtype), ldo, _ptr(a), lda, _ptr(b), ldb, qt, M, N, K,
            _ptr(sa), 0 if sa is None else sa.numel(), _ptr(sb),
            0 if sb is None else sb.numel())
    if workspace == "static":
        _call("w8a8_scaled_mm_noalloc", *args, _stream(a))
    elif workspace is None:
        _call("w8a8_scaled_mm", *args, _stream(a))
    else:
        _call("w8a8_scaled_mm_ws", *args, _ptr(workspace),
              workspace.numel() * workspace.element_size(), _stream(a))
    return out


def w8a8_scaled_mm_noalloc(a: torch.Tensor, b: torch.Tensor, a_scales: torch.Tensor | None,
                           b_scales: torch.Tensor | None, out_dtype=torch.bfloat16,
                           out: torch.Tensor | None = None) -> torch.Tensor:
    """w8a8_scaled_mm with split K through the library's static device
    scratch instead of a workspace (the C call allocates nothing; pass `out`
    to allocate nothing here either). Calls that overlap on one GPU race on
    the scratch."""
    return w8a8_scaled_mm(a, b, a_scales, b_scales, out_dtype, out, workspace="static")


def w8a8_quant_scaled_mm(x: torch.Tensor, b: torch.Tensor, b_scales: torch.Tensor | None,
                         qtype="fp8", out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                         q: torch.Tensor | None = None,
                         a_scales: torch.Tensor | None = None) -> torch.Tensor:
    """Dynamic per-token quantisation of x, then D = a_scales (x) b_scales * (q @ b).

    x: bf16/fp16/fp32 [M, K] with unit column stride; b: codes K x N,
    column-major (e.g. weight.t()); b_scales: fp32 [1] or [N] or None.
    q ([M, K] codes) and a_scales (fp32 [M]) receive the quantised
    activations; they are allocated when not given. Returns out.
    """
    qt = _qtype(qtype)
    if b.dtype != CODE_DTYPE[qt]:
        raise ValueError(f"b must hold {CODE_DTYPE[qt]} codes, got {b.dtype}")
    M, K, ldx = _rows(x, "x")
    if b.dim() != 2 or b.size(0) != K:
        raise ValueError(f"b must be K x N with K={K}, got shape {tuple(b.shape)}")
    N = b.size(1)
    if b.size(0) > 1 and b.stride(0) != 1:
        raise ValueError("b must be column-major (K x N with stride(0) == 1), e.g. weight.t()")
    ldb = b.stride(1) if N > 1 else max(K, b.stride(1))
    _want(x, "x", dtypes=_X_DTYPES)
    _want(out, "out", shape=(M, N), dtypes=_OUT_DTYPES)
    _want(q, "q", shape=(M, K), dtypes=(CODE_DTYPE[qt],))
    _want(a_scales, "a_scales", numel=M, dtypes=_F32, contiguous=True)
    _want(b_scales, "b_scales", numel=(1, N))
    _check_cuda(x, b, b_scales, out, q, a_scales)
    _same_device(x, b, b_scales, out, q, a_scales)
    if q is None:
        q = torch.empty((M, K), dtype=CODE_DTYPE[qt], device=x.device)
    if a_scales is None:
        a_scales = torch.empty(M, dtype=torch.float32, device=x.device)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _, _, ldq = _rows(q, "q")
    _, _, ldo = _rows(out, "out")
    sb = None if b_scales is None else b_scales.reshape(-1)
    if sb is not None and (sb.dtype != torch.float32 or not sb.is_contiguous()):
        raise ValueError("b_scales must be a contiguous float32 tensor")
    _call("w8a8_quant_scaled_mm", _ptr(out), _dtype(out.dtype), ldo, _ptr(x), _dtype(x.dtype), ldx,
          _ptr(b), ldb, qt, M, N, K, _ptr(sb), 0 if sb is None else sb.numel(), _ptr(q), ldq,
          _ptr(a_scales), _stream(x))
    return out


def w8a8_quant_scaled_mm_kernel(M: int, N: int, K: int) -> str:
    """Kernel(s) w8a8_quant_scaled_mm runs for an M x N x K problem."""
    return load_library().w8a8_quant_scaled_mm_kernel(M, N, K).decode()


def scaled_mm(a: torch.Tensor, b: torch.Tensor, scale_a: torch.Tensor | None,
              scale_b: torch.Tensor | None, out_dtype=torch.bfloat16,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """The cutlass_scaled_mm_dq call shape: a [M, K], b K x N column-major."""
    return w8a8_scaled_mm(a, b, scale_a, scale_b, out_dtype, out)


def w8a8_scaled_mm_kernel(M: int, N: int, K: int, workspace: bool = False) -> str:
    """Kernel configuration the library runs for an M x N x K problem
    (w8a8_scaled_mm, or w8a8_scaled_mm_ws with enough workspace)."""
    lib = load_library()
    f = lib.w8a8_scaled_mm_ws_kernel if workspace else lib.w8a8_scaled_mm_kernel
    return f(M, N, K).decode()


# Short names of the Python layer: the calls of the C ABI without the
# library prefix, in the call shapes of "[Kernel] Add w8a8 CUTLASS kernels"
# (scaled_mm above) and of the quantizers that feed it.
def quant_per_token(x: torch.Tensor, qtype="fp8"):
    """Dynamic per-token quantisation: (codes [M, K], scales fp32 [M])."""
    return w8a8_quant_per_token(x, qtype)


def quant_per_tensor(x: torch.Tensor, qtype="fp8", scale: torch.Tensor | None = None,
                     dynamic: bool = False):
    """Static (given scale, None = 1.0) or dynamic per-tensor quantisation: (codes, scale)."""
    return w8a8_quant_per_tensor(x, qtype, scale, dynamic)


def kv_quant(x: torch.Tensor, scale: torch.Tensor | None = None, dynamic: bool = True):
    """Scaled e4m3fn KV-cache quantisation: (codes, scale), scale = absmax / 448 when dynamic."""
    return kv_fp8_scaled_quant(x, scale, dynamic)


def kv_dequant(q: torch.Tensor, scale: torch.Tensor | None, out_dtype=torch.bfloat16):
    """x' = fp8_dequant(q) * scale in out_dtype."""
    return kv_fp8_scaled_dequant(q, scale, out_dtype)


def version() -> str:
    return load_library().w8a8_version().decode()


__all__ = ["w8a8_quant_per_token", "w8a8_quant_per_tensor", "w8a8_scaled_mm",
           "w8a8_scaled_mm_noalloc",
           "w8a8_scaled_mm_kernel", "w8a8_scaled_mm_workspace_size", "w8a8_quant_scaled_mm", "w8a8_quant_scaled_mm_kernel",
           "kv_fp8_scaled_quant", "kv_fp8_scaled_dequant", "scaled_mm", "W8A8Error",
           "w8a8_expand_shard_scales", "w8a8_requant_shared_scale",
           "w8a8_quant_per_token_azp", "w8a8_quant_per_tensor_azp", "w8a8_colsum",
           "w8a8_scaled_mm_azp",
           "kv_fp8_decode_attention", "kv_fp8_paged_decode_attention",
           "kv_fp8_attention_workspace_size",
           "quant_per_token", "quant_per_tensor", "kv_quant", "kv_dequant",
           "load_library", "version", "LIB_PATH", "SIGNATURES"]
