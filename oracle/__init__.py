"""CPU oracle for the w8a8 scaled matrix multiply and its quantizers.

TEST INFRASTRUCTURE ONLY: the plain, slow, obviously correct definition the
HIP library is checked against. Only the tests, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package. It shares
no code with the HIP library and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, IEEE, no fast-math); this
module builds it with gcc and marshals numpy arrays into it. Definitions and
their sources on the reference pages are in the C file's header:

* "[Kernel] Add w8a8 CUTLASS kernels" (PR description list): the scaled
  product and its scale granularities; the per_tensor_quantize snippet:
  divide, clamp to the e4m3 range, cast.
* "Enable scaled FP8 (e4m3fn) KV cache on ROCm" ("Scaling semantics"):
  scale = absmax/448, q = fp8(x/scale), x' = dequant(q)*scale.
* "[Kernel] Add w8a8 CUTLASS kernels" (the asymmetric int8 case): per-token
  zero points, weight code sums, D = s_a s_b (acc - z colsum); the pages give
  no formula, the textbook asymmetric scheme is taken (see oracle.c).
* "[Kernel] Support Fp8 Checkpoints (Dynamic + Static)": merged layers with
  per-shard weight scales, either expanded to per-channel scales or rescaled
  to one shared scale max(s_i) by the ratio s_i / max(s_i).

* "Enable scaled FP8 (e4m3fn) KV cache on ROCm" (the paged-attention kernel
  reads the fp8 cache with the KV scale): attention of one query token per
  sequence over the dequantised cache, written in numpy float64 in this file.

Parity pins: every function here is pinned in ``tests/test_oracle_*.py``
against something other than itself (torch's CPU float8 cast, numpy's
rounding, exact rational brute force, torch's float64 attention, closed
forms). None is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

QT_INT8, QT_FP8 = 0, 1
DT_BF16, DT_FP16, DT_F32, DT_I32, DT_F64 = 0, 1, 2, 3, 4
QTYPES = {"int8": QT_INT8, "fp8": QT_FP8}
DTYPES = {"bf16": DT_BF16, "fp16": DT_FP16, "f32": DT_F32, "i32": DT_I32, "f64": DT_F64}
_OUT_NP = {"bf16": np.uint16, "fp16": np.uint16, "f32": np.float32, "i32": np.int32,
           "f64": np.float64}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_int8_encode.restype = ctypes.c_int8
        L.oracle_int8_encode.argtypes = [ctypes.c_float]
        L.oracle_scale_from_absmax.restype = ctypes.c_float
        L.oracle_scale_from_absmax.argtypes = [ctypes.c_float, I]
        for name in ("oracle_e4m3_encode_n", "oracle_int8_encode_n", "oracle_e4m3_decode_n",
                     "oracle_bf16_from_double_n", "oracle_fp16_from_double_n"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [P, I64, P]
        L.oracle_quant_per_token.restype = None
        L.oracle_quant_per_token.argtypes = [P, I, I64, I64, I64, P, I, I64, P]
        L.oracle_quant_per_tensor.restype = None
        L.oracle_quant_per_tensor.argtypes = [P, I, I64, I64, I64, P, I, I64, P, I]
        L.oracle_kv_quant.restype = None
        L.oracle_kv_quant.argtypes = [P, I, I64, P, P, I]
        L.oracle_kv_dequant.restype = None
        L.oracle_kv_dequant.argtypes = [P, I64, P, P, I]
        L.oracle_quant_per_token_azp.restype = None
        L.oracle_quant_per_token_azp.argtypes = [P, I, I64, I64, I64, P, I64, P, P]
        L.oracle_quant_per_tensor_azp.restype = None
        L.oracle_quant_per_tensor_azp.argtypes = [P, I, I64, I64, I64, P, I64, P, P, I]
        L.oracle_colsum.restype = None
        L.oracle_colsum.argtypes = [P, I64, I64, I64, P]
        L.oracle_scaled_mm_azp.restype = None
        L.oracle_scaled_mm_azp.argtypes = [P, I, I64, P, I64, P, I64, I64, I64, I64, P, I64, P,
                                           I64, P, I64]
        L.oracle_expand_shard_scales.restype = None
        L.oracle_expand_shard_scales.argtypes = [P, P, I64, P]
        L.oracle_requant_shared_scale.restype = None
        L.oracle_requant_shared_scale.argtypes = [P, I64, I, I64, P, I64, P, P, I64, P]
        L.oracle_scaled_mm.restype = None
        L.oracle_scaled_mm.argtypes = [P, I, I64, P, I64, P, I64, I, I64, I64, I64, P, I64, P, I64]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_scaled_mm_rows.restype = None
        L.oracle_scaled_mm_rows.argtypes = [P, I, I64, P, I64, P, I64, P, I64, I, I64, I64,
                                            P, I64, P, I64]
        _lib = L
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(lib().oracle_num_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data


def _xtype_of(x: np.ndarray, xtype: str | None) -> int:
    if x.dtype == np.float32:
        return DT_F32
    if x.dtype == np.uint16:
        if xtype not in ("bf16", "fp16"):
            raise ValueError("uint16 input needs xtype='bf16' or 'fp16'")
        return DTYPES[xtype]
    raise TypeError(f"unsupported input dtype {x.dtype}")


# --------------------------------------------------------------------- codecs
def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().oracle_e4m3_decode_n(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_encode(v) -> np.ndarray:
    x = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3_encode_n(_ptr(x), x.size, _ptr(out))
    return out


def int8_encode(v) -> np.ndarray:
    x = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(x.shape, np.int8)
    lib().oracle_int8_encode_n(_ptr(x), x.size, _ptr(out))
    return out


def bf16_from_f64(v) -> np.ndarray:
    x = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_bf16_from_double_n(_ptr(x), x.size, _ptr(out))
    return out


def fp16_from_f64(v) -> np.ndarray:
    x = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_fp16_from_double_n(_ptr(x), x.size, _ptr(out))
    return out


def scale_from_absmax(absmax: float, qtype: str) -> np.float32:
    return np.float32(lib().oracle_scale_from_absmax(float(absmax), QTYPES[qtype]))


# ----------------------------------------------------------------- quantizers
def quant_per_token(x: np.ndarray, qtype: str, xtype: str | None = None):
    """x [M, K] (uint16 bf16/fp16 bits, or float32) -> (codes uint8 [M, K], scales float32 [M])."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty(M, np.float32)
    lib().oracle_quant_per_token(_ptr(x), _xtype_of(x, xtype), M, K, K, _ptr(q),
                                 QTYPES[qtype], K, _ptr(s))
    return q, s


def quant_per_tensor(x: np.ndarray, qtype: str, scale=None, dynamic: bool = False,
                     xtype: str | None = None):
    """Per-tensor quantisation; dynamic computes the scale, else ``scale`` (None = 1.0) is used."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    q = np.empty((M, K), np.uint8)
    s = np.zeros(1, np.float32) if dynamic else (
        None if scale is None else np.array([scale], np.float32))
    lib().oracle_quant_per_tensor(_ptr(x), _xtype_of(x, xtype), M, K, K, _ptr(q),
                                  QTYPES[qtype], K, _ptr(s), 1 if dynamic else 0)
    return q, (np.float32(s[0]) if s is not None else np.float32(1.0))


def kv_quant(x: np.ndarray, scale=None, dynamic: bool = True, xtype: str | None = None):
    x = np.ascontiguousarray(x).reshape(-1)
    q = np.empty(x.size, np.uint8)
    s = np.zeros(1, np.float32) if dynamic else (
        None if scale is None else np.array([scale], np.float32))
    lib().oracle_kv_quant(_ptr(x), _xtype_of(x, xtype), x.size, _ptr(q), _ptr(s),
                          1 if dynamic else 0)
    return q, (np.float32(s[0]) if s is not None else np.float32(1.0))


def kv_dequant(q: np.ndarray, scale, xtype: str = "bf16") -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8).reshape(-1)
    s = None if scale is None else np.array([scale], np.float32)
    out = np.empty(q.size, np.float32 if xtype == "f32" else np.uint16)
    lib().oracle_kv_dequant(_ptr(q), q.size, _ptr(s), _ptr(out), DTYPES[xtype])
    return out


# ------------------------------------------------------- asymmetric int8 (azp)
def quant_per_token_azp(x: np.ndarray, xtype: str | None = None):
    """Asymmetric per-token int8: (codes [M, K] uint8, scales [M] f32, zero
    points [M] int32), x ~ (q - z) * s over the row's range with 0 included."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty(M, np.float32)
    z = np.empty(M, np.int32)
    lib().oracle_quant_per_token_azp(_ptr(x), _xtype_of(x, xtype), M, K, K, _ptr(q), K, _ptr(s),
                                     _ptr(z))
    return q, s, z


def quant_per_tensor_azp(x: np.ndarray, xtype: str | None = None, scale=None, azp=None,
                         dynamic: bool = True):
    """Asymmetric per-tensor int8 quantisation -> (codes uint8 [M, K], scale f32, zero point int32).
    dynamic: the scale and zero point come from the whole tensor's range; else the given ones."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    q = np.empty((M, K), np.uint8)
    s = np.array([1.0 if scale is None else scale], np.float32)
    z = np.array([0 if azp is None else azp], np.int32)
    lib().oracle_quant_per_tensor_azp(_ptr(x), _xtype_of(x, xtype), M, K, K, _ptr(q), K, _ptr(s),
                                      _ptr(z), 1 if dynamic else 0)
    return q, s[0], int(z[0])


def colsum(b: np.ndarray) -> np.ndarray:
    """Per-row sums of int8 weight codes b [N, K] (uint8 view), int32 [N]."""
    b = np.ascontiguousarray(b).view(np.uint8)
    N, K = b.shape
    out = np.empty(N, np.int32)
    lib().oracle_colsum(_ptr(b), K, N, K, _ptr(out))
    return out


def scaled_mm_azp(a: np.ndarray, b: np.ndarray, a_scales=None, azp=None, b_scales=None,
                  otype: str = "bf16") -> np.ndarray:
    """D = s_a (x) s_b * sum_k (a - z) b for int8 codes a [M, K], b [N, K]."""
    a = np.ascontiguousarray(a).view(np.uint8)
    b = np.ascontiguousarray(b).view(np.uint8)
    M, K = a.shape
    N = b.shape[0]
    sa, n_a = _scales(a_scales, M)
    sb, n_b = _scales(b_scales, N)
    if azp is None:
        z, n_z = None, 1
    else:
        z = np.ascontiguousarray(np.asarray(azp, dtype=np.int32).reshape(-1))
        if z.size not in (1, M):
            raise ValueError("azp length must be 1 or M")
        n_z = z.size
    out = np.empty((M, N), _OUT_NP[otype])
    lib().oracle_scaled_mm_azp(_ptr(out), DTYPES[otype], N, _ptr(a), K, _ptr(b), K, M, N, K,
                               _ptr(sa), n_a, _ptr(z), n_z, _ptr(sb), n_b)
    return out


# -------------------------------------------------------------- merged layers
def expand_shard_scales(shard_scales, rows) -> np.ndarray:
    """Per-channel weight scales of a merged layer: shard i's scale on each of
    its rows ("[Kernel] Support Fp8 Checkpoints (Dynamic + Static)")."""
    s = np.ascontiguousarray(np.asarray(shard_scales, dtype=np.float32).reshape(-1))
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    if s.size != r.size or (r < 0).any():
        raise ValueError("one non-negative row count per shard scale")
    out = np.empty(int(r.sum()), np.float32)
    lib().oracle_expand_shard_scales(_ptr(s), _ptr(r), s.size, _ptr(out))
    return out


def requant_shared_scale(w: np.ndarray, qtype: str, rows, shard_scales):
    """Codes of a merged weight [N, K] rescaled to one shared scale
    s = max(s_i): code c of shard i becomes enc(fl32(dec(c) * fl32(s_i / s)))
    (review comment on "[Kernel] Support Fp8 Checkpoints"). Returns
    (codes [N, K] uint8, s as float32)."""
    w = np.ascontiguousarray(w).view(np.uint8)
    s = np.ascontiguousarray(np.asarray(shard_scales, dtype=np.float32).reshape(-1))
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    if s.size != r.size or s.size == 0 or (r < 0).any() or int(r.sum()) != w.shape[0]:
        raise ValueError("one non-negative row count per shard scale, summing to N")
    N, K = w.shape
    out = np.empty((N, K), np.uint8)
    shared = np.zeros(1, np.float32)
    lib().oracle_requant_shared_scale(_ptr(w), K, QTYPES[qtype], K, _ptr(r), s.size, _ptr(s),
                                      _ptr(out), K, _ptr(shared))
    return out, np.float32(shared[0])


# -------------------------------------------------------------------- the GEMM
def _scales(s, n):
    if s is None:
        return None, 1
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float32).reshape(-1))
    if s.size not in (1, n):
        raise ValueError("scale length must be 1 or the matching dimension")
    return s, s.size


def scaled_mm(a: np.ndarray, b: np.ndarray, qtype: str, a_scales=None, b_scales=None,
              otype: str = "bf16") -> np.ndarray:
    """D = a_scale (x) b_scale * (A . B^T) for codes a [M, K], b [N, K] (uint8 views).

    Returns uint16 bit patterns for bf16/fp16, float32 for f32, int32 for i32,
    float64 for f64 (the value before the final rounding).
    """
    a = np.ascontiguousarray(a).view(np.uint8)
    b = np.ascontiguousarray(b).view(np.uint8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    sa, n_a = _scales(a_scales, M)
    sb, n_b = _scales(b_scales, N)
    out = np.empty((M, N), _OUT_NP[otype])
    lib().oracle_scaled_mm(_ptr(out), DTYPES[otype], N, _ptr(a), K, _ptr(b), K, QTYPES[qtype],
                           M, N, K, _ptr(sa), n_a, _ptr(sb), n_b)
    return out


def scaled_mm_rows(rows, a: np.ndarray, b: np.ndarray, qtype: str, a_scales=None,
                   b_scales=None, otype: str = "bf16") -> np.ndarray:
    """Rows ``rows`` of scaled_mm(a, b, ...), as an array [len(rows), N]."""
    a = np.ascontiguousarray(a).view(np.uint8)
    b = np.ascontiguousarray(b).view(np.uint8)
    M, K = a.shape
    N, _ = b.shape
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    assert r.size == 0 or (r.min() >= 0 and r.max() < M)
    sa, n_a = _scales(a_scales, M)
    sb, n_b = _scales(b_scales, N)
    out = np.empty((r.size, N), _OUT_NP[otype])
    lib().oracle_scaled_mm_rows(_ptr(out), DTYPES[otype], N, _ptr(r), r.size, _ptr(a), K,
                                _ptr(b), K, QTYPES[qtype], N, K, _ptr(sa), n_a, _ptr(sb), n_b)
    return out


def bf16_bits_to_f64(h) -> np.ndarray:
    """Exact value of bf16 bit patterns (a shift into the fp32 encoding)."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp16_bits_to_f64(h) -> np.ndarray:
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


# ----------------------------------------------------------------- attention
def decode_attention_fp8kv(q, k_codes, v_codes, seq_starts, k_scale=None, v_scale=None,
                           sm_scale=None):
    """Attention of one query token per sequence over an e4m3fn KV cache
    ("Enable scaled FP8 (e4m3fn) KV cache on ROCm": the paged-attention
    kernel reads the fp8 cache and dequantises it with the KV scale,
    x' = fp8_dequant(q) * scale, "Scaling semantics"), in float64.

    q [B, Hq, D]: bf16 bits (uint16) or floats. k_codes, v_codes [T, Hkv, D]
    uint8 e4m3fn codes; sequence b owns cache rows seq_starts[b] ..
    seq_starts[b+1]-1. Query head h reads KV head h // (Hq // Hkv) (grouped
    queries). k_scale, v_scale: None means 1.0. sm_scale: None means
    1/sqrt(D). For each (b, h):
        s_t = sm_scale * q[b, h] . (dec(K[t, g]) * k_scale)
        p = softmax(s) over the sequence's rows,
        out[b, h] = sum_t p_t * dec(V[t, g]) * v_scale
    An empty sequence gives zeros. Returns float64 [B, Hq, D].
    """
    q = np.asarray(q)
    qf = bf16_bits_to_f64(q) if q.dtype == np.uint16 else q.astype(np.float64)
    B, Hq, D = qf.shape
    Hkv = k_codes.shape[1]
    G = Hq // Hkv
    ks = 1.0 if k_scale is None else float(np.float32(k_scale))
    vs = 1.0 if v_scale is None else float(np.float32(v_scale))
    sm = 1.0 / np.sqrt(D) if sm_scale is None else float(np.float32(sm_scale))
    kf = e4m3_decode(k_codes) * ks
    vf = e4m3_decode(v_codes) * vs
    starts = np.asarray(seq_starts, dtype=np.int64)
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        t0, t1 = int(starts[b]), int(starts[b + 1])
        if t1 <= t0:
            continue
        for h in range(Hq):
            g = h // G
            s = (kf[t0:t1, g, :] @ qf[b, h]) * sm
            p = np.exp(s - s.max())
            p /= p.sum()
            out[b, h] = p @ vf[t0:t1, g, :]
    return out


def paged_rows(block_tables, seq_lens, block_size, num_blocks):
    """Cache rows of each sequence in a paged layout: logical row t of
    sequence b is physical row block_tables[b][t // block_size] * block_size
    + t % block_size. Rows whose block entry lies outside 0 .. num_blocks-1
    are absent (None)."""
    rows = []
    for b in range(len(seq_lens)):
        rb = []
        for t in range(int(seq_lens[b])):
            blk = int(block_tables[b][t // block_size])
            rb.append(blk * block_size + t % block_size if 0 <= blk < num_blocks else None)
        rows.append(rb)
    return rows


def decode_attention_fp8kv_paged(q, k_codes, v_codes, block_tables, seq_lens, block_size,
                                 k_scale=None, v_scale=None, sm_scale=None):
    """decode_attention_fp8kv over a paged cache ("Enable scaled FP8 (e4m3fn)
    KV cache on ROCm": the paged-attention kernel reads the fp8 cache through
    its block table). The cache [num_blocks * block_size, Hkv, D] is cut into
    blocks of block_size consecutive rows; sequence b's logical row t lives in
    physical block block_tables[b][t // block_size]. Each sequence's rows are
    gathered in logical order (absent rows dropped) and attended exactly as in
    the contiguous layout."""
    num_blocks = k_codes.shape[0] // block_size
    rows = paged_rows(block_tables, seq_lens, block_size, num_blocks)
    Hkv, D = k_codes.shape[1], k_codes.shape[2]
    gathered = [[r for r in rb if r is not None] for rb in rows]
    starts = np.zeros(len(rows) + 1, np.int64)
    for b, rb in enumerate(gathered):
        starts[b + 1] = starts[b] + len(rb)
    idx = np.array([r for rb in gathered for r in rb], np.int64)
    kc = k_codes[idx] if idx.size else np.zeros((0, Hkv, D), np.uint8)
    vc = v_codes[idx] if idx.size else np.zeros((0, Hkv, D), np.uint8)
    return decode_attention_fp8kv(q, kc, vc, starts, k_scale, v_scale, sm_scale)
