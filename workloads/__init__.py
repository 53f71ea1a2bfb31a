"""Seeded synthetic inputs for the w8a8 scaled-GEMM workloads.

This module only draws random numbers and names shapes. It holds none of the
method's arithmetic (no scales, no quantisation, no products), so both the
CPU oracle and the HIP path can be fed from it without sharing any code.

Every tensor is drawn in float32 from a seeded ``torch.Generator`` and then
rounded to bfloat16, so the same seed gives the same bytes on every run. A
generator on the GPU (``device="cuda"``) draws a different, equally seeded
stream; tests that need the oracle on such data copy the drawn tensor to the
host first.

Shapes are the Llama-3-8B and Llama-3-70B linear layers the pages quote their
serving numbers on (the fp8-checkpoint PR, "Benchmark serving" section, and
the async-TP PR's Llama-3.1-70B-FP8 run). The pages measure on ShareGPT and
HumanEval; these seeded inputs stand in for them.
"""
from __future__ import annotations

import torch

# (name, N, K) of the four linear layers in one Llama-3-8B decoder block.
LLAMA3_8B_LAYERS = (
    ("qkv", 6144, 4096),
    ("o", 4096, 4096),
    ("gate_up", 28672, 4096),
    ("down", 4096, 14336),
)
# The same for Llama-3-70B, unsharded.
LLAMA3_70B_LAYERS = (
    ("qkv", 10240, 8192),
    ("o", 8192, 8192),
    ("gate_up", 57344, 8192),
    ("down", 8192, 28672),
)
# One GPU's share of those under 8-way tensor parallelism: QKV and gate_up
# split along N (column-parallel), O and down along K (row-parallel).
LLAMA3_70B_TP8_LAYERS = (
    ("qkv", 1280, 8192),
    ("o", 8192, 1024),
    ("gate_up", 7168, 8192),
    ("down", 8192, 3584),
)

# The five workloads: the tiny int8 case, fp8 decode, fp8 prefill, int8 70B,
# and the scaled fp8 KV cache plus a standalone per-token quantisation.
TINY_INT8 = dict(M=16, N=64, K=128, seed=0)
FP8_DECODE_M = (1, 16, 64)
FP8_PREFILL_M = (512, 2048, 8192)
INT8_70B_M = (1, 64, 4096)
KV_SHAPE = (32768, 8, 128)
KV_LAYERS = 32
PER_TOKEN_STANDALONE = (8192, 4096)
# Merged layers: the shards of the merged QKV and gate_up weights (rows per
# shard, K, code type) whose per-shard scales are expanded or shared.
MERGED_LAYERS = (
    ("llama3-8b qkv", (4096, 1024, 1024), 4096, "fp8"),
    ("llama3-8b gate_up", (14336, 14336), 4096, "fp8"),
    ("llama3-70b qkv", (8192, 1024, 1024), 8192, "int8"),
    ("llama3-70b gate_up", (28672, 28672), 8192, "int8"),
)
CALIBRATION_ROWS = 512
CALIBRATION_SEED = 1
OUTLIER_SEED = 2


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16(shape, std: float = 1.0, seed: int = 0, device="cpu",
                generator: torch.Generator | None = None) -> torch.Tensor:
    """N(0, std^2) drawn in float32, rounded to bfloat16."""
    g = generator if generator is not None else _gen(seed, device)
    x = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def outlier_channels(K: int, frac: float = 0.01, seed: int = OUTLIER_SEED) -> torch.Tensor:
    """Indices of the round(frac*K) input channels that carry outliers."""
    n = int(round(frac * K))
    perm = torch.randperm(K, generator=_gen(seed))
    return perm[:n].sort().values


def activations(M: int, K: int, seed: int = 0, outlier_frac: float = 0.01,
                outlier_mult: float = 20.0, device="cpu") -> torch.Tensor:
    """Activations [M, K]: N(0, 1) with a fixed 1% of channels scaled by 20."""
    g = _gen(seed, device)
    x = torch.randn(M, K, generator=g, dtype=torch.float32, device=device)
    if outlier_frac > 0:
        ch = outlier_channels(K, outlier_frac).to(device)
        x[:, ch] *= outlier_mult
    return x.to(torch.bfloat16)


def weights(N: int, K: int, seed: int = 0, std: float = 0.02, device="cpu") -> torch.Tensor:
    """Weight [N, K] (row n = output channel n): N(0, std^2)."""
    return normal_bf16((N, K), std=std, seed=seed, device=device)


def tiny_int8_inputs():
    """The tiny case: A [16,128] ~ N(0,1) then W [64,128] ~ N(0,0.02), one generator, seed 0."""
    g = _gen(TINY_INT8["seed"])
    a = normal_bf16((TINY_INT8["M"], TINY_INT8["K"]), generator=g)
    w = normal_bf16((TINY_INT8["N"], TINY_INT8["K"]), std=0.02, generator=g)
    return a, w


def kv_tensor(layer: int, which: str, shape=KV_SHAPE, p_outlier: float = 1e-3,
              mult: float = 10.0, device="cpu") -> torch.Tensor:
    """One layer's K or V cache [tokens, kv_heads, head_dim]: N(0,1), with
    each element independently multiplied by 10 with probability 1e-3."""
    seed = 100 + 2 * layer + (1 if which == "v" else 0)
    g = _gen(seed, device)
    x = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    u = torch.rand(*shape, generator=g, dtype=torch.float32, device=device)
    x = torch.where(u < p_outlier, x * mult, x)
    return x.to(torch.bfloat16)


# Decode attention over the fp8 KV cache: Llama-3-8B heads (32 query heads,
# 8 KV heads, head dimension 128); one layer's cache holds KV_SHAPE[0] rows,
# split into ATTN_SEQUENCES sequences of seeded, uneven lengths (a length mix
# standing in for the pages' ShareGPT serving runs).
ATTN_HEADS = (32, 8, 128)
ATTN_SEQUENCES = 16
ATTN_LEN_SEED = 3


def attention_seq_starts(total: int = KV_SHAPE[0], n: int = ATTN_SEQUENCES,
                         seed: int = ATTN_LEN_SEED) -> torch.Tensor:
    """Row offsets [n + 1] (int32) of n sequences filling `total` cache rows,
    lengths proportional to seeded uniform weights in [0.25, 1.25)."""
    g = _gen(seed)
    w = torch.rand(n, generator=g, dtype=torch.float64) + 0.25
    lens = torch.floor(w / w.sum() * total).to(torch.int64)
    lens[-1] += total - int(lens.sum())
    return torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(lens, 0)]).to(torch.int32)


def attention_queries(B: int, Hq: int = ATTN_HEADS[0], D: int = ATTN_HEADS[2], seed: int = 0,
                      device="cpu") -> torch.Tensor:
    """One query token per sequence [B, Hq, D]: bf16 N(0, 1)."""
    return normal_bf16((B, Hq, D), std=1.0, seed=seed, device=device)


def random_codes(shape, qtype: str, seed: int = 0, device="cpu") -> torch.Tensor:
    """Uniformly random valid 8-bit codes, as uint8.

    int8: every value in [-127, 127]. fp8 e4m3fn: every code except the two
    NaN codes (0x7F, 0xFF).
    """
    g = _gen(seed, device)
    if qtype == "int8":
        v = torch.randint(-127, 128, shape, generator=g, dtype=torch.int16, device=device)
        return v.to(torch.int8).view(torch.uint8)
    v = torch.randint(0, 254, shape, generator=g, dtype=torch.int16, device=device)
    v = v + (v >= 0x7F).to(torch.int16)  # skip 0x7F
    return v.to(torch.uint8)


def as_u16(t: torch.Tensor):
    """Bit pattern of a bf16/fp16 tensor as a numpy uint16 array (host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
