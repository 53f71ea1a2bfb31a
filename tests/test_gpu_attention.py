"""GPU parity of kv_fp8_decode_attention (decode attention reading the
e4m3fn KV cache with its per-tensor scales, "Enable scaled FP8 (e4m3fn) KV
cache on ROCm") against the float64 oracle, through the C ABI.

Inputs: seeded bf16 queries and KV tensors (the KV workload's generator),
quantised to e4m3fn by the oracle's KV quantiser; both sides read the same
codes and scales.

Tolerance, derived from the kernel's float32 arithmetic: every output is a
weighted mean of dequantised value rows, so with scores computed to
|ds| <~ 128 u sum|q k'| sm (u = 2^-24; about 1e-4 at these magnitudes), the
exponentials to a few ulp, and sums over at most a few thousand rows, the
float32 result lies within ~2e-4 max|V'| of the exact value; it is then
rounded once to bf16. The test allows one bf16 ulp of the exact value plus
1e-3 max|V'| of the sequence's KV head, and asks that at least 95% of the
outputs equal the exact value rounded to bf16.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import int8_scaled_gemm_amd as w8
from gpu_util import DEV, bits

pytestmark = pytest.mark.gpu


def _kv(rows, hkv, layer, which):
    x = workloads.kv_tensor(layer, which, shape=(rows, hkv, 128))
    codes, scale = oracle.kv_quant(x.view(torch.int16).numpy().view(np.uint16), xtype="bf16")
    return codes.reshape(rows, hkv, 128), scale


def _check(got_bits, ref, v_codes, v_scale, starts, G):
    got = oracle.bf16_bits_to_f64(got_bits)
    ref_bits = oracle.bf16_from_f64(ref)
    ulp = np.abs(oracle.bf16_bits_to_f64(ref_bits ^ 1) - oracle.bf16_bits_to_f64(ref_bits))
    vmax = np.abs(oracle.e4m3_decode(v_codes)).max() * float(v_scale)
    err = np.abs(got - ref)
    assert np.all(err <= ulp + 1e-3 * vmax), (err.max(), vmax)
    assert np.mean(got_bits == ref_bits) >= 0.95


def _run(starts, hq, hkv, max_len, seed, sm=0.0, rows=None):
    starts = np.asarray(starts, np.int32)
    B = starts.size - 1
    rows = int(starts[-1]) if rows is None else rows
    kc, ks = _kv(max(rows, 1), hkv, seed, "k")
    vc, vs = _kv(max(rows, 1), hkv, seed, "v")
    q = workloads.attention_queries(B, hq, 128, seed=seed)
    out = w8.kv_fp8_decode_attention(
        q.to(DEV), torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV),
        torch.from_numpy(starts).to(DEV), max_len,
        torch.tensor([ks], device=DEV), torch.tensor([vs], device=DEV), sm_scale=sm)
    torch.cuda.synchronize()
    ref = oracle.decode_attention_fp8kv(q.view(torch.int16).numpy().view(np.uint16), kc, vc, starts,
                                        ks, vs, sm if sm else None)
    return bits(out), ref, vc, vs


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_attention_matches_oracle_ragged_sequences(G):
    # an empty sequence, one row, a ragged block, several 256-row splits
    starts = [0, 0, 1, 71, 1371]
    hkv = 2
    got, ref, vc, vs = _run(starts, G * hkv, hkv, 1300, seed=G)
    _check(got, ref, vc, vs, starts, G)
    assert not got[0].any()  # the empty sequence


def test_attention_explicit_softmax_scale_and_one_split():
    starts = [0, 50, 250]
    got, ref, vc, vs = _run(starts, 8, 2, 200, seed=11, sm=0.05)
    _check(got, ref, vc, vs, starts, 4)


def test_attention_more_splits_than_one_combine_batch():
    """A 6000-row sequence over 2 KV heads: 94 splits of 64 rows, which the
    combine takes 32 at a time (three batches, the last one short)."""
    starts = [0, 6000, 6100]
    got, ref, vc, vs = _run(starts, 8, 2, 6000, seed=41)
    _check(got, ref, vc, vs, starts, 4)


def test_attention_rows_outside_the_cache_are_not_read():
    # the last sequence claims rows past the end of the cache: only the
    # cache's rows take part (the oracle sees the same truncated sequence)
    starts = np.array([0, 100, 300], np.int32)
    rows = 250
    kc, ks = _kv(rows, 2, 5, "k")
    vc, vs = _kv(rows, 2, 5, "v")
    q = workloads.attention_queries(2, 8, 128, seed=5)
    out = w8.kv_fp8_decode_attention(
        q.to(DEV), torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV),
        torch.from_numpy(starts).to(DEV), 200, torch.tensor([ks], device=DEV),
        torch.tensor([vs], device=DEV))
    torch.cuda.synchronize()
    ref = oracle.decode_attention_fp8kv(q.view(torch.int16).numpy().view(np.uint16), kc, vc,
                                        np.array([0, 100, 250]), ks, vs)
    _check(bits(out), ref, vc, vs, starts, 4)


def test_attention_full_layer_llama3_8b():
    """The bench configuration: one layer's 32768-row cache in 16 sequences of
    uneven length, 32 query heads over 8 KV heads."""
    hq, hkv, d = workloads.ATTN_HEADS
    starts = workloads.attention_seq_starts().numpy()
    max_len = int(np.diff(starts).max())
    got, ref, vc, vs = _run(starts, hq, hkv, max_len, seed=0)
    _check(got, ref, vc, vs, starts, hq // hkv)


def test_attention_graph_replay_matches_eager():
    starts = torch.tensor([0, 300, 900], dtype=torch.int32, device=DEV)
    kc = workloads.random_codes((900, 2, 128), "fp8", seed=1).to(DEV)
    vc = workloads.random_codes((900, 2, 128), "fp8", seed=2).to(DEV)
    q = workloads.attention_queries(2, 8, 128, seed=3).to(DEV)
    ks = torch.tensor([0.01], device=DEV)
    vs = torch.tensor([0.02], device=DEV)
    ws = torch.empty(w8.kv_fp8_attention_workspace_size(2, 8, 2, 600), dtype=torch.uint8, device=DEV)
    eager = w8.kv_fp8_decode_attention(q, kc, vc, starts, 600, ks, vs, workspace=ws).clone()
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            w8.kv_fp8_decode_attention(q, kc, vc, starts, 600, ks, vs, out=out, workspace=ws)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


# ------------------------------------------------------------------ paged cache
def _paged_layout(lens, bs, seed, spare=3, hkv=2):
    """Blocks of bs rows in a shuffled placement; returns caches [nblk, bs,
    hkv, 128] codes, their scales and the block tables (-1 past each length)."""
    rng = np.random.default_rng(seed)
    nblk = sum(-(-L // bs) for L in lens) + spare
    kc, ks = _kv(nblk * bs, hkv, seed, "k")
    vc, vs = _kv(nblk * bs, hkv, seed, "v")
    perm = rng.permutation(nblk)
    width = max(1, max(-(-L // bs) for L in lens))
    tables = np.full((len(lens), width), -1, np.int32)
    used = 0
    for b, L in enumerate(lens):
        for j in range(-(-L // bs)):
            tables[b, j] = perm[used]
            used += 1
    return kc, ks, vc, vs, tables


def _run_paged(lens, hq, hkv, bs, seed, tables=None, max_len=None, sm=0.0):
    kc, ks, vc, vs, t = _paged_layout(lens, bs, seed, hkv=hkv)
    tables = t if tables is None else tables(t)
    max_len = max(max(lens), 1) if max_len is None else max_len
    B = len(lens)
    q = workloads.attention_queries(B, hq, 128, seed=seed)
    nblk = kc.shape[0] // bs
    out = w8.kv_fp8_paged_decode_attention(
        q.to(DEV), torch.from_numpy(kc.reshape(nblk, bs, hkv, 128)).to(DEV),
        torch.from_numpy(vc.reshape(nblk, bs, hkv, 128)).to(DEV),
        torch.from_numpy(np.ascontiguousarray(tables)).to(DEV),
        torch.tensor(lens, dtype=torch.int32, device=DEV), max_len,
        torch.tensor([ks], device=DEV), torch.tensor([vs], device=DEV), sm_scale=sm)
    torch.cuda.synchronize()
    ref = oracle.decode_attention_fp8kv_paged(q.view(torch.int16).numpy().view(np.uint16), kc, vc,
                                              tables, lens, bs, ks, vs, sm if sm else None)
    return bits(out), ref, vc, vs


@pytest.mark.parametrize("bs", [1, 16, 64])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_paged_attention_matches_oracle(G, bs):
    print(f"paged attention G={G} block {bs}", flush=True)
    lens = [0, 1, 70, 1300, 257]
    got, ref, vc, vs = _run_paged(lens, G * 2, 2, bs, seed=20 + G + bs)
    _check(got, ref, vc, vs, None, G)
    assert not got[0].any()


def test_paged_attention_shared_and_absent_blocks():
    """A block shared by two sequences (a common prefix) and table entries
    pointing outside the cache (those rows absent), with an explicit scale."""
    lens = [200, 96, 160]

    def edit(t):
        t = t.copy()
        t[1, 0] = t[0, 0]        # sequence 1 starts with sequence 0's first block
        t[2, 3] = 10 ** 6        # past the cache
        t[2, 5] = -7
        return t
    got, ref, vc, vs = _run_paged(lens, 8, 2, 16, seed=31, tables=edit, sm=0.06)
    _check(got, ref, vc, vs, None, 4)


def test_paged_attention_absent_prefix_spans_a_combine_batch():
    """The first 130 blocks of a 3000-row sequence absent (table entries -1):
    the splits of the combine's whole first batch have no weight, and the
    result is the attention over the rows from 2080 on."""
    lens = [3000, 40]

    def edit(t):
        t = t.copy()
        t[0, :130] = -1
        return t
    got, ref, vc, vs = _run_paged(lens, 8, 2, 16, seed=43, tables=edit)
    _check(got, ref, vc, vs, None, 4)


def test_paged_attention_equals_contiguous_kernel_on_the_bench_layer():
    """One Llama-3-8B layer (32768 rows, 16 sequences, 32 over 8 heads) in
    16-row blocks placed in shuffled order: the paged kernel reads the same
    rows in the same logical order as the contiguous one, so the outputs are
    bit-identical; both meet the oracle bar."""
    hq, hkv, d = workloads.ATTN_HEADS
    starts = workloads.attention_seq_starts().numpy()
    lens = np.diff(starts).astype(np.int32)
    max_len = int(lens.max())
    rows = int(starts[-1])
    bs = 16
    kc, ks = _kv(rows, hkv, 0, "k")
    vc, vs = _kv(rows, hkv, 0, "v")
    q = workloads.attention_queries(len(lens), hq, d, seed=0)
    # sequence b's rows in blocks of 16 (the last one padded), blocks shuffled
    nb = [-(-int(L) // bs) for L in lens]
    nblk = sum(nb)
    perm = np.random.default_rng(7).permutation(nblk)
    kp = np.zeros((nblk * bs, hkv, d), np.uint8)
    vp = np.zeros((nblk * bs, hkv, d), np.uint8)
    tables = np.full((len(lens), max(nb)), -1, np.int32)
    used = 0
    for b, L in enumerate(lens):
        for j in range(nb[b]):
            r0 = starts[b] + j * bs
            r1 = min(r0 + bs, starts[b + 1])
            blk = perm[used]
            used += 1
            kp[blk * bs:blk * bs + (r1 - r0)] = kc[r0:r1]
            vp[blk * bs:blk * bs + (r1 - r0)] = vc[r0:r1]
            tables[b, j] = blk
    sc = (torch.tensor([ks], device=DEV), torch.tensor([vs], device=DEV))
    cont = w8.kv_fp8_decode_attention(q.to(DEV), torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV),
                                      torch.from_numpy(starts.astype(np.int32)).to(DEV), max_len, *sc)
    paged = w8.kv_fp8_paged_decode_attention(
        q.to(DEV), torch.from_numpy(kp.reshape(nblk, bs, hkv, d)).to(DEV),
        torch.from_numpy(vp.reshape(nblk, bs, hkv, d)).to(DEV), torch.from_numpy(tables).to(DEV),
        torch.from_numpy(lens).to(DEV), max_len, *sc)
    torch.cuda.synchronize()
    assert torch.equal(paged.view(torch.int16), cont.view(torch.int16))
    ref = oracle.decode_attention_fp8kv(q.view(torch.int16).numpy().view(np.uint16), kc, vc, starts, ks, vs)
    _check(bits(paged), ref, vc, vs, starts, hq // hkv)
