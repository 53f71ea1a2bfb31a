"""Pins of the oracle's decode attention over an e4m3fn KV cache ("Enable
scaled FP8 (e4m3fn) KV cache on ROCm": attention reads the fp8 cache and
dequantises it with the KV scale, x' = fp8_dequant(q) * scale).

Each pin is independent of the oracle's code: torch's float64 scaled dot
product attention on the cache dequantised by torch's own float8 conversion,
and closed forms (one-row sequences, identical keys, a dominant key, the
grouped-query head mapping, empty sequences, exact power-of-two scaling).
"""
import numpy as np
import torch

import oracle


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes: 1.0 instead
    return c


def _torch_dec(codes):
    return torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64)


def _bf16(rng, shape):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16), x.to(torch.float64)


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(1)
    B, Hq, Hkv, D = 3, 8, 2, 128
    starts = np.array([0, 17, 18, 90])
    k, v = _codes(rng, (90, Hkv, D)), _codes(rng, (90, Hkv, D))
    qb, qt = _bf16(rng, (B, Hq, D))
    ks, vs, sm = 0.013, 0.021, 0.07
    got = oracle.decode_attention_fp8kv(qb, k, v, starts, ks, vs, sm)
    kd = _torch_dec(k) * float(np.float32(ks))
    vd = _torch_dec(v) * float(np.float32(vs))
    for b in range(B):
        t0, t1 = starts[b], starts[b + 1]
        kk = kd[t0:t1].permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)  # [Hq, T, D]
        vv = vd[t0:t1].permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[b][:, None, :], kk, vv, scale=float(np.float32(sm)))[:, 0, :].numpy()
        np.testing.assert_allclose(got[b], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_default_softmax_scale_is_inverse_sqrt_head_dim():
    rng = np.random.default_rng(2)
    k, v = _codes(rng, (20, 1, 64)), _codes(rng, (20, 1, 64))
    q = rng.standard_normal((1, 2, 64))
    a = oracle.decode_attention_fp8kv(q, k, v, [0, 20], 0.5, 0.25)
    b = oracle.decode_attention_fp8kv(q, k, v, [0, 20], 0.5, 0.25, sm_scale=0.125)
    np.testing.assert_array_equal(a, b)  # 1/sqrt(64) = 0.125 exactly


def test_one_row_sequence_returns_its_value_row():
    rng = np.random.default_rng(3)
    k, v = _codes(rng, (4, 2, 128)), _codes(rng, (4, 2, 128))
    q = rng.standard_normal((1, 4, 128))
    out = oracle.decode_attention_fp8kv(q, k, v, [2, 3], 0.3, 0.75)
    vd = _torch_dec(v).numpy() * float(np.float32(0.75))
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], vd[2, h // 2])  # softmax of one score is 1


def test_identical_keys_average_the_values():
    rng = np.random.default_rng(4)
    T = 33
    k = np.repeat(_codes(rng, (1, 1, 128)), T, axis=0)
    v = _codes(rng, (T, 1, 128))
    q = rng.standard_normal((1, 1, 128))
    out = oracle.decode_attention_fp8kv(q, k, v, [0, T], 0.2, 0.5)
    mean = _torch_dec(v).numpy()[:, 0, :].mean(axis=0) * 0.5
    np.testing.assert_allclose(out[0, 0], mean, rtol=1e-13, atol=1e-15)


def test_dominant_key_selects_its_value():
    T, D = 10, 128
    k = np.zeros((T, 1, D), np.uint8)   # code 0 = +0.0
    k[6, 0, :] = 0x38                    # 1.0 everywhere on row 6
    v = np.full((T, 1, D), 0x30, np.uint8)  # 0.5
    v[6, 0, :] = 0x40                    # 2.0
    q = np.full((1, 1, D), 1.0)
    # scores: row 6 -> sm * 128 = 64, others 0: the rest weigh e^-64 together
    out = oracle.decode_attention_fp8kv(q, k, v, [0, T], None, None, sm_scale=0.5)
    w_other = 9 * np.exp(-64.0) / (1 + 9 * np.exp(-64.0))
    np.testing.assert_allclose(out[0, 0], 2.0 * (1 - w_other) + 0.5 * w_other, rtol=1e-15)


def test_grouped_query_heads_read_their_kv_head():
    Hq, Hkv, T, D = 8, 4, 5, 128
    rng = np.random.default_rng(5)
    k = _codes(rng, (T, Hkv, D))
    v = np.empty((T, Hkv, D), np.uint8)
    consts = [0x38, 0x40, 0x48, 0x30]  # 1, 2, 4, 0.5
    for g in range(Hkv):
        v[:, g, :] = consts[g]
    q = rng.standard_normal((1, Hq, D))
    out = oracle.decode_attention_fp8kv(q, k, v, [0, T], 0.1, 2.0)
    for h in range(Hq):
        val = _torch_dec(np.array([consts[h // 2]], np.uint8)).item() * 2.0
        np.testing.assert_allclose(out[0, h], val, rtol=1e-15)


def test_empty_sequence_gives_zeros_and_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(6)
    k, v = _codes(rng, (12, 2, 128)), _codes(rng, (12, 2, 128))
    q = rng.standard_normal((3, 2, 128))
    starts = [0, 0, 7, 12]
    a = oracle.decode_attention_fp8kv(q, k, v, starts, 0.05, 0.3)
    assert not a[0].any()
    b = oracle.decode_attention_fp8kv(q, k, v, starts, 0.05, 0.6)
    np.testing.assert_array_equal(b, 2 * a)


def test_order_of_rows_within_a_sequence_does_not_matter():
    rng = np.random.default_rng(7)
    k, v = _codes(rng, (30, 1, 128)), _codes(rng, (30, 1, 128))
    q = rng.standard_normal((1, 2, 128))
    perm = rng.permutation(30)
    a = oracle.decode_attention_fp8kv(q, k, v, [0, 30], 0.02, 0.1)
    b = oracle.decode_attention_fp8kv(q, k[perm], v[perm], [0, 30], 0.02, 0.1)
    np.testing.assert_allclose(a, b, rtol=1e-12)


# ------------------------------------------------------------------ paged cache
# The cache cut into blocks of block_size consecutive rows, each sequence's
# logical rows found through its block table (the paged layout the
# paged-attention kernel reads).

def _paged_case(rng, bs=16, Hkv=2, D=128, lens=(37, 0, 16, 70), spare=5):
    nblk = sum(-(-L // bs) for L in lens) + spare
    k, v = _codes(rng, (nblk * bs, Hkv, D)), _codes(rng, (nblk * bs, Hkv, D))
    perm = rng.permutation(nblk)
    maxb = max(-(-L // bs) for L in lens)
    tables = np.full((len(lens), maxb + 1), -1, np.int64)
    used = 0
    for b, L in enumerate(lens):
        for j in range(-(-L // bs)):
            tables[b, j] = perm[used]
            used += 1
    return k, v, tables, np.array(lens), bs


def test_paged_matches_torch_sdpa_on_gathered_rows():
    rng = np.random.default_rng(11)
    k, v, tables, lens, bs = _paged_case(rng)
    B, Hq, Hkv, D = len(lens), 4, 2, 128
    qb, qt = _bf16(rng, (B, Hq, D))
    got = oracle.decode_attention_fp8kv_paged(qb, k, v, tables, lens, bs, 0.02, 0.03, 0.09)
    kd = _torch_dec(k) * float(np.float32(0.02))
    vd = _torch_dec(v) * float(np.float32(0.03))
    for b in range(B):
        if lens[b] == 0:
            assert (got[b] == 0).all()
            continue
        idx = torch.tensor([tables[b][t // bs] * bs + t % bs for t in range(lens[b])])
        kk = kd[idx].permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        vv = vd[idx].permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[b][:, None, :], kk, vv, scale=float(np.float32(0.09)))[:, 0, :].numpy()
        np.testing.assert_allclose(got[b], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_paged_in_order_blocks_equal_the_contiguous_layout():
    """Tables that list consecutive blocks for sequences starting on block
    boundaries give exactly the contiguous result over the same rows."""
    rng = np.random.default_rng(12)
    bs, lens = 8, [20, 8, 31]
    starts = [0, 24, 32, 64]   # each sequence starts on a block boundary
    k, v = _codes(rng, (64, 2, 128)), _codes(rng, (64, 2, 128))
    tables = np.array([[0, 1, 2, -1], [3, -1, -1, -1], [4, 5, 6, 7]])
    q = rng.standard_normal((3, 4, 128))
    paged = oracle.decode_attention_fp8kv_paged(q, k, v, tables, lens, bs, 0.5, 0.25)
    kc = np.concatenate([k[starts[b]:starts[b] + lens[b]] for b in range(3)])
    vc = np.concatenate([v[starts[b]:starts[b] + lens[b]] for b in range(3)])
    cont = oracle.decode_attention_fp8kv(q, kc, vc, np.cumsum([0] + lens), 0.5, 0.25)
    np.testing.assert_array_equal(paged, cont)


def test_paged_block_placement_does_not_matter():
    """Moving the physical blocks (and the tables with them) leaves every
    output unchanged; a block shared by two sequences is read by both."""
    rng = np.random.default_rng(13)
    k, v, tables, lens, bs = _paged_case(rng, lens=(40, 33, 16))
    tables[2, 0] = tables[0, 0]          # the third sequence shares the first's first block
    q = rng.standard_normal((3, 2, 128))
    a = oracle.decode_attention_fp8kv_paged(q, k, v, tables, lens, bs)
    nblk = k.shape[0] // bs
    move = rng.permutation(nblk)         # physical block i goes to slot move[i]
    k2 = np.empty_like(k); v2 = np.empty_like(v)
    for i in range(nblk):
        k2[move[i] * bs:(move[i] + 1) * bs] = k[i * bs:(i + 1) * bs]
        v2[move[i] * bs:(move[i] + 1) * bs] = v[i * bs:(i + 1) * bs]
    t2 = np.where(tables >= 0, move[np.clip(tables, 0, None)], -1)
    b = oracle.decode_attention_fp8kv_paged(q, k2, v2, t2, lens, bs)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a[2], oracle.decode_attention_fp8kv(
        q[2:3], k[tables[0, 0] * bs:tables[0, 0] * bs + 16], v[tables[0, 0] * bs:tables[0, 0] * bs + 16],
        [0, 16])[0])


def test_paged_blocks_outside_the_cache_are_absent():
    rng = np.random.default_rng(14)
    k, v, tables, lens, bs = _paged_case(rng, lens=(48,))
    q = rng.standard_normal((1, 2, 128))
    nblk = k.shape[0] // bs
    t_bad = tables.copy()
    t_bad[0, 1] = nblk + 3               # the middle block points past the cache
    got = oracle.decode_attention_fp8kv_paged(q, k, v, t_bad, lens, bs)
    keep = [tables[0, 0], tables[0, 2]]  # the other two blocks, in order
    kc = np.concatenate([k[i * bs:(i + 1) * bs] for i in keep])
    vc = np.concatenate([v[i * bs:(i + 1) * bs] for i in keep])
    np.testing.assert_array_equal(got, oracle.decode_attention_fp8kv(q, kc, vc, [0, 32]))
