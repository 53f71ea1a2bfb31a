"""Pins of the oracle's merged-layer functions ("[Kernel] Support Fp8
Checkpoints (Dynamic + Static)": merged QKV / gate_up layers whose shards
carry their own weight scales; the review comment on the same page: rescale
every shard to the shared scale max(s_i) by the ratio s_i / max(s_i)).

Each pin is independent of the oracle's code: closed forms (the identity at
ratio 1, the exponent step at ratio 1/2), brute force over all 256 e4m3 codes
with numpy's binary32 arithmetic and torch's float8 cast as the encoder, and
the rounding-error bound and monotonicity the rescaled codes must satisfy.
"""
import numpy as np
import pytest
import torch

import oracle

FP8_CODES = np.arange(256, dtype=np.uint8)
NAN_CODES = {0x7F, 0xFF}
INT8_CODES = np.arange(-127, 128, dtype=np.int8).view(np.uint8)


def _torch_dec(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn).float().numpy()


def _torch_enc(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_expand_shard_scales_layout():
    s = np.array([0.5, 3.0, 0.125, 7.0], np.float32)
    rows = [3, 0, 2, 1]
    e = oracle.expand_shard_scales(s, rows)
    assert e.size == 6
    assert e.tolist() == [0.5, 0.5, 0.5, 0.125, 0.125, 7.0]  # an empty shard adds no row
    assert oracle.expand_shard_scales([2.5], [5]).tolist() == [2.5] * 5
    with pytest.raises(ValueError):
        oracle.expand_shard_scales([1.0, 2.0], [1])
    with pytest.raises(ValueError):
        oracle.expand_shard_scales([1.0], [-1])


def _requant_table(qtype, codes, shard_scale, smax):
    """Requantise one row of codes as shard 0 of a two-shard weight whose
    other shard holds the maximum scale."""
    w = np.stack([codes, codes]).astype(np.uint8)
    out, shared = oracle.requant_shared_scale(w, qtype, [1, 1], [shard_scale, smax])
    assert shared == np.float32(max(shard_scale, smax))
    return out[0], out[1]


def test_requant_identity_at_the_shared_scale():
    """The shard that holds the maximum scale (ratio exactly 1) keeps its codes."""
    for qtype, codes in (("fp8", FP8_CODES), ("int8", INT8_CODES)):
        r0, r1 = _requant_table(qtype, codes, 0.75, 3.0)
        keep = [c for c in codes if not (qtype == "fp8" and c in NAN_CODES)]
        idx = [int(np.where(codes == c)[0][0]) for c in keep]
        assert np.array_equal(r1[idx], codes[idx])
    # the NaN codes stay NaN (0x7F)
    _, r1 = _requant_table("fp8", FP8_CODES, 0.75, 3.0)
    assert r1[0x7F] == 0x7F and r1[0xFF] == 0x7F


def test_requant_half_ratio_closed_form():
    """Ratio 1/2: an e4m3 normal with biased exponent >= 2 keeps its
    mantissa and loses one exponent step (code - 8, sign kept); int8 codes
    halve with ties to even."""
    r0, _ = _requant_table("fp8", FP8_CODES, 1.0, 2.0)
    for c in range(256):
        e = (c >> 3) & 15
        if c in NAN_CODES or e < 2:
            continue
        assert r0[c] == c - 8, hex(c)
    r0, _ = _requant_table("int8", INT8_CODES, 1.0, 2.0)
    ints = INT8_CODES.view(np.int8).astype(np.float64)
    assert np.array_equal(r0.view(np.int8), np.round(ints / 2).astype(np.int8))  # numpy rounds half to even


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_requant_brute_force_all_codes(seed):
    """Every code against numpy binary32 steps and torch's e4m3 cast."""
    rng = np.random.default_rng(seed)
    smax = np.float32(rng.uniform(1e-3, 1e-1))
    for _ in range(8):
        si = np.float32(smax * rng.uniform(0.05, 1.0))
        t = np.float32(si) / np.float32(smax)  # binary32 IEEE division
        keep = np.array([c for c in FP8_CODES if c not in NAN_CODES], np.uint8)
        v = _torch_dec(keep).astype(np.float32) * np.float32(t)  # binary32 product
        want = _torch_enc(v)
        r0, _ = _requant_table("fp8", FP8_CODES, si, smax)
        assert np.array_equal(r0[keep], want)
        ints = INT8_CODES.view(np.int8).astype(np.float32)
        vi = ints * np.float32(t)
        want_i = np.clip(np.round(vi), -127, 127).astype(np.int8)
        r0, _ = _requant_table("int8", INT8_CODES, si, smax)
        assert np.array_equal(r0.view(np.int8), want_i)


def test_requant_error_bound_and_order():
    """dec(q') * s stays within half a code spacing of dec(q) * s_i (e4m3:
    2^-4 relative in the normal range, 2^-10 * s absolute below it); the
    order of the codes and their signs are kept."""
    rng = np.random.default_rng(7)
    keep = np.array([c for c in FP8_CODES if c not in NAN_CODES], np.uint8)
    dec = _torch_dec(keep).astype(np.float64)
    order = np.argsort(dec, kind="stable")
    for _ in range(20):
        smax = float(rng.uniform(1e-3, 1.0))
        si = float(np.float32(smax * rng.uniform(0.01, 1.0)))
        r0, _ = _requant_table("fp8", keep, si, smax)
        shared = np.float32(smax)  # the larger of the two shard scales
        got = _torch_dec(r0).astype(np.float64) * float(shared)
        exact = dec * si
        bound = np.maximum(2.0 ** -4 * np.abs(exact), 2.0 ** -10 * float(shared)) * (1 + 2.0 ** -20)
        assert (np.abs(got - exact) <= bound).all()
        assert (np.diff(got[order]) >= 0).all()
        assert (np.sign(got) * np.sign(exact) >= 0).all()


def test_requant_rows_follow_their_shards():
    """Ragged shards, an empty one among them: each row uses its own shard's
    ratio and the shared scale is the largest one."""
    rng = np.random.default_rng(3)
    rows = [5, 0, 3, 9]
    scales = np.array([0.02, 0.5, 0.08, 0.05], np.float32)
    w = rng.integers(0, 256, size=(17, 32), dtype=np.uint8)
    w[w == 0x7F] = 0x7E
    w[w == 0xFF] = 0xFE
    out, shared = oracle.requant_shared_scale(w, "fp8", rows, scales)
    assert shared == np.float32(0.5)
    n0 = 0
    for r, s in zip(rows, scales):
        for i in range(r):
            t = np.float32(s) / np.float32(0.5)
            assert np.array_equal(out[n0 + i], _torch_enc(_torch_dec(w[n0 + i]) * np.float32(t)))
        n0 += r
    with pytest.raises(ValueError):
        oracle.requant_shared_scale(w, "fp8", [5, 3], scales[:2])  # rows must sum to N
